"""GPU parity of the context-parallel prefill pieces (a query shard against a key
shard, and the merge that adds the sink once), against oracle.context_parallel,
through the C ABI.

A shard's output uses the elementwise tolerance of helpers.py; its lse the
bound of the forward's log-sum-exp (the row sum adds bf16-rounded p: at most
U = 2^-8 relative in the sum). A simulated ring -- every query shard against
every key shard on this one GPU, then the merge -- must reproduce the
prefill definition for contiguous and zig-zag shardings, full and window.
"""

import numpy as np
import pytest
import torch

import attention_yarn_rope_amd as gx
import oracle
from attention_yarn_rope_amd import workloads as wl
from helpers import assert_close, np64, say
from oracle import context_parallel as cp

pytestmark = pytest.mark.gpu
CFG = oracle.RopeConfig()
TAU = 0.125
U = 2.0 ** -8


@pytest.fixture(scope="module")
def table():
    return gx.rope_table(140000)


def _check_lse(got, ref, what):
    g = np64(got).reshape(ref.shape)
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(g), inf) and np.all(g[inf] == ref[inf]), f"{what}: -inf rows differ"
    err = float(np.abs(g[~inf] - ref[~inf]).max()) if (~inf).any() else 0.0
    say(f"  {what} lse: max_abs={err:.3e}")
    assert err <= U + 1e-4, f"{what}: lse error {err}"


@pytest.mark.parametrize("Sq,Sk,qo,ko,window", [
    (128, 128, 256, 256, 0),      # the diagonal block of a ring
    (100, 77, 500, 100, 0),       # every key visible, ragged sizes
    (96, 160, 300, 200, 128),     # window: a band of the keys
    (64, 64, 0, 512, 0),          # keys after every query: nothing visible
    (200, 300, 250, 0, 64),       # window starting inside the shard
])
def test_shard_against_oracle(table, Sq, Sk, qo, ko, window):
    g = torch.Generator().manual_seed(Sq + Sk + qo)
    q = torch.randn((2, Sq, 64, 64), generator=g).to(torch.bfloat16)
    k = torch.randn((2, Sk, 8, 64), generator=g).to(torch.bfloat16)
    v = torch.randn((2, Sk, 8, 64), generator=g).to(torch.bfloat16)
    say(f"[gpu] shard Sq={Sq} Sk={Sk} q_offset={qo} kv_offset={ko} W={window}")
    out, lse = gx.attn_prefill_shard(q.cuda(), k.cuda(), v.cuda(), qo, ko, window=window, table=table)
    ro, rl = cp.shard_attention(np64(q), np64(k), np64(v), TAU, window, qo, ko, CFG)
    assert_close(out, ro, f"shard o")
    _check_lse(lse, rl, "shard")


def _ring(q, k, v, sinks, window, table, q_chunks, kv_chunks):
    """Every query chunk against every key chunk on this GPU, then the merge; returns rows in q order."""
    outs = []
    for lo, hi in q_chunks:
        parts_o, parts_l = [], []
        for a, b in kv_chunks:
            o, l = gx.attn_prefill_shard(q[:, lo:hi].contiguous(), k[:, a:b].contiguous(), v[:, a:b].contiguous(),
                                         lo, a, window=window, table=table)
            parts_o.append(o.reshape(-1, q.shape[2], 64))
            parts_l.append(l.reshape(-1))
        outs.append(gx.attn_merge(torch.stack(parts_o), torch.stack(parts_l), sinks).reshape(q.shape[0], hi - lo,
                                                                                             q.shape[2], 64))
    return outs


@pytest.mark.parametrize("window", [0, 128])
def test_ring_contiguous_shards(table, window):
    inp = wl.prefill_bshd(1, 2048, seed=71)
    q, k, v, s = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda()
    chunks = [(512 * r, 512 * r + 512) for r in range(4)]
    say(f"[gpu] ring of 4 contiguous shards W={window}")
    outs = _ring(q, k, v, s, window, table, chunks, chunks)
    ref = oracle.prefill_bshd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.sinks), TAU, window, CFG)
    for (lo, hi), o in zip(chunks, outs):
        assert_close(o, ref[:, lo:hi], f"ring rows {lo}..{hi - 1}")
    full = gx.attn_prefill(q, k, v, s, window=window, table=table)
    assert_close(torch.cat(outs, dim=1), np64(full), "ring vs the one-call prefill")


def test_ring_zigzag_shards(table):
    inp = wl.prefill_bshd(2, 1200, seed=72)
    q, k, v, s = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda()
    chunks = [(150 * i, 150 * i + 150) for i in range(8)]
    say("[gpu] ring of 4 ranks, zig-zag chunks")
    ref = oracle.prefill_bshd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.sinks), TAU, 0, CFG)
    for r in range(4):
        mine = [chunks[r], chunks[7 - r]]
        outs = _ring(q, k, v, s, 0, table, mine, chunks)
        for (lo, hi), o in zip(mine, outs):
            assert_close(o, ref[:, lo:hi], f"rank {r} rows {lo}..{hi - 1}")


def test_merge_against_oracle():
    g = torch.Generator().manual_seed(73)
    P, T, H = 5, 300, 64
    o = torch.randn((P, T, H, 64), generator=g).to(torch.bfloat16)
    lse = torch.randn((P, T * H), generator=g) * 3
    lse[1, ::7] = -float("inf")                      # parts without keys for some rows
    lse[:, 5] = -float("inf")                        # a row with no keys in any part
    sinks = torch.randn(H, generator=g)
    lo = torch.empty(T * H, dtype=torch.float32, device="cuda")
    out = gx.attn_merge(o.cuda(), lse.cuda(), sinks.cuda(), lse_out=lo)
    parts = [(np64(o[p]), np64(lse[p]).reshape(T, H)) for p in range(P)]
    ro, rl = cp.merge(parts, np64(sinks))
    assert_close(out, ro, "merge")
    np.testing.assert_allclose(np64(lo).reshape(T, H), rl, rtol=1e-5, atol=1e-5)
    none = gx.attn_merge(o[:0].cuda(), lse[:0].cuda(), sinks.cuda())
    assert not none.any()


@pytest.mark.parametrize("P", [1, 8, 9, 17])
def test_merge_part_batches_and_strides(P):
    """Part counts around the kernel's batch of 8 loads (one part, one full batch, a batch and
    one more, three batches), with the parts a view into a larger buffer and a strided output."""
    g = torch.Generator().manual_seed(80 + P)
    T, H = 77, 16
    buf = torch.randn((P, T + 3, H, 64), generator=g).to(torch.bfloat16)
    lse = torch.randn((P, T * H), generator=g) * 4
    lse[P // 2, ::5] = -float("inf")
    sinks = torch.randn(H, generator=g)
    sinks[3] = -float("inf")
    o = buf.cuda()[:, :T]                               # part stride (T + 3) * H * 64
    big = torch.zeros((T, H, 72), dtype=torch.bfloat16, device="cuda")
    out = big[..., :64]                                 # token stride H * 72, head stride 72
    lo = torch.empty(T * H, dtype=torch.float32, device="cuda")
    say(f"[gpu] merge P={P} strided parts and output")
    gx.attn_merge(o, lse.cuda(), sinks.cuda(), out=out, lse_out=lo)
    parts = [(np64(buf[p, :T]), np64(lse[p]).reshape(T, H)) for p in range(P)]
    ro, rl = cp.merge(parts, np64(sinks))
    assert_close(out, ro, f"merge P={P}")
    assert not big[..., 64:].any(), "the merge wrote past the rows' 64 dims"
    np.testing.assert_allclose(np64(lo).reshape(T, H), rl, rtol=1e-5, atol=1e-5)


def test_ring_step_at_128k(table):
    """One ring step of the 128K-token prefill split over 8 ranks (16384 tokens each): the last
    rank's queries against the first rank's keys (all visible) and against its own keys (the
    diagonal), on sampled rows against the oracle."""
    S, R = 131072, 8
    n = S // R
    g = torch.Generator().manual_seed(74)
    q = torch.randn((1, n, 64, 64), generator=g).to(torch.bfloat16)
    k = torch.randn((1, n, 8, 64), generator=g).to(torch.bfloat16)
    v = torch.randn((1, n, 8, 64), generator=g).to(torch.bfloat16)
    rows = sorted(set([0, 1, 31, 32, 8191, n - 1] + torch.randperm(n, generator=g)[:10].tolist()))
    qo = (R - 1) * n
    for ko in (0, qo):
        say(f"[gpu] 128K ring step: q_offset={qo} kv_offset={ko}")
        out, lse = gx.attn_prefill_shard(q.cuda(), k.cuda(), v.cuda(), qo, ko, table=table)
        ro = np.stack([cp.shard_attention(np64(q[:, r:r + 1]), np64(k), np64(v), TAU, 0, qo + r, ko, CFG)[0][:, 0]
                       for r in rows], axis=1)
        assert_close(out[:, rows], ro, f"ring step kv_offset={ko}")
