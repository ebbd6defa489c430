"""GPU parity of the split-KV decode kernels against the fp64 oracle (through the C ABI).

Also: decode equals the last row of prefill on the same data (the cache holds
rope_qk's rotated k), results do not depend on the split count beyond fp32
reassociation, sequences of length 1 and sinks of -inf behave, and 600 sequences
(several per planning thread) are planned and merged correctly.
"""

import numpy as np
import pytest
import torch

import attention_yarn_rope_amd as gx
import oracle
from attention_yarn_rope_amd import workloads as wl
from helpers import assert_close, np64, say

pytestmark = pytest.mark.gpu
CFG = oracle.RopeConfig()
TAU = 0.125


@pytest.fixture(scope="module")
def table():
    return gx.rope_table(40000)


def _ref(inp, window, rows=None):
    rows = range(len(inp.lengths)) if rows is None else rows
    idx = list(rows)
    return oracle.decode(np64(inp.q[idx]), np64(inp.k_cache[idx]), np64(inp.v_cache[idx]),
                         [inp.lengths[i] for i in idx], np64(inp.sinks), TAU, window, CFG)


def _run(inp, window, table, num_splits=0):
    return gx.attn_decode(inp.q.cuda(), inp.k_cache.cuda(), inp.v_cache.cuda(), inp.cache_seqlens.cuda(),
                          inp.sinks.cuda(), window=window, table=table, num_splits=num_splits)


@pytest.mark.parametrize("window", [0, 128])
def test_decode_ragged(table, window):
    inp = wl.decode(0, 0, 0, seed=21, max_len=2100, lengths=[1, 2, 127, 128, 129, 511, 512, 513, 2000, 2100])
    say(f"[gpu] decode ragged window={window}")
    assert_close(_run(inp, window, table), _ref(inp, window), f"decode W={window}")


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_decode_split_counts(table, splits):
    inp = wl.decode(0, 0, 0, seed=22, max_len=3000, lengths=[3000, 1700, 900])
    say(f"[gpu] decode num_splits={splits}")
    out = _run(inp, 0, table, num_splits=splits)
    auto = _run(inp, 0, table)
    assert_close(out, _ref(inp, 0), f"decode splits={splits}")
    assert (np64(out) - np64(auto)).__abs__().max() <= 2 ** -6


@pytest.mark.parametrize("window", [0, 128])
def test_decode_many_sequences(table, window):
    """600 sequences (more than the planning kernel's 256 threads, so each thread plans several),
    cache lengths uniform in [1, 1500], one KV head: every row against the oracle."""
    inp = wl.decode(600, 1, 1500, seed=25, max_len=1500, hq=8, hkv=1)
    say(f"[gpu] decode 600 sequences window={window}")
    assert_close(_run(inp, window, table), _ref(inp, window), f"decode N=600 W={window}")


def test_decode_single_split_finish_equals_combine(table):
    """With one split per sequence the split kernel adds the sink and normalises its partial
    itself (no combine launch). Forcing the planned path (num_splits=2, every sequence shorter
    than one 128-key split) runs the same single partial through the combine kernel: the two
    must agree bit for bit, the direct form using the combine's operation order. Lengths 1 to
    128, sinks including -inf and a large value."""
    inp = wl.decode(0, 0, 0, seed=26, max_len=128, lengths=[1, 2, 17, 64, 100, 127, 128, 128, 5, 33])
    inp.sinks[0] = float("-inf")
    inp.sinks[9] = 30.0
    say("[gpu] decode one-split finish == combine")
    for window in (0, 128):
        direct = _run(inp, window, table)                 # eff <= 512 keys: one split, no combine
        combined = _run(inp, window, table, num_splits=2)  # 128-key splits: one each, through the combine
        assert torch.equal(direct, combined), f"window {window}"
        assert_close(direct, _ref(inp, window), f"decode one split W={window}")


def test_decode_equals_last_prefill_row(table):
    """Cache k = rope_qk(k); decode's q is the raw q of the last token."""
    B, S = 2, 777
    inp = wl.prefill_bshd(B, S, seed=23)
    q, k, v, s = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda()
    say("[gpu] decode == last prefill row")
    for window in (0, 128):
        pre = gx.attn_prefill(q, k, v, s, window=window, table=table)
        _, kr = gx.rope_qk(q, k, table)
        lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
        dec = gx.attn_decode(q[:, S - 1].contiguous(), kr, v, lens, s, window=window, table=table)
        # different blockings of the same sums: fp32 reassociation plus one bf16 rounding apart
        assert_close(dec, np64(pre[:, S - 1]), f"decode vs prefill W={window}", atol=4e-3, rtol=1e-2)


def test_decode_sink_minus_inf_and_hkv2(table):
    inp = wl.decode(0, 0, 0, seed=24, max_len=700, lengths=[700, 1, 300], hq=16, hkv=2)
    inp.sinks = torch.full((16,), -float("inf"))
    say("[gpu] decode sink -inf, Hkv=2")
    for w in (0, 128):
        assert_close(_run(inp, w, table), _ref(inp, w), f"decode -inf W={w}")


def test_decode_deterministic(table):
    inp = wl.decode(0, 0, 0, seed=25, max_len=5000, lengths=[5000, 4000])
    a, b = _run(inp, 0, table), _run(inp, 0, table)
    assert torch.equal(a, b)


@pytest.mark.parametrize("window", [0, 128])
def test_decode_128k_context(window):
    """The longest context (131072 positions): a full cache, a ragged one and a one-token one,
    from a contiguous cache and from a shuffled pool of 64-row pages holding the same rows
    (bit-identical to the contiguous decode for the full layer)."""
    lengths = [131072, 77777, 1]
    inp = wl.decode(0, 0, 0, seed=26, max_len=131072, lengths=lengths)
    table = gx.rope_table(131072)
    say(f"[gpu] decode 128K context window={window}")
    out = _run(inp, window, table)
    assert_close(out, _ref(inp, window), f"decode 128K W={window}")
    N, Lmax, ps = len(lengths), 131072, 64
    npages = N * Lmax // ps
    perm = torch.randperm(npages, generator=torch.Generator().manual_seed(27))
    kc, vc = inp.k_cache.cuda(), inp.v_cache.cuda()
    k_pool = torch.empty((npages, ps, 8, 64), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.empty_like(k_pool)
    k_pool[perm.cuda()] = kc.reshape(npages, ps, 8, 64)
    v_pool[perm.cuda()] = vc.reshape(npages, ps, 8, 64)
    del kc, vc
    bt = perm.to(torch.int32).reshape(N, Lmax // ps).contiguous().cuda()
    paged = gx.attn_decode_kv(inp.q.cuda(), k_pool, v_pool, inp.cache_seqlens.cuda(), inp.sinks.cuda(), kind="paged",
                              block_table=bt, window=window, table=table)
    if window == 0:
        assert torch.equal(paged, out), "paged decode differs from the contiguous decode of the same rows"
    else:
        assert_close(paged, _ref(inp, window), f"paged decode 128K W={window}")
