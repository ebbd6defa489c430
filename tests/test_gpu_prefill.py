"""GPU parity of the prefill kernel against the fp64 oracle (through the C ABI).

Sizes span several 64-key tiles and 32-query blocks with ragged tails; the
bar is the elementwise tolerance in helpers.py. Cross-kernel identities are
checked bit-for-bit: k rotated in the tile loads == k rotated by a separate
pass == rope_qk followed by the pre-rotated kernel; a window at least the
sequence length == full causal; repeated runs are identical.
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
    return gx.rope_table(16384)


def _run_bshd(inp, window, table, k_rotation="auto"):
    return gx.attn_prefill(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), window=window,
                           table=table, k_rotation=k_rotation)


def _ref_bshd(inp, window):
    return oracle.prefill_bshd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.sinks), TAU, window, CFG)


@pytest.mark.parametrize("window", [0, 128])
@pytest.mark.parametrize("k_rotation", ["fused", "separate"])
def test_tiny_config(table, window, k_rotation):
    inp = wl.tiny()
    say(f"[gpu] prefill tiny B1 S256 window={window} k_rotation={k_rotation}")
    out = _run_bshd(inp, window, table, k_rotation)
    assert_close(out, _ref_bshd(inp, window), f"tiny W={window} {k_rotation}")


@pytest.mark.parametrize("B,S", [(2, 700), (1, 33), (1, 1), (3, 129)])
@pytest.mark.parametrize("window", [0, 1, 128, 300])
def test_bshd_ragged(table, B, S, window):
    inp = wl.prefill_bshd(B, S, seed=200 + S + window)
    say(f"[gpu] prefill bshd B={B} S={S} window={window}")
    out = _run_bshd(inp, window, table)
    assert_close(out, _ref_bshd(inp, window), f"bshd B={B} S={S} W={window}")


@pytest.mark.parametrize("window", [161, 162])
def test_window_staging_boundary(table, window):
    """W = 161 is the widest window whose 32-query items span at most 3 key
    tiles (all staged at once); W = 162 needs 4 tiles and streams them."""
    inp = wl.prefill_bshd(2, 700, seed=400 + window)
    say(f"[gpu] prefill window staging boundary W={window}")
    out = _run_bshd(inp, window, table)
    assert_close(out, _ref_bshd(inp, window), f"bshd B=2 S=700 W={window}")


@pytest.mark.parametrize("window", [32, 64, 96, 160])
def test_window_fixed_step_masks(table, window):
    """Windows that are multiples of 32 use fixed masks for the first and last key step of
    every 32-query item whose keys start W - 1 before it (not the first items of a sequence):
    BSHD with a ragged tail, and THD sequences that start at and after such offsets."""
    inp = wl.prefill_bshd(2, 517, seed=500 + window)
    say(f"[gpu] prefill fixed window masks W={window}")
    out = _run_bshd(inp, window, table)
    assert_close(out, _ref_bshd(inp, window), f"bshd B=2 S=517 W={window}")
    t = wl.prefill_thd(0, 0, 0, seed=510 + window, lengths=[window + 1, 300, 0, 31, 400])
    cu = t.cu_seqlens.cuda()
    out = gx.attn_prefill(t.q.cuda(), t.k.cuda(), t.v.cuda(), t.sinks.cuda(), window=window, table=table,
                          cu_seqlens=cu, max_seqlen=t.max_seqlen)
    ref = oracle.prefill_thd(np64(t.q), np64(t.k), np64(t.v), t.cu_seqlens.numpy(), np64(t.sinks), TAU, window,
                             CFG)
    assert_close(out, ref, f"thd W={window}")


@pytest.mark.parametrize("hkv", [1, 2])
def test_other_group_counts(table, hkv):
    inp = wl.prefill_bshd(1, 300, seed=300 + hkv, hq=8 * hkv, hkv=hkv)
    say(f"[gpu] prefill Hkv={hkv}")
    for w in (0, 64):
        out = _run_bshd(inp, w, table)
        assert_close(out, _ref_bshd(inp, w), f"Hkv={hkv} W={w}")


@pytest.mark.parametrize("window", [0, 128])
def test_thd_ragged(table, window):
    inp = wl.prefill_thd(0, 0, 0, seed=11, lengths=[37, 1, 0, 300, 128, 65, 512])
    say(f"[gpu] prefill thd window={window}")
    out = gx.attn_prefill(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), window=window, table=table,
                          cu_seqlens=inp.cu_seqlens.cuda(), max_seqlen=inp.max_seqlen)
    ref = oracle.prefill_thd(np64(inp.q), np64(inp.k), np64(inp.v), inp.cu_seqlens.numpy(), np64(inp.sinks),
                             TAU, window, CFG)
    assert_close(out, ref, f"thd W={window}")


@pytest.mark.parametrize("window", [0, 128])
def test_thd_many_short_sequences(table, window):
    """1500 packed sequences of 0 .. 40 tokens (more sequences than the device scheduler's 1024
    threads, so each thread walks several; window layers cut them into many short runs), one KV
    head: every row against the oracle."""
    g = torch.Generator().manual_seed(520 + window)
    lengths = torch.randint(0, 41, (1500,), generator=g).tolist()
    inp = wl.prefill_thd(0, 0, 0, seed=521 + window, lengths=lengths, hq=8, hkv=1)
    say(f"[gpu] thd 1500 short sequences window={window} (T={sum(lengths)})")
    out = gx.attn_prefill(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), window=window, table=table,
                          cu_seqlens=inp.cu_seqlens.cuda(), max_seqlen=inp.max_seqlen)
    ref = oracle.prefill_thd(np64(inp.q), np64(inp.k), np64(inp.v), inp.cu_seqlens.numpy(), np64(inp.sinks),
                             TAU, window, CFG)
    assert_close(out, ref, f"thd N=1500 W={window}")


def test_thd_equals_per_sequence_bshd(table):
    lengths = [100, 33, 250]
    inp = wl.prefill_thd(0, 0, 0, seed=12, lengths=lengths)
    say("[gpu] thd == per-sequence bshd")
    out = gx.attn_prefill(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), window=0, table=table,
                          cu_seqlens=inp.cu_seqlens.cuda(), max_seqlen=inp.max_seqlen)
    cu = inp.cu_seqlens.tolist()
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        o = gx.attn_prefill(inp.q[None, a:b].cuda(), inp.k[None, a:b].cuda(), inp.v[None, a:b].cuda(),
                            inp.sinks.cuda(), window=0, table=table)
        assert torch.equal(out[a:b], o[0])


@pytest.mark.parametrize("window", [0, 128])
def test_fused_separate_prerotated_identical(table, window):
    inp = wl.prefill_bshd(2, 333, seed=13)
    say(f"[gpu] k rotation paths identical window={window}")
    q, k, v, s = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda()
    a = gx.attn_prefill(q, k, v, s, window=window, table=table, k_rotation="fused")
    b = gx.attn_prefill(q, k, v, s, window=window, table=table, k_rotation="separate")
    qr, kr = gx.rope_qk(q, k, table)
    c = gx.attn_prefill(qr, kr, v, s, window=window, table=None)
    assert torch.equal(a, b) and torch.equal(a, c)


def test_window_at_least_length_equals_full(table):
    inp = wl.prefill_bshd(1, 200, seed=14)
    full = _run_bshd(inp, 0, table)
    for w in (200, 257, 100000):
        assert torch.equal(_run_bshd(inp, w, table), full)


def test_sink_minus_inf_and_large(table):
    inp = wl.prefill_bshd(1, 160, seed=15)
    for sinks in (torch.full((64,), -float("inf")), torch.linspace(-30.0, 30.0, 64)):
        inp.sinks = sinks
        say(f"[gpu] sinks {sinks[0].item()}..{sinks[-1].item()}")
        for w in (0, 128):
            assert_close(_run_bshd(inp, w, table), _ref_bshd(inp, w), f"special sinks W={w}")


def test_explicit_and_default_scale(table):
    """softmax_scale = 0 (the binding's default) is head_dim ** -0.5 inside the library; an
    explicit scale is used as given."""
    inp = wl.prefill_bshd(1, 150, seed=18)
    q, k, v, s = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda()
    say("[gpu] prefill softmax_scale default and 0.2")
    assert torch.equal(gx.attn_prefill(q, k, v, s, table=table), gx.attn_prefill(q, k, v, s, table=table,
                                                                               softmax_scale=0.125))
    for w in (0, 128):
        out = gx.attn_prefill(q, k, v, s, window=w, table=table, softmax_scale=0.2)
        ref = oracle.prefill_bshd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.sinks), 0.2, w, CFG)
        assert_close(out, ref, f"scale 0.2 W={w}")


def test_strided_inputs_and_output(table):
    """q/k/v as views of one fused qkv buffer; output written into a strided view."""
    g = torch.Generator().manual_seed(16)
    B, S = 2, 190
    qkv = torch.randn((B, S, 80, 64), generator=g).to(torch.bfloat16)
    sinks = torch.randn(64, generator=g)
    d = qkv.cuda()
    big = torch.zeros((B, S, 96, 64), dtype=torch.bfloat16, device="cuda")
    out = big[:, :, 16:80]
    gx.attn_prefill(d[:, :, :64], d[:, :, 64:72], d[:, :, 72:80], sinks.cuda(), window=0, table=table, out=out)
    ref = oracle.prefill_bshd(np64(qkv[:, :, :64]), np64(qkv[:, :, 64:72]), np64(qkv[:, :, 72:80]),
                              np64(sinks), TAU, 0, CFG)
    assert_close(out, ref, "strided")
    assert torch.count_nonzero(big[:, :, :16]) == 0 and torch.count_nonzero(big[:, :, 80:]) == 0


def test_deterministic(table):
    inp = wl.prefill_bshd(2, 500, seed=17)
    a = _run_bshd(inp, 0, table)
    b = _run_bshd(inp, 0, table)
    assert torch.equal(a, b)


def test_empty_inputs(table):
    q = torch.zeros((0, 64, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((0, 8, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = gx.attn_prefill(q, kv, kv, torch.zeros(64, device="cuda"), table=table, cu_seqlens=cu, max_seqlen=0)
    assert out.shape == q.shape
    cu = torch.tensor([0, 0, 0], dtype=torch.int32, device="cuda")
    out = gx.attn_prefill(q, kv, kv, torch.zeros(64, device="cuda"), table=table, cu_seqlens=cu, max_seqlen=0)
    assert out.numel() == 0
