"""GPU parity of the window-run prefill path (BSHD, window a multiple of 32, at most 128).

Such layers run as runs of consecutive 32-query blocks per (sequence, KV head),
each key rotated once as it enters the run's LDS ring. The cases cover: a
single position; runs of two blocks and of four (a sequence of 8192 positions
over 8 KV heads); both work-group placements (the KV heads of a run on one
XCD when the run count allows it, and the plain one otherwise); ragged tails;
KV head counts 1, 2, 4 and 8; windows 32, 64, 96 and 128; the natural-log LSE
output; equality with the pre-rotated path; and packed THD sequences (runs from
the device-built run list, lengths from 0 to 4100), also equal bit for bit to
each sequence run alone as BSHD. The bar is the elementwise
tolerance in helpers.py against the fp64 oracle on every output.
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
    return gx.rope_table(8192)


# (B, S, Hkv, window): work groups = B * ceil(ceil(S / 32) / run_len) * Hkv with
# run_len = max(2, ceil(blocks / 512)); the XCD placement needs a multiple of 8 * Hkv
CASES = [
    (1, 1, 1, 128),      # one position, one run of one block
    (2, 97, 2, 32),      # 4 blocks a sequence, 2 runs: 8 work groups, plain placement
    (1, 700, 8, 128),    # 22 blocks, 11 runs of 2: 88 work groups, plain placement
    (3, 513, 1, 64),     # ragged tail of one position
    (1, 2048, 2, 96),    # 64 blocks, 32 runs: 64 work groups, XCD placement
    (1, 8192, 8, 128),   # 256 blocks, runs of 4: 512 work groups, XCD placement
]


@pytest.mark.parametrize("B,S,hkv,window", CASES)
def test_window_runs_against_oracle(table, B, S, hkv, window):
    inp = wl.prefill_bshd(B, S, seed=800 + S + window, hq=8 * hkv, hkv=hkv)
    say(f"[gpu] window runs B={B} S={S} Hkv={hkv} W={window}")
    out = gx.attn_prefill(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), window=window, table=table)
    ref = oracle.prefill_bshd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.sinks), TAU, window, CFG)
    assert_close(out, ref, f"B={B} S={S} Hkv={hkv} W={window}")


def test_window_runs_lse(table):
    """The LSE of the window-run path (natural log per row and head) against the oracle's."""
    B, S, window = 2, 300, 128
    inp = wl.prefill_bshd(B, S, seed=871)
    q, k, v, s = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.sinks))
    say("[gpu] window runs lse")
    o, lse = gx.attn_prefill_lse(q, k, v, s, window=window, table=table)
    dout = np.zeros((B, S, 64, 64))
    ref = oracle.prefill_bshd_backward(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.sinks), TAU, window, dout, CFG)
    assert_close(o, ref["o"], "window runs o (lse call)")
    # the row sum is formed from bf16-rounded probabilities: lse within 2^-8 (+ fp32 log)
    err = np.abs(np64(lse) - ref["lse"].reshape(B * S, 64))
    say(f"  lse max_abs={float(err.max()):.3e}")
    assert float(err.max()) <= 2.0 ** -8 + 1e-4


@pytest.mark.parametrize("window", [32, 128])
def test_window_runs_prerotated_identical(table, window):
    """Keys rotated as they enter the ring and q rotated in the kernel give the same bits as
    gptoss_rope_qk followed by the pre-rotated call."""
    inp = wl.prefill_bshd(2, 450, seed=880 + window)
    q, k, v, s = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.sinks))
    say(f"[gpu] window runs fused == pre-rotated W={window}")
    a = gx.attn_prefill(q, k, v, s, window=window, table=table)
    qr, kr = gx.rope_qk(q, k, table)
    b = gx.attn_prefill(qr, kr, v, s, window=window, table=None)
    assert torch.equal(a, b)


THD_LENGTHS = [0, 1, 31, 32, 33, 700, 1000, 129, 4100, 0, 64]


@pytest.mark.parametrize("window", [32, 128])
def test_window_runs_thd_against_oracle(table, window):
    """Packed sequences (lengths 0, 1, 31, 32, 33, 64, 129, 700, 1000, 4100): runs from the
    device-built run list, positions restarting per sequence, against the oracle."""
    inp = wl.prefill_thd(0, 0, 0, seed=890 + window, lengths=THD_LENGTHS)
    q, k, v, s, cu = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), inp.cu_seqlens.cuda()
    say(f"[gpu] window runs THD W={window}")
    o = gx.attn_prefill(q, k, v, s, window=window, table=table, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    ref = oracle.prefill_thd(np64(inp.q), np64(inp.k), np64(inp.v), inp.cu_seqlens.numpy(), np64(inp.sinks), TAU,
                             window, CFG)
    assert_close(o, ref, f"THD W={window}")


def test_window_runs_thd_lse(table):
    """The LSE of packed sequences on the window-run path against the oracle's."""
    inp = wl.prefill_thd(0, 0, 0, seed=893, lengths=[0, 1, 33, 300, 129])
    q, k, v, s, cu = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), inp.cu_seqlens.cuda()
    say("[gpu] window runs THD lse")
    o, lse = gx.attn_prefill_lse(q, k, v, s, window=128, table=table, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    ref = oracle.prefill_thd_backward(np64(inp.q), np64(inp.k), np64(inp.v), inp.cu_seqlens.numpy(),
                                      np64(inp.sinks), TAU, 128, np.zeros(tuple(inp.q.shape)), CFG)
    assert_close(o, ref["o"], "THD o (lse call)")
    err = np.abs(np64(lse) - ref["lse"])
    say(f"  lse max_abs={float(err.max()):.3e}")
    assert float(err.max()) <= 2.0 ** -8 + 1e-4


def test_window_runs_thd_equals_per_sequence_bshd(table):
    """A packed sequence's rows equal the same sequence run alone as BSHD, bit for bit (each
    block's result does not depend on how the blocks are grouped into runs)."""
    inp = wl.prefill_thd(0, 0, 0, seed=895, lengths=[700, 33, 1000, 0, 129])
    q, k, v, s, cu = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), inp.cu_seqlens.cuda()
    say("[gpu] window runs THD == per-sequence BSHD")
    out = gx.attn_prefill(q, k, v, s, window=128, table=table, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    c = inp.cu_seqlens.tolist()
    for n in range(len(c) - 1):
        a, b = c[n], c[n + 1]
        if b == a:
            continue
        o = gx.attn_prefill(q[None, a:b], k[None, a:b], v[None, a:b], s, window=128, table=table)
        assert torch.equal(out[a:b], o[0]), f"sequence {n}"


def test_window_runs_strided_inputs_and_output(table):
    """q/k/v as views of one fused qkv buffer (token stride 80 heads) and the output written into
    a strided view: the ring loads and the clipped stores use the given strides."""
    g = torch.Generator().manual_seed(897)
    B, S = 2, 333
    qkv = torch.randn((B, S, 80, 64), generator=g).to(torch.bfloat16)
    sinks = torch.randn(64, generator=g)
    d = qkv.cuda()
    big = torch.zeros((B, S, 96, 64), dtype=torch.bfloat16, device="cuda")
    out = big[:, :, 16:80]
    say("[gpu] window runs strided")
    gx.attn_prefill(d[:, :, :64], d[:, :, 64:72], d[:, :, 72:80], sinks.cuda(), window=128, table=table, out=out)
    ref = oracle.prefill_bshd(np64(qkv[:, :, :64]), np64(qkv[:, :, 64:72]), np64(qkv[:, :, 72:80]),
                              np64(sinks), TAU, 128, CFG)
    assert_close(out, ref, "strided W=128")
    assert torch.count_nonzero(big[:, :, :16]) == 0 and torch.count_nonzero(big[:, :, 80:]) == 0
