"""GPU parity of the prefill backward (dq, dk, dv, dsinks) and the forward's
log-sum-exp against the fp64 oracle (oracle.backward), through the C ABI.

Sizes span several 128-key work items and 32-query blocks with ragged tails, full
causal and window layers, BSHD and packed THD, one and two KV heads. The
gradients are held to the error bound of tests/backward_tolerance.py (derived
there from the bf16 roundings a correct kernel makes, and shown on the CPU to
reject plausible kernel mistakes); the forward's LSE to U + 1e-4.
"""

import numpy as np
import pytest
import torch

import attention_yarn_rope_amd as gx
import oracle
from attention_yarn_rope_amd import workloads as wl
import backward_tolerance as bt
from backward_tolerance import grad_close
from helpers import np64, say

pytestmark = pytest.mark.gpu
CFG = oracle.RopeConfig()
TAU = 0.125


@pytest.fixture(scope="module")
def table():
    return gx.rope_table(16384)


U = bt.U


def _assert_all(ratios, what):
    assert max(ratios) <= 1.0, f"{what}: tolerance exceeded (worst ratios {[round(x, 3) for x in ratios]})"


def _bshd_case(B, S, window, table, seed, hq=64, hkv=8):
    inp = wl.prefill_bshd(B, S, seed=seed, hq=hq, hkv=hkv)
    dout = wl.grad_out((B, S, hq, 64), seed + 1000)
    q, k, v, s = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.sinks))
    o, lse = gx.attn_prefill_lse(q, k, v, s, window=window, table=table)
    dq, dk, dv, ds = gx.attn_prefill_backward(q, k, v, s, o, dout.cuda(), lse, window=window, table=table)
    torch.cuda.synchronize()
    args = (np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.sinks), TAU, window, np64(dout), CFG)
    ref = oracle.prefill_bshd_backward(*args)
    ref["noise"] = bt.noise_bshd(*args)
    return (o, lse, dq, dk, dv, ds), ref


def _check(got, ref, what):
    o, lse, dq, dk, dv, ds = got
    lse_ref = ref["lse"].reshape(-1, ref["lse"].shape[-1])
    # the forward sums bf16-rounded p: l is off by at most U relative, lse by U (plus fp32 log)
    err = np.abs(np64(lse) - lse_ref)
    say(f"  {what} lse: max_abs={float(err.max()):.3e}")
    assert float(err.max()) <= U + 1e-4, f"{what}: lse error {float(err.max())}"
    n = ref["noise"]
    _assert_all([grad_close(dq, ref["dq"], n["dq"], f"{what} dq"), grad_close(dk, ref["dk"], n["dk"], f"{what} dk"),
                 grad_close(dv, ref["dv"], n["dv"], f"{what} dv"),
                 grad_close(ds, ref["dsinks"], n["dsinks"], f"{what} dsinks", mag=n["m_dsinks"])], what)


def test_lse_forward_output_unchanged(table):
    inp = wl.prefill_bshd(2, 300, seed=51)
    q, k, v, s = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.sinks))
    say("[gpu] attn_prefill_lse output == attn_prefill output")
    for w in (0, 128):
        o1 = gx.attn_prefill(q, k, v, s, window=w, table=table)
        o2, _ = gx.attn_prefill_lse(q, k, v, s, window=w, table=table)
        assert torch.equal(o1, o2)


@pytest.mark.parametrize("B,S", [(1, 256), (2, 300), (1, 129)])
@pytest.mark.parametrize("window", [0, 128])
def test_backward_bshd(table, B, S, window):
    say(f"[gpu] backward bshd B={B} S={S} W={window}")
    got, ref = _bshd_case(B, S, window, table, seed=60 + S + window)
    _check(got, ref, f"B={B} S={S} W={window}")


@pytest.mark.parametrize("B,S", [(2, 512), (1, 1024)])
def test_backward_full_causal_tile_pairs(table, B, S):
    """Full-causal layers with a multiple of 4 key tiles of 128 give each dk / dv work group two
    tiles of complementary work ({i, 3T/4 - 1 - i} and {T/4 + i, T - 1 - i}); every key of every
    tile against the oracle (T = 4 and 8)."""
    say(f"[gpu] backward tile pairs B={B} S={S}")
    got, ref = _bshd_case(B, S, 0, table, seed=70 + S)
    _check(got, ref, f"tile pairs B={B} S={S}")


@pytest.mark.parametrize("window", [0, 300])
def test_backward_ragged_long(table, window):
    say(f"[gpu] backward bshd B=2 S=700 W={window}")
    got, ref = _bshd_case(2, 700, window, table, seed=90 + window)
    _check(got, ref, f"B=2 S=700 W={window}")


@pytest.mark.parametrize("hkv", [1, 2])
def test_backward_other_group_counts(table, hkv):
    say(f"[gpu] backward Hkv={hkv}")
    for w in (0, 64):
        got, ref = _bshd_case(1, 300, w, table, seed=110 + hkv + w, hq=8 * hkv, hkv=hkv)
        _check(got, ref, f"Hkv={hkv} W={w}")


@pytest.mark.parametrize("window", [0, 128])
def test_backward_thd(table, window):
    lengths = [37, 1, 0, 300, 128, 65, 200]
    inp = wl.prefill_thd(0, 0, 0, seed=120 + window, lengths=lengths)
    T = sum(lengths)
    dout = wl.grad_out((T, 64, 64), 1120 + window)
    say(f"[gpu] backward thd W={window}")
    q, k, v, s = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.sinks))
    cu = inp.cu_seqlens.cuda()
    o, lse = gx.attn_prefill_lse(q, k, v, s, window=window, table=table, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    grads = gx.attn_prefill_backward(q, k, v, s, o, dout.cuda(), lse, window=window, table=table, cu_seqlens=cu,
                                     max_seqlen=inp.max_seqlen)
    args = (np64(inp.q), np64(inp.k), np64(inp.v), inp.cu_seqlens.numpy(), np64(inp.sinks), TAU, window,
            np64(dout), CFG)
    ref = oracle.prefill_thd_backward(*args)
    ref["noise"] = bt.noise_thd(*args)
    _check((o, lse) + tuple(grads), ref, f"thd W={window}")


@pytest.mark.parametrize("window", [0, 128])
def test_backward_thd_many_short_sequences(table, window):
    """300 packed sequences of 0 .. 60 tokens, one KV head: the dq and dk / dv work lists hold
    hundreds of tiny items; every gradient against the oracle."""
    g = torch.Generator().manual_seed(130 + window)
    lengths = torch.randint(0, 61, (300,), generator=g).tolist()
    inp = wl.prefill_thd(0, 0, 0, seed=131 + window, lengths=lengths, hq=8, hkv=1)
    T = sum(lengths)
    dout = wl.grad_out((T, 8, 64), 1130 + window)
    say(f"[gpu] backward thd 300 sequences W={window} (T={T})")
    q, k, v, s = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.sinks))
    cu = inp.cu_seqlens.cuda()
    o, lse = gx.attn_prefill_lse(q, k, v, s, window=window, table=table, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    grads = gx.attn_prefill_backward(q, k, v, s, o, dout.cuda(), lse, window=window, table=table, cu_seqlens=cu,
                                     max_seqlen=inp.max_seqlen)
    args = (np64(inp.q), np64(inp.k), np64(inp.v), inp.cu_seqlens.numpy(), np64(inp.sinks), TAU, window,
            np64(dout), CFG)
    ref = oracle.prefill_thd_backward(*args)
    ref["noise"] = bt.noise_thd(*args)
    _check((o, lse) + tuple(grads), ref, f"thd N=300 W={window}")


def test_backward_prerotated_and_deterministic(table):
    """table = None takes q and k as already rotated: gradients then equal the
    rotated-space ones, i.e. R^T undone; two calls give identical bits."""
    inp = wl.prefill_bshd(1, 200, seed=130)
    dout = wl.grad_out((1, 200, 64, 64), 1130).cuda()
    q, k, v, s = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.sinks))
    qr, kr = gx.rope_qk(q, k, table)
    say("[gpu] backward pre-rotated inputs, repeatability")
    o, lse = gx.attn_prefill_lse(qr, kr, v, s, window=0)
    g1 = gx.attn_prefill_backward(qr, kr, v, s, o, dout, lse, window=0)
    g2 = gx.attn_prefill_backward(qr, kr, v, s, o, dout, lse, window=0)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    args = (np64(qr), np64(kr), np64(inp.v), np64(inp.sinks), TAU, 0, np64(dout))
    ref = oracle.prefill_bshd_backward(*args, rotate_qk=False)
    ref["noise"] = bt.noise_bshd(*args, rotate_qk=False)
    _check((o, lse) + tuple(g1), ref, "pre-rotated")


def test_backward_strided_inputs_equal_contiguous(table):
    """q, k, v as views of one fused qkv buffer (token stride 80 heads), with the table: the dq
    kernel reads and rotates q through the caller's strides and k is rotated from its own. The
    gradients equal those of the same values passed contiguous, bit for bit (layout only)."""
    g = torch.Generator().manual_seed(150)
    B, S = 2, 333
    qkv = torch.randn((B, S, 80, 64), generator=g).to(torch.bfloat16).cuda()
    sinks = torch.randn(64, generator=g).cuda()
    dout = wl.grad_out((B, S, 64, 64), 1150).cuda()
    q, k, v = qkv[:, :, :64], qkv[:, :, 64:72], qkv[:, :, 72:80]
    say("[gpu] backward strided q/k/v == contiguous")
    for window in (0, 128):
        o, lse = gx.attn_prefill_lse(q, k, v, sinks, window=window, table=table)
        strided = gx.attn_prefill_backward(q, k, v, sinks, o, dout, lse, window=window, table=table)
        contig = gx.attn_prefill_backward(q.contiguous(), k.contiguous(), v.contiguous(), sinks, o, dout, lse,
                                          window=window, table=table)
        for name, a, b in zip(("dq", "dk", "dv", "dsinks"), strided, contig):
            assert torch.equal(a, b), f"{name} window {window}"


def test_backward_special_sinks(table):
    """sigma = -inf (no sink: dsigma = 0) and a large sigma = +30 (the sink takes almost all weight)."""
    inp = wl.prefill_bshd(1, 150, seed=140)
    dout = wl.grad_out((1, 150, 64, 64), 1140)
    for val in (-np.inf, 30.0):
        sinks = torch.full((64,), float(val))
        say(f"[gpu] backward sinks={val}")
        q, k, v, s = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), sinks.cuda()
        o, lse = gx.attn_prefill_lse(q, k, v, s, window=0, table=table)
        grads = gx.attn_prefill_backward(q, k, v, s, o, dout.cuda(), lse, window=0, table=table)
        args = (np64(inp.q), np64(inp.k), np64(inp.v), sinks.double().numpy(), TAU, 0, np64(dout), CFG)
        ref = oracle.prefill_bshd_backward(*args)
        ref["noise"] = bt.noise_bshd(*args)
        _check((o, lse) + tuple(grads), ref, f"sinks={val}")
        if val == -np.inf:
            assert torch.all(grads[3] == 0)


@pytest.mark.parametrize("window", [0, 128])
def test_backward_full_size_sampled(table, window):
    """The benchmark's configuration (dense B=4 S=4096, both layers, the same inputs and
    dO as bench.py): dq on 32 sampled query rows and dk, dv on whole 128-key work items,
    of batch 3, against the oracle's exact gradients at those rows and keys."""
    inp = wl.dense()
    dout = wl.grad_out(inp.q.shape, 7)
    tab = gx.rope_table(4096)
    q, k, v, s = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.sinks))
    say(f"[gpu] backward full size B=4 S=4096 W={window}")
    o, lse = gx.attn_prefill_lse(q, k, v, s, window=window, table=tab)
    dq, dk, dv, ds = gx.attn_prefill_backward(q, k, v, s, o, dout.cuda(), lse, window=window, table=tab)
    torch.cuda.synchronize()
    b = 3
    extra = torch.randperm(4096, generator=torch.Generator().manual_seed(17))[:24].tolist()
    rows = sorted(set([0, 1, 31, 32, 63, 64, 2047, 4095] + extra))
    f64 = lambda t: t[b].double().numpy()
    tiles = [(3968, 4096)] + ([(2048, 2176), (0, 128)] if window else [])
    for lo, hi in tiles:
        args = (f64(inp.q), f64(inp.k), f64(inp.v), np64(inp.sinks), TAU, window, f64(dout), rows, lo, hi, CFG)
        ref = oracle.prefill_backward_rows(*args)
        n = bt.noise_rows(*args)
        _assert_all([grad_close(dq[b, rows], ref["dq"], n["dq"], f"W={window} dq rows"),
                     grad_close(dk[b, lo:hi], ref["dk"], n["dk"], f"W={window} dk keys {lo}..{hi - 1}"),
                     grad_close(dv[b, lo:hi], ref["dv"], n["dv"], f"W={window} dv keys {lo}..{hi - 1}")],
                    f"full size W={window}")


@pytest.mark.parametrize("window", [0, 128])
def test_backward_no_sink_far_below_zero(window):
    """sigma = -inf with every logit near -512 (already-rotated q = -8 + a, k = 8 + b): the
    forward's lse must be each row's own log-sum-exp, not -inf, for the gradients to be right."""
    q, k, v = wl.far_below((1, 300), (1, 300), 0.5, seed=850 + window)
    sinks = torch.full((64,), -float("inf"))
    dout = wl.grad_out((1, 300, 64, 64), 1850 + window)
    say(f"[gpu] backward, no sink, logits near -512, W={window}")
    qc, kc, vc, sc = q.cuda(), k.cuda(), v.cuda(), sinks.cuda()
    o, lse = gx.attn_prefill_lse(qc, kc, vc, sc, window=window)
    grads = gx.attn_prefill_backward(qc, kc, vc, sc, o, dout.cuda(), lse, window=window)
    args = (np64(q), np64(k), np64(v), np64(sinks), TAU, window, np64(dout))
    ref = oracle.prefill_bshd_backward(*args, rotate_qk=False)
    ref["noise"] = bt.noise_bshd(*args, rotate_qk=False)
    _check((o, lse) + tuple(grads), ref, f"no sink far below W={window}")
    assert torch.all(grads[3] == 0)
