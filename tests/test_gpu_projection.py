"""GPU parity of the q/k/v projections with the RoPE in their epilogue, against
oracle.projection, through the C ABI.

The kernel accumulates x W^T + b in fp32 and rounds once to bf16; the oracle
sums exactly and rounds once. Bound per output: one bf16 ulp of the oracle's
value plus the fp32 summation error, at most (hidden / 32) * 2^-24 * A with
A = sum |x_k w_k| + |b| (each MFMA adds 32 exact products into the fp32
accumulator: hidden / 32 roundings of a partial sum no larger than A). The
second term matters only where large terms cancel to a tiny result. Almost
all outputs must equal the oracle exactly. The rotated outputs are checked in
two steps: bit-identical to the standalone rotation (itself bit-exact against
the oracle) applied to the unrotated output, and bit-identical to the oracle
wherever the two unrotated inputs of a pair agree with the oracle's.
"""

import numpy as np
import pytest
import torch

import attention_yarn_rope_amd as gx
import oracle
from attention_yarn_rope_amd import workloads as wl
from helpers import np64, say
from oracle import projection as pj

pytestmark = pytest.mark.gpu


def _ulp(r):
    """One bf16 ulp at |r| (8 significant bits); for r = 0 the smallest normal's."""
    a = np.maximum(np.abs(r), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _gpu(w, table=None, cu=None, max_seqlen=None, B=None):
    x = w.x.cuda()
    if cu is None:   # BSHD: B sequences of equal length (one when B is None)
        x = x.reshape(B or 1, -1, x.shape[-1])
    dev = lambda t: t.cuda() if t is not None else None
    return gx.qkv_proj_rope(x, dev(w.wq), dev(w.bq), dev(w.wk), dev(w.bk), dev(w.wv), dev(w.bv), table=table,
                            cu_seqlens=dev(cu), max_seqlen=max_seqlen)


def _ref(w, rows=None):
    """The oracle's outputs and each output's bound on the fp32 summation error."""
    x = np64(w.x) if rows is None else np64(w.x[rows])
    hidden = x.shape[1]
    out, bounds = [], []
    for wt, b in ((w.wq, w.bq), (w.wk, w.bk), (w.wv, w.bv)):
        wt = np64(wt)
        b = np64(b) if b is not None else None
        out.append(oracle.round_bf16(pj.linear(x, wt, b)).reshape(x.shape[0], -1, 64))
        a = np.abs(x) @ np.abs(wt).T + (np.abs(b)[None, :] if b is not None else 0.0)
        bounds.append(((hidden / 32) * 2.0 ** -24 * a).reshape(out[-1].shape))
    return out, bounds


def _check_unrotated(got, ref, bound, what):
    g, r = np64(got).reshape(ref.shape), ref
    err = np.abs(g - r)
    tol = _ulp(r) + bound
    ratio = float((err / tol).max())
    same = float((g == r).mean())
    say(f"  {what}: {100 * same:.3f} % equal to the oracle; worst error / bound {ratio:.3f}")
    assert ratio <= 1.0, f"{what}: error beyond one ulp plus the summation bound (ratio {ratio:.3f})"
    assert same >= 0.99, f"{what}: only {100 * same:.2f} % equal"


@pytest.mark.parametrize("T,hkv", [(300, 8), (1, 8), (256, 4), (513, 8)])
def test_projection_unrotated(T, hkv):
    w = wl.projection(T, seed=10 + T + hkv, hkv=hkv, hq=8 * hkv)
    say(f"[gpu] projection T={T} Hkv={hkv}")
    q, k, v = _gpu(w)
    refs, bounds = _ref(w)
    for g, r, bd, n in zip((q, k, v), refs, bounds, "qkv"):
        _check_unrotated(g.reshape(T, -1, 64), r, bd, f"T={T} {n}")


def test_projection_without_bias_and_other_hidden():
    w = wl.projection(200, seed=20, hidden=576)
    w.bq = w.bk = w.bv = None
    q, k, v = _gpu(w)
    refs, bounds = _ref(w)
    for g, r, bd, n in zip((q, k, v), refs, bounds, "qkv"):
        _check_unrotated(g.reshape(r.shape), r, bd, f"no bias {n}")


def _rotated_checks(w, table, cfg, positions, q, k, v, qu, ku, vu, what):
    """q, k, v: fused outputs; qu, ku, vu: the same call without a table."""
    assert torch.equal(v, vu)
    # against the oracle where the pair's unrotated inputs equal the oracle's
    rq, rk, rv = pj.qkv_projection(np64(w.x), np64(w.wq), np64(w.bq), np64(w.wk), np64(w.bk), np64(w.wv),
                                   np64(w.bv))
    tq, tk, _ = pj.qkv_projection_rope(np64(w.x), np64(w.wq), np64(w.bq), np64(w.wk), np64(w.bk), np64(w.wv),
                                       np64(w.bv), positions, cfg)
    h = cfg.rotary_dim // 2
    for g, gu, r, t, n in ((q, qu, rq, tq, "q"), (k, ku, rk, tk, "k")):
        g, gu = np64(g).reshape(t.shape), np64(gu).reshape(r.shape)
        ok = gu == r
        pair = np.concatenate([ok[..., :h] & ok[..., h:2 * h], ok[..., :h] & ok[..., h:2 * h], ok[..., 2 * h:]],
                              axis=-1)
        assert np.array_equal(g[pair], t[pair]), f"{what} {n}: rotated output differs where its inputs agree"
        say(f"  {what} {n}: {100 * pair.mean():.3f} % of elements compared bit for bit")


@pytest.mark.parametrize("rd", [64, 32])
def test_projection_rope_bshd(rd):
    B, S = 2, 300
    cfg = oracle.RopeConfig(rotary_dim=rd)
    table = gx.rope_table(S, gx.rope_config(rotary_dim=rd))
    w = wl.projection(B * S, seed=30 + rd)
    say(f"[gpu] projection + rope BSHD rd={rd}")
    q, k, v = _gpu(w, table=table, B=B)
    qu, ku, vu = _gpu(w, B=B)
    # fused == rope_qk(unfused), bit for bit
    qr, kr = gx.rope_qk(qu, ku, table)
    assert torch.equal(q, qr) and torch.equal(k, kr)
    pos = np.concatenate([np.arange(S)] * B)
    _rotated_checks(w, table, cfg, pos, q.reshape(B * S, -1, 64), k.reshape(B * S, -1, 64), v.reshape(B * S, -1, 64),
                    qu.reshape(B * S, -1, 64), ku.reshape(B * S, -1, 64), vu.reshape(B * S, -1, 64), f"bshd rd={rd}")


def test_projection_rope_thd():
    lengths = [37, 0, 300, 1, 129]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    T = int(cu[-1])
    table = gx.rope_table(300)
    w = wl.projection(T, seed=40)
    say("[gpu] projection + rope THD")
    q, k, v = _gpu(w, table=table, cu=cu, max_seqlen=300)
    qu, ku, vu = _gpu(w, cu=cu, max_seqlen=300)
    qr, kr = gx.rope_qk(qu, ku, table, cu_seqlens=cu.cuda(), max_seqlen=300)
    assert torch.equal(q, qr) and torch.equal(k, kr)
    _rotated_checks(w, table, oracle.RopeConfig(), oracle.thd_positions(cu.numpy(), T), q, k, v, qu, ku, vu, "thd")


def test_projection_full_size_sampled():
    """The dense prefill's tokens (B=4 S=4096, hidden 2880): sampled rows of every output
    against the oracle, and the fused output against the standalone rotation everywhere."""
    B, S = 4, 4096
    table = gx.rope_table(S)
    w = wl.projection(B * S, seed=50)
    say("[gpu] projection + rope full size")
    q, k, v = _gpu(w, table=table, B=B)
    qu, ku, vu = _gpu(w, B=B)
    qr, kr = gx.rope_qk(qu, ku, table)
    assert torch.equal(q, qr) and torch.equal(k, kr)
    rows = sorted(set([0, 1, 255, 256, 4095, 4096, 8191, 16383] +
                      torch.randperm(B * S, generator=torch.Generator().manual_seed(51))[:56].tolist()))
    refs, bounds = _ref(w, rows)
    flat = lambda t: t.reshape(B * S, -1, 64)[rows]
    for g, r, bd, n in zip((flat(qu), flat(ku), flat(vu)), refs, bounds, "qkv"):
        _check_unrotated(g, r, bd, f"full size {n}")
