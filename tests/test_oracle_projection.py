"""Pins of oracle.projection (q/k/v projections and the RoPE applied to their output).

The projection is pinned by a pure-Python dot product on tiny inputs, by
one-hot weights that pick single input features, by zero weights (bias only)
and by the exactness of the fp64 sum on bf16 inputs; its single rounding by
comparison with round_bf16 of the exact value. The fused form is pinned to the
composition of the pinned pieces: projection, then the pinned rotation at the
BSHD / THD positions.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import projection as pj

CFG = oracle.RopeConfig()


def _bf(rng, shape, scale=1.0):
    return oracle.round_bf16(rng.standard_normal(shape) * scale)


def _weights(rng, hidden, hq=16, hkv=2):
    return (_bf(rng, (hq * 64, hidden), hidden ** -0.5), _bf(rng, hq * 64, 0.1),
            _bf(rng, (hkv * 64, hidden), hidden ** -0.5), _bf(rng, hkv * 64, 0.1),
            _bf(rng, (hkv * 64, hidden), hidden ** -0.5), _bf(rng, hkv * 64, 0.1))


def test_linear_brute_force():
    rng = np.random.default_rng(1)
    x, w, b = _bf(rng, (3, 5)), _bf(rng, (4, 5)), _bf(rng, 4)
    z = pj.linear(x, w, b)
    for t in range(3):
        for o in range(4):
            acc = math.fsum([float(x[t, i]) * float(w[o, i]) for i in range(5)] + [float(b[o])])
            assert z[t, o] == acc


def test_linear_matches_the_correctly_rounded_sum():
    """At the real hidden size (2880): products of bf16 values are exact in fp64, so the
    oracle's fp64 matrix product can differ from the correctly rounded sum (math.fsum of
    the same products) only by fp64 summation error, far below a bf16 ulp."""
    rng = np.random.default_rng(2)
    x, w = _bf(rng, (2, 2880)), _bf(rng, (3, 2880), 2880 ** -0.5)
    z = pj.linear(x, w, None)
    for t in range(2):
        for o in range(3):
            terms = (x[t] * w[o]).tolist()
            ref = math.fsum(terms)
            assert abs(z[t, o] - ref) <= 1e-13 * math.fsum(abs(a) for a in terms)


def test_one_hot_and_zero_weights():
    rng = np.random.default_rng(3)
    hidden = 192
    x = _bf(rng, (7, hidden))
    wq = np.zeros((64, hidden)); wq[np.arange(64), 3 * np.arange(64)] = 1.0     # q feature j = x[:, 3j]
    bq = _bf(rng, 64)
    z = np.zeros((64, hidden))
    bk = _bf(rng, 64)
    q, k, v = pj.qkv_projection(x, wq, bq, z, bk, z, None)
    assert np.array_equal(q[:, 0, :], oracle.round_bf16(x[:, ::3] + bq))
    assert np.array_equal(k[:, 0, :], np.broadcast_to(bk, (7, 64)))
    assert np.array_equal(v, np.zeros((7, 1, 64)))


def test_rounded_once():
    rng = np.random.default_rng(4)
    x = _bf(rng, (5, 128))
    w = _weights(rng, 128, hq=8, hkv=1)
    q, k, v = pj.qkv_projection(x, *w)
    exact = pj.linear(x, w[0], w[1])
    assert np.array_equal(q.reshape(5, -1), oracle.round_bf16(exact))
    assert np.array_equal(oracle.round_bf16(q), q)


@pytest.mark.parametrize("rd", [64, 32])
def test_rope_form_is_projection_then_rotation(rd):
    cfg = oracle.RopeConfig(rotary_dim=rd)
    rng = np.random.default_rng(5)
    S, hidden = 23, 128
    x = _bf(rng, (2 * S, hidden))
    w = _weights(rng, hidden)
    q, k, v = pj.qkv_projection(x, *w)
    # BSHD: two sequences of S tokens, positions 0..S-1 each
    pos = np.concatenate([np.arange(S), np.arange(S)])
    qr, kr, vr = pj.qkv_projection_rope(x, *w, pos, cfg)
    rq, rk = oracle.rope_qk_bshd(q.reshape(2, S, 16, 64), k.reshape(2, S, 2, 64), cfg)
    assert np.array_equal(qr, rq.reshape(2 * S, 16, 64)) and np.array_equal(kr, rk.reshape(2 * S, 2, 64))
    assert np.array_equal(vr, v)
    # THD positions restart per packed sequence
    cu = np.array([0, 5, 5, 2 * S])
    qt, kt, _ = pj.qkv_projection_rope(x, *w, oracle.thd_positions(cu, 2 * S), cfg)
    rq, rk = oracle.rope_qk_thd(q, k, cu, cfg)
    assert np.array_equal(qt, rq) and np.array_equal(kt, rk)
