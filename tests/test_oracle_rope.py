"""Pins for the oracle's q/k rotation.

* The rotation is complex multiplication of x1 + i*x2 by the table entry
  C + i*S (Python complex arithmetic, a library routine), which fixes the sign
  convention and the half-split pairing.
* With unrounded tables and outputs, <R_p q, R_p' k> depends only on p - p'
  (the relative-position property RoPE exists for), and each pair's norm
  grows by the concentration c.
* With the bf16 table, position 0 multiplies by R(c) = 1.34375 exactly.
* Each output is the exact rational result rounded once (fractions.Fraction).
* Partial rotary: only the first rotary_dim dims rotate (apply_rotary_emb).
* THD positions restart at 0 for every packed sequence.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from test_oracle_bf16_yarn import _rne_fraction

CFG = oracle.RopeConfig()


def _bf16_randn(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16).double().numpy()


def test_rotation_is_complex_multiplication():
    x = _bf16_randn((50, 64), 1)
    pos = np.arange(0, 131072, 131072 // 50)[:50]
    cos, sin = oracle.cos_sin_table(CFG, pos)
    y = oracle.rotate(x, cos, sin, round_output=False)
    for r in range(50):
        for i in range(32):
            z = complex(x[r, i], x[r, i + 32]) * complex(cos[r, i], sin[r, i])
            assert y[r, i] == pytest.approx(z.real, abs=1e-15)
            assert y[r, i + 32] == pytest.approx(z.imag, abs=1e-15)


@pytest.mark.parametrize("p,pp,delta", [(5, 3, 100), (0, 7, 4096), (131000, 60000, 71),
                                        (127, 128, 65536)])
def test_relative_position_property(p, pp, delta):
    q = _bf16_randn((64,), 2)
    k = _bf16_randn((64,), 3)

    def dot(a, b):
        ca, sa = oracle.cos_sin_table(CFG, [a], rounded=False)
        cb, sb = oracle.cos_sin_table(CFG, [b], rounded=False)
        return float(oracle.rotate(q, ca[0], sa[0], False) @ oracle.rotate(k, cb[0], sb[0], False))

    d0, d1 = dot(p, pp), dot(p + delta, pp + delta)
    assert d1 == pytest.approx(d0, rel=1e-9, abs=1e-10)


def test_pair_norm_scales_by_concentration():
    _, c, _ = oracle.yarn_params(CFG)
    x = _bf16_randn((20, 64), 4)
    cos, sin = oracle.cos_sin_table(CFG, np.arange(1000, 1020), rounded=False)
    y = oracle.rotate(x, cos, sin, round_output=False)
    n_in = x[:, :32] ** 2 + x[:, 32:] ** 2
    n_out = y[:, :32] ** 2 + y[:, 32:] ** 2
    assert np.allclose(n_out, c * c * n_in, rtol=1e-12)


def test_position_zero_scales_by_rounded_concentration():
    x = _bf16_randn((30, 64), 5)
    cos, sin = oracle.cos_sin_table(CFG, np.zeros(30, dtype=np.int64))
    y = oracle.rotate(x, cos, sin)
    assert np.array_equal(y, oracle.round_bf16(1.34375 * x))


def test_single_rounding_of_exact_result():
    x = _bf16_randn((40, 64), 6)
    pos = np.random.default_rng(0).integers(0, 131072, 40)
    cos, sin = oracle.cos_sin_table(CFG, pos)
    y = oracle.rotate(x, cos, sin)
    for r in range(40):
        for i in range(32):
            x1, x2 = Fraction(float(x[r, i])), Fraction(float(x[r, i + 32]))
            C, S = Fraction(float(cos[r, i])), Fraction(float(sin[r, i])),
            assert Fraction(float(y[r, i])) == _rne_fraction(x1 * C - x2 * S)
            assert Fraction(float(y[r, i + 32])) == _rne_fraction(x2 * C + x1 * S)


def test_partial_rotary_passes_tail_through():
    cfg = oracle.RopeConfig(rotary_dim=32)
    x = _bf16_randn((10, 64), 7)
    cos, sin = oracle.cos_sin_table(cfg, np.arange(10))
    assert cos.shape == (10, 16)
    y = oracle.rotate(x, cos, sin)
    assert np.array_equal(y[:, 32:], x[:, 32:])
    z = (x[:, :16] + 1j * x[:, 16:32]) * (cos + 1j * sin)
    assert np.array_equal(y[:, :16], oracle.round_bf16(z.real))
    assert np.array_equal(y[:, 16:32], oracle.round_bf16(z.imag))


def test_thd_positions_restart_per_sequence():
    lengths = [5, 0, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    q = _bf16_randn((T, 4, 64), 8)
    k = _bf16_randn((T, 2, 64), 9)
    rq, rk = oracle.rope_qk_thd(q, k, cu, CFG)
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        if b == a:
            continue
        bq, bk = oracle.rope_qk_bshd(q[None, a:b], k[None, a:b], CFG)
        assert np.array_equal(rq[a:b], bq[0]) and np.array_equal(rk[a:b], bk[0])
    assert np.array_equal(oracle.thd_positions(cu, T), [0, 1, 2, 3, 4, 0, 1, 2, 3, 4, 5, 6, 7, 8, 0, 1, 2])
