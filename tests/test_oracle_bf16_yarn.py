"""Pins for the oracle's bf16 rounding, YaRN frequencies and cos/sin table.

The rounding is pinned against torch's float32 -> bfloat16 conversion (a library
routine, correct for fp32 inputs) and hand-built ties. The YaRN frequencies are
pinned by what the YaRN "NTK-by-parts" construction promises rather than by its
formula: the ramp boundaries are the dimensions that complete ntk_beta and
ntk_alpha turns over the original context, dimensions below / above them keep /
divide their frequency, and plain RoPE (a geometric sequence starting at 1)
comes back at scaling factor 1. The table is pinned by the angle-addition
identity, cos^2 + sin^2 = c^2 and row 0.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------- bf16 rounding ----------------

def _rne_fraction(x: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a rational to bf16 (8-bit significand), for the pins."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    ulp = Fraction(2) ** max(e - 7, -133)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def test_round_bf16_matches_torch_for_fp32_inputs():
    g = torch.Generator().manual_seed(11)
    x32 = torch.randn(200000, generator=g, dtype=torch.float32) * torch.exp(
        torch.randn(200000, generator=g) * 8)
    ref = x32.to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x32.to(torch.float64).numpy())
    assert np.array_equal(got, ref)


def test_round_bf16_ties_and_double_rounding():
    one = 1.0
    assert oracle.round_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0                    # tie -> even
    assert oracle.round_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6     # tie -> even
    # Just above a tie: one rounding goes up. Rounding through float32 first would
    # land on the tie and then go down to 1.0.
    x = one + 2.0 ** -8 + 2.0 ** -30
    assert np.float32(x) == np.float32(one + 2.0 ** -8)
    assert oracle.round_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(np.array([-x]))[0] == -(1.0 + 2.0 ** -7)
    # subnormals: spacing 2^-133
    assert oracle.round_bf16(np.array([2.0 ** -134]))[0] == 0.0
    assert oracle.round_bf16(np.array([3 * 2.0 ** -134]))[0] == 2.0 ** -132
    # overflow
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127          # largest finite bf16 (odd significand)
    assert oracle.round_bf16(np.array([big]))[0] == big
    assert oracle.round_bf16(np.array([big + 2.0 ** 118]))[0] == big
    assert np.isinf(oracle.round_bf16(np.array([big + 2.0 ** 119]))[0])   # tie -> even = 2^128


def test_round_bf16_matches_exact_rationals():
    rng = np.random.default_rng(5)
    xs = rng.standard_normal(2000) * np.exp2(rng.integers(-20, 20, 2000))
    got = oracle.round_bf16(xs)
    for x, y in zip(xs, got):
        assert Fraction(float(y)) == _rne_fraction(Fraction(float(x)))


def test_bf16_bits_roundtrip():
    assert oracle.bf16_bits(np.array([1.0, -2.0, 1.34375])).tolist() == [0x3F80, 0xC000, 0x3FAC]
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    vals = oracle.from_bf16_bits(bits)
    fin = np.isfinite(vals)
    assert np.array_equal(oracle.bf16_bits(vals[fin]), bits[fin])
    with pytest.raises(ValueError):
        oracle.bf16_bits(np.array([1.0 + 2.0 ** -9]))


# ---------------- YaRN ----------------

CFG = oracle.RopeConfig()


def test_page_constants():
    # gpt-oss-20b print-out: q_proj 2880->4096, k/v_proj 2880->512; head_dim 64.
    assert 4096 // CFG.head_dim == 64 and 512 // CFG.head_dim == 8
    # GptOssAttention.softmax_scale = head_dim ** -0.5
    assert CFG.head_dim ** -0.5 == 0.125
    # RotaryEmbedding defaults: initial_context_length 4096, ntk_alpha 1, ntk_beta 32;
    # factor 32 gives the 128K context of the release notes.
    assert CFG.initial_context_length * CFG.scaling_factor == 131072


def test_concentration_closed_form():
    _, c, _ = oracle.yarn_params(CFG)
    assert c == pytest.approx(1.0 + 0.1 * math.log(32.0), abs=0)
    assert abs(c - 1.3465735902799727) < 1e-15
    _, c1, _ = oracle.yarn_params(oracle.RopeConfig(scaling_factor=1.0))
    assert c1 == 1.0


def test_plain_rope_at_factor_one():
    om, c, _ = oracle.yarn_params(oracle.RopeConfig(scaling_factor=1.0))
    assert om[0] == 1.0 and c == 1.0
    ratio = om[1:] / om[:-1]
    assert np.allclose(ratio, 150000.0 ** (-2.0 / 64), rtol=1e-14, atol=0)


def _theta_cont(x, cfg):
    return cfg.base ** (-2.0 * x / cfg.rotary_dim)


def test_yarn_boundaries_are_turn_counts():
    om, c, (lo, hi) = oracle.yarn_params(CFG)
    L0 = CFG.initial_context_length
    # The boundary dimension lo turns ntk_beta times over the original context,
    # hi turns ntk_alpha times.
    assert L0 * _theta_cont(lo, CFG) / (2 * math.pi) == pytest.approx(CFG.ntk_beta, rel=1e-12)
    assert L0 * _theta_cont(hi, CFG) / (2 * math.pi) == pytest.approx(CFG.ntk_alpha, rel=1e-12)
    assert lo < hi


def test_yarn_regions_and_ramp():
    om, c, (lo, hi) = oracle.yarn_params(CFG)
    s = CFG.scaling_factor
    i = np.arange(32)
    theta = np.array([_theta_cont(x, CFG) for x in i])
    fast = i <= lo          # many turns: keep the frequency
    slow = i >= hi          # few turns: interpolate (divide by s)
    assert fast.sum() == 9 and slow.sum() == 14
    assert np.allclose(om[fast], theta[fast], rtol=1e-14)
    assert np.allclose(om[slow], theta[slow] / s, rtol=1e-14)
    # wavelengths of the slow dims are stretched exactly s times
    assert np.allclose((2 * np.pi / om[slow]) / (2 * np.pi / theta[slow]), s, rtol=1e-13)
    # in between, the blend weight is affine in the index, 0 at lo and 1 at hi
    mid = ~fast & ~slow
    w = (theta[mid] - om[mid]) / (theta[mid] - theta[mid] / s)
    A = np.stack([i[mid], np.ones(mid.sum())], axis=1)
    coef, res, *_ = np.linalg.lstsq(A, w, rcond=None)
    assert np.allclose(A @ coef, w, atol=1e-13)
    assert coef[0] * lo + coef[1] == pytest.approx(0.0, abs=1e-12)
    assert coef[0] * hi + coef[1] == pytest.approx(1.0, abs=1e-12)
    # monotone and bracketed
    assert np.all(np.diff(om) < 0)
    assert np.all(om <= theta + 1e-18) and np.all(om >= theta / s - 1e-18)


# ---------------- table ----------------

def test_table_row0_and_norm():
    cos, sin = oracle.cos_sin_table(CFG, [0])
    assert np.all(cos == 1.34375) and np.all(sin == 0.0)
    assert np.all(oracle.bf16_bits(cos) == 0x3FAC)
    cu, su = oracle.cos_sin_table(CFG, np.arange(0, 131072, 97), rounded=False)
    _, c, _ = oracle.yarn_params(CFG)
    assert np.allclose(cu ** 2 + su ** 2, c * c, rtol=1e-13)


def test_table_angle_addition():
    """(C_p + iS_p)(C_q + iS_q) / c = C_{p+q} + i S_{p+q}: the angle is linear in p."""
    _, c, _ = oracle.yarn_params(CFG)
    rng = np.random.default_rng(3)
    p = rng.integers(0, 65536, 64)
    q = rng.integers(0, 65536, 64)
    cp, sp = oracle.cos_sin_table(CFG, p, rounded=False)
    cq, sq = oracle.cos_sin_table(CFG, q, rounded=False)
    cpq, spq = oracle.cos_sin_table(CFG, p + q, rounded=False)
    prod = (cp + 1j * sp) * (cq + 1j * sq) / c
    assert np.allclose(prod.real, cpq, atol=1e-9)
    assert np.allclose(prod.imag, spq, atol=1e-9)
    # the per-position step of the angle is the YaRN frequency, recovered by atan2
    om, _, _ = oracle.yarn_params(CFG)
    c1, s1 = oracle.cos_sin_table(CFG, [1], rounded=False)
    assert np.allclose(np.arctan2(s1[0], c1[0]), om, rtol=1e-13, atol=0)


def test_table_is_rounded_once():
    pos = np.arange(0, 131072, 13)
    cu, su = oracle.cos_sin_table(CFG, pos, rounded=False)
    cr, sr = oracle.cos_sin_table(CFG, pos, rounded=True)
    assert np.array_equal(cr, oracle.round_bf16(cu)) and np.array_equal(sr, oracle.round_bf16(su))
    assert np.max(np.abs(cr - cu)) <= 2.0 ** -8      # half an ulp of values below 2


def test_freqs_cis_layout():
    fc = oracle.freqs_cis(CFG, 4)
    cos, sin = oracle.cos_sin_table(CFG, np.arange(4))
    assert fc.shape == (4, 64)
    assert np.array_equal(fc[:, :32], cos) and np.array_equal(fc[:, 32:], sin)


def test_table_golden_regression():
    """Stored by tests/golden/make_golden.py, which calls only the oracle."""
    with open(os.path.join(GOLDEN, "yarn_table.json")) as f:
        gold = json.load(f)
    om, c, (lo, hi) = oracle.yarn_params(CFG)
    assert [float.fromhex(h) for h in gold["omega_hex"]] == om.tolist()
    assert float.fromhex(gold["concentration_hex"]) == c
    pos = gold["positions"]
    cs = oracle.freqs_cis(CFG, max(pos) + 1)[pos]
    assert oracle.bf16_bits(cs).tolist() == gold["table_bits"]
