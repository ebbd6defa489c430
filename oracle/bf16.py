"""Rounding of fp64 values to bfloat16 (test infrastructure, part of the oracle).

bfloat16 keeps the float32 exponent range and an 8-bit significand (7 stored
bits). The rounding is IEEE round-to-nearest, ties-to-even, applied ONCE to the
fp64 value. Going through float32 first would round twice and can move a value
that sits just off a bf16 midpoint onto it, which is why this is not
``torch.tensor(x, dtype=float64).to(torch.bfloat16)``.

The rotated q and k, and the cos/sin table, keep the q/k dtype per the
rope_utils page ("nemo_automodel.components.models.gpt_oss.rope_utils",
_apply_rotary_emb_qk: tables rounded to the dtype; outputs preserve the dtype).
"""

import numpy as np

_MIN_EXP_ULP = -133          # ulp of the bf16 subnormals: 2^-126 * 2^-7
_OVERFLOW = 2.0 ** 128       # first value past the largest finite bf16


def round_bf16(x):
    """Round an fp64 array to the nearest bf16 value (ties to even), returned as fp64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    xf = x[finite]
    # frexp: x = m * 2^e with 0.5 <= |m| < 1, so the leading bit is 2^(e-1) and
    # an 8-bit significand has its last bit at 2^(e-8).
    _, e = np.frexp(xf)
    ulp_exp = np.maximum(e.astype(np.int64) - 8, _MIN_EXP_ULP)
    scaled = np.ldexp(xf, -ulp_exp)          # exact: scaling by a power of two
    rounded = np.ldexp(np.rint(scaled), ulp_exp)  # rint is ties-to-even
    rounded = np.where(np.abs(rounded) >= _OVERFLOW, np.copysign(np.inf, rounded), rounded)
    out[finite] = rounded
    return out


def bf16_bits(x):
    """Bit pattern (uint16) of fp64 values that are already exact bf16 values."""
    x = np.asarray(x, dtype=np.float64)
    f32 = x.astype(np.float32)  # exact for bf16-representable values
    if not np.array_equal(f32.astype(np.float64), x, equal_nan=True):
        raise ValueError("bf16_bits: input holds values that are not exact bf16")
    bits = f32.view(np.uint32) >> np.uint32(16)
    lost = f32.view(np.uint32) & np.uint32(0xFFFF)
    if np.any(lost[np.isfinite(x)] != 0):
        raise ValueError("bf16_bits: input holds values that are not exact bf16")
    return bits.astype(np.uint16)


def from_bf16_bits(bits):
    """fp64 values of a uint16 array of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)
