"""The q/k/v projections of GPT-OSS attention, with and without the RoPE applied to their output (oracle).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``.

The gpt-oss-20b module print-out ("gpt-oss-20b 模型结构") lists q_proj
2880 -> 4096, k_proj and v_proj 2880 -> 512, each a Linear with bias, ahead of
the attention; the rope_utils page ("nemo_automodel.components.models.gpt_oss
.rope_utils", _apply_rotary_emb_qk) then rotates q and k, which keep their
dtype. Readings used here:

* A projection is z = x W^T + b with x [T, hidden], W [out, hidden] (Linear's
  weight layout) and b [out], all bf16 values; z is computed exactly (fp64 on
  bf16 inputs) and rounded once to bf16, the projection's output dtype.
* q and k are the rounded projections reshaped to heads of 64 ([T, Hq, 64] and
  [T, Hkv, 64]); the fused form rotates exactly those bf16 values at each
  token's position (oracle.rope: exact rotation, one more rounding), so it
  equals the unfused sequence projection -> rotation element for element.

Pinned by tests/test_oracle_projection.py.
"""

import numpy as np

from .bf16 import round_bf16
from .rope import rotate
from .yarn import RopeConfig, cos_sin_table


def linear(x, w, b):
    """Unrounded x W^T + b in fp64: x [T, hidden], w [out, hidden], b [out] -> [T, out]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    z = x @ w.T
    if b is not None:
        z = z + np.asarray(b, dtype=np.float64)[None, :]
    return z


def qkv_projection(x, wq, bq, wk, bk, wv, bv, head_dim=64):
    """q [T, Hq, D], k [T, Hkv, D], v [T, Hkv, D]: each projection rounded once to bf16."""
    T = np.shape(x)[0]
    out = []
    for w, b in ((wq, bq), (wk, bk), (wv, bv)):
        z = round_bf16(linear(x, w, b))
        out.append(z.reshape(T, -1, head_dim))
    return tuple(out)


def qkv_projection_rope(x, wq, bq, wk, bk, wv, bv, positions, cfg: RopeConfig = RopeConfig()):
    """The projections, then q and k rotated at positions [T] (v unrotated)."""
    q, k, v = qkv_projection(x, wq, bq, wk, bk, wv, bv, cfg.head_dim)
    c, s = cos_sin_table(cfg, np.asarray(positions, dtype=np.int64))
    c, s = c[:, None, :], s[:, None, :]
    return rotate(q, c, s), rotate(k, c, s), v
