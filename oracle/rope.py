"""Rotation of q and k by the YaRN table (oracle).

Page "nemo_automodel.components.models.gpt_oss.rope_utils":
  * apply_rotary_emb: cos and sin each cover rotary_dim/2; when rotary_dim is
    below head_dim only the first rotary_dim dims rotate and the rest pass
    through unchanged.
  * _apply_rotary_emb_qk: q and k rotate with one shared, dtype-rounded table;
    each output keeps its input's dtype.
  * apply_rotary_emb_qk: BSHD [batch, seq, heads, head_dim] or packed THD
    [tokens, heads, head_dim] with cu_seqlens [num_sequences + 1].
  * position_ids_to_freqs_cis: table rows are picked by position id.

Readings (listed in the design doc): the pairs are half-split, so dim i pairs with
dim i + rotary_dim/2 and both use omega_i (the table concatenates a cos half and
a sin half). The pair (x1, x2) is treated as the complex number x1 + i*x2 and
multiplied by (C + i*S), which is the usual RoPE sign convention:
  y1 = x1*C - x2*S,  y2 = x2*C + x1*S.
Each y is formed exactly in fp64 (products of two bf16 values are exact) and
rounded once to bf16. Positions: BSHD p = s; THD p = t - cu_seqlens[n], so
every packed sequence starts again at 0.
"""

import numpy as np

from .bf16 import round_bf16
from .yarn import RopeConfig, cos_sin_table


def rotate(x, cos, sin, round_output=True):
    """Rotate the first rotary_dim dims of x[..., D] by per-row cos/sin [..., rotary_dim/2].

    cos and sin broadcast against x[..., 0]; rotary_dim = 2 * cos.shape[-1].
    """
    x = np.asarray(x, dtype=np.float64)
    half = cos.shape[-1]
    rd = 2 * half
    if rd > x.shape[-1]:
        raise ValueError("rotary_dim exceeds head_dim")
    x1 = x[..., :half]
    x2 = x[..., half:rd]
    y1 = x1 * cos - x2 * sin
    y2 = x2 * cos + x1 * sin
    y = np.concatenate([y1, y2, x[..., rd:]], axis=-1)
    if round_output:
        y = np.concatenate([round_bf16(y[..., :rd]), y[..., rd:]], axis=-1)
    return y


def rope_qk_bshd(q, k, cfg: RopeConfig = RopeConfig(), round_output=True, rounded_table=True):
    """q [B,S,Hq,D], k [B,S,Hkv,D] (fp64 holding bf16 values) -> rotated (q, k)."""
    S = q.shape[1]
    cos, sin = cos_sin_table(cfg, np.arange(S), rounded=rounded_table)
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    return rotate(q, c, s, round_output), rotate(k, c, s, round_output)


def thd_positions(cu_seqlens, total):
    """Position of every packed token: its offset inside its own sequence."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pos = np.zeros(total, dtype=np.int64)
    for n in range(len(cu) - 1):
        pos[cu[n]:cu[n + 1]] = np.arange(cu[n + 1] - cu[n])
    return pos


def rope_qk_thd(q, k, cu_seqlens, cfg: RopeConfig = RopeConfig(), round_output=True):
    """q [T,Hq,D], k [T,Hkv,D] packed by cu_seqlens -> rotated (q, k)."""
    T = q.shape[0]
    pos = thd_positions(cu_seqlens, T)
    cos, sin = cos_sin_table(cfg, pos)
    c = cos[:, None, :]
    s = sin[:, None, :]
    return rotate(q, c, s, round_output), rotate(k, c, s, round_output)
