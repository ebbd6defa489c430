"""YaRN rotary frequencies, concentration and the bf16 cos/sin table (oracle).

Page "nemo_automodel.components.models.gpt_oss.rope_utils", entry RotaryEmbedding:
constructor arguments head_dim, base, initial_context_length (default 4096),
scaling_factor (default 1.0), ntk_alpha (default 1.0), ntk_beta (default 32.0),
partial_rotary_factor (rotary_dim = int(head_dim * partial_rotary_factor));
_compute_concentration_and_inv_freq points at the YaRN paper and works over
rotary_dim; _compute_cos_sin builds the tables for num_tokens positions.
Page "nemo_automodel.components.models.gpt_oss.layers", GptOssAttention:
yarn_concentration is the YaRN mscale of rope_scaling['factor'].

Readings where the pages are silent (each listed in the design doc):
  * The frequency ramp is the YaRN "NTK-by-parts" blend, linear in the
    rotary-dimension index i between two unrounded boundaries lo and hi. lo is
    the index whose wavelength fits ntk_beta (beta_fast) times into the original
    context, hi the one that fits ntk_alpha (beta_slow) times. Below lo the
    frequency is kept (extrapolation), above hi it is divided by the scaling
    factor (interpolation).
  * The concentration is the YaRN temperature sqrt(1/t) = 0.1 ln(s) + 1, folded
    into both the cos and the sin table, so q and k each carry one factor.
  * Angles p * omega_i are formed in fp64 from an integer position p; the
    product c * cos(angle) is rounded once to bf16.
"""

import math
from dataclasses import dataclass

import numpy as np

from .bf16 import round_bf16


@dataclass(frozen=True)
class RopeConfig:
    """RotaryEmbedding configuration (rope_utils page, RotaryEmbedding constructor).

    Defaults are GPT-OSS's: head_dim 64 (q_proj 2880->4096 over 64 heads in the
    gpt-oss-20b print-out), RoPE base 150000, YaRN factor 32 over an original
    context of 4096 (4096 * 32 = the "128K context" of the Transformers
    v4.55.0 "Architecture" list), ntk_alpha 1 and ntk_beta 32 (the
    constructor's defaults).
    """

    head_dim: int = 64
    rotary_dim: int = 64
    base: float = 150000.0
    scaling_factor: float = 32.0
    initial_context_length: int = 4096
    ntk_alpha: float = 1.0
    ntk_beta: float = 32.0


def yarn_params(cfg: RopeConfig):
    """Per-pair angular frequencies omega[rotary_dim/2], concentration c, and (lo, hi).

    theta_i = base^(-2i/d) is plain RoPE (d = rotary_dim). With s > 1:
      lo = (d/2) ln(L0 / (2 pi beta_fast)) / ln(base)
      hi = (d/2) ln(L0 / (2 pi beta_slow)) / ln(base)
      gamma_i = clamp((i - lo) / (hi - lo), 0, 1)
      omega_i = theta_i (1 - gamma_i) + (theta_i / s) gamma_i
      c = 0.1 ln(s) + 1
    With s <= 1 the result is plain RoPE: omega = theta and c = 1.
    """
    d = cfg.rotary_dim
    if d <= 0 or d % 2 != 0 or d > cfg.head_dim:
        raise ValueError("rotary_dim must be even, positive and at most head_dim")
    half = d // 2
    idx = np.arange(half, dtype=np.float64)
    # math.pow is the C library's pow, correctly rounded; numpy's vectorised
    # power can be one ulp away from it.
    theta = np.array([math.pow(float(cfg.base), -(2.0 * i) / d) for i in range(half)])
    s = float(cfg.scaling_factor)
    if s <= 1.0:
        return theta, 1.0, (None, None)
    L0 = float(cfg.initial_context_length)
    log_base = math.log(cfg.base)
    lo = half * math.log(L0 / (2.0 * math.pi * cfg.ntk_beta)) / log_base
    hi = half * math.log(L0 / (2.0 * math.pi * cfg.ntk_alpha)) / log_base
    gamma = np.clip((idx - lo) / (hi - lo), 0.0, 1.0)
    omega = theta * (1.0 - gamma) + (theta / s) * gamma
    c = 0.1 * math.log(s) + 1.0
    return omega, c, (lo, hi)


def cos_sin_table(cfg: RopeConfig, positions, rounded=True):
    """cos and sin tables for integer positions: c*cos(p*omega_i), c*sin(p*omega_i).

    Returns two fp64 arrays of shape [len(positions), rotary_dim/2]; with
    ``rounded`` each entry is rounded once to bf16 (the q/k dtype).
    """
    omega, c, _ = yarn_params(cfg)
    p = np.asarray(positions, dtype=np.int64).astype(np.float64)
    angle = p[:, None] * omega[None, :]
    cos = c * np.cos(angle)
    sin = c * np.sin(angle)
    if rounded:
        cos = round_bf16(cos)
        sin = round_bf16(sin)
    return cos, sin


def freqs_cis(cfg: RopeConfig, num_positions, rounded=True):
    """The [num_positions, rotary_dim] table: cos (rotary_dim/2) then sin (rotary_dim/2).

    The rope_utils page (_apply_rotary_emb_qk, freqs_cis argument) describes the
    last dimension as the cosine table concatenated with the sine table.
    """
    cos, sin = cos_sin_table(cfg, np.arange(num_positions), rounded=rounded)
    return np.concatenate([cos, sin], axis=-1)
