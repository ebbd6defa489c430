"""Sink + GQA + sliding-window causal attention, written as its plain definition (oracle).

Sources:
  * "nemo_automodel.components.models.gpt_oss.layers", GptOssAttention:
    softmax_scale = head_dim ** -0.5; attributes sinks (one per query head) and
    sliding_window; num_attention_heads / num_key_value_heads (grouped-query
    attention); use_sliding_attention picks the window layers.
  * Transformers v4.55.0 release notes, section "Architecture": layers alternate
    between full context and a sliding 128-token window; each head has a learned
    sink that adds a term to the denominator of the softmax.
  * "nemo_automodel.components.models.gpt_oss.model", GptOssForCausalLM.forward:
    BSHD [batch, seq] inputs or packed THD inputs described by cu_seqlens.

For query token t at position i, query head h, and key token u at position j in
the same sequence (readings listed in the design doc):
  g(h)  = floor(h / (Hq / Hkv))                    contiguous head groups
  s     = tau * <q~_{t,h}, k~_{u,g(h)}>            tau = softmax_scale
  visible(i, j) = j <= i and (W == 0 or i - j < W)  W counts the query itself
  M     = max(sigma_h, max over visible s)
  Z     = exp(sigma_h - M) + sum over visible exp(s - M)
  o_{t,h} = sum over visible exp(s - M) * v_{u,g(h)} / Z
sigma_h is the sink logit, in the same units as s. A row with no visible key
returns 0 (also with sigma_h = -inf, where the formula would give 0/0).

Everything is fp64; the result is not rounded. Rows are evaluated in blocks of
independent query rows, and the keys no row of a block can see are left out of
that block's sums (their weight is exactly zero); neither changes the
definition.
"""

import numpy as np

from .rope import rotate, rope_qk_bshd, rope_qk_thd, thd_positions
from .yarn import RopeConfig, cos_sin_table


def _visible(q_pos, k_pos, window):
    vis = k_pos[None, :] <= q_pos[:, None]
    if window > 0:
        vis &= (q_pos[:, None] - k_pos[None, :]) < window
    return vis


def sink_attention(q, k, v, sinks, scale, q_pos, k_pos, window, row_block=256):
    """One sequence. q [Tq,Hq,D], k/v [Tk,Hkv,D] (already rotated), positions int [Tq]/[Tk].

    Returns fp64 [Tq, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    sinks = np.asarray(sinks, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    Tq, Hq, D = q.shape
    Tk, Hkv, _ = k.shape
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    out = np.zeros((Tq, Hq, v.shape[-1]), dtype=np.float64)
    if Tq == 0 or Tk == 0:
        return out
    for r0 in range(0, Tq, row_block):
        r1 = min(Tq, r0 + row_block)
        vis = _visible(q_pos[r0:r1], k_pos, window)          # [rows, Tk]
        cols = np.nonzero(vis.any(axis=0))[0]
        if cols.size == 0:
            continue
        vis = vis[:, cols]
        rows = r1 - r0
        for g in range(Hkv):
            K = k[cols, g, :]                                 # [n, D]
            V = v[cols, g, :]
            Q = q[r0:r1, g * G:(g + 1) * G, :].reshape(rows * G, D)
            s = scale * (Q @ K.T).reshape(rows, G, cols.size)
            s = np.where(vis[:, None, :], s, -np.inf)
            sig = sinks[g * G:(g + 1) * G][None, :]           # [1, G]
            smax = s.max(axis=-1)                              # [rows, G]
            M = np.maximum(sig, smax)
            dead = ~np.isfinite(M)                             # sigma = -inf and nothing visible
            Ms = np.where(dead, 0.0, M)
            e = np.exp(s - Ms[..., None])                      # masked -> exp(-inf) = 0
            Z = np.exp(sig - Ms) + e.sum(axis=-1)
            o = (e.reshape(rows * G, cols.size) @ V).reshape(rows, G, -1)
            Zs = np.where(Z > 0, Z, 1.0)
            o = o / Zs[..., None]
            o[dead] = 0.0
            out[r0:r1, g * G:(g + 1) * G, :] = o
    return out


def prefill_bshd(q, k, v, sinks, scale, window, cfg: RopeConfig = RopeConfig(), rotate_qk=True):
    """BSHD prefill. q [B,S,Hq,D], k/v [B,S,Hkv,D] (fp64 holding bf16 values).

    With rotate_qk the YaRN rotation is applied first (q and k rounded to bf16);
    otherwise q and k are taken as already rotated. Returns fp64 [B,S,Hq,D].
    """
    if rotate_qk:
        q, k = rope_qk_bshd(q, k, cfg)
    B, S = q.shape[:2]
    pos = np.arange(S)
    out = np.zeros(q.shape[:3] + (v.shape[-1],), dtype=np.float64)
    for b in range(B):
        out[b] = sink_attention(q[b], k[b], v[b], sinks, scale, pos, pos, window)
    return out


def prefill_thd(q, k, v, cu_seqlens, sinks, scale, window, cfg: RopeConfig = RopeConfig(), rotate_qk=True):
    """Packed THD prefill. q [T,Hq,D], k/v [T,Hkv,D], cu_seqlens [N+1]. Returns fp64 [T,Hq,D]."""
    if rotate_qk:
        q, k = rope_qk_thd(q, k, cu_seqlens, cfg)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.zeros(q.shape[:2] + (v.shape[-1],), dtype=np.float64)
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        if b <= a:
            continue
        pos = np.arange(b - a)
        out[a:b] = sink_attention(q[a:b], k[a:b], v[a:b], sinks, scale, pos, pos, window)
    return out


def prefill_rows(q, k, v, sinks, scale, window, rows, cfg: RopeConfig = RopeConfig(), rotate_qk=True,
                 positions=None):
    """Selected query rows of one sequence: q [S,Hq,D], k/v [S,Hkv,D]; rows int [R].

    Only the keys the selected rows can see are rotated and used. ``positions``
    (default 0..S-1) gives each token's position. Returns fp64 [R, Hq, D].
    """
    rows = np.asarray(rows, dtype=np.int64)
    S = q.shape[0]
    pos = np.arange(S) if positions is None else np.asarray(positions, dtype=np.int64)
    kmax = int(rows.max()) + 1
    kmin = 0 if window <= 0 else max(0, int(rows.min()) - window + 1)
    kr = np.arange(kmin, kmax)
    qs, ks, vs = q[rows], k[kr], v[kr]
    if rotate_qk:
        cq, sq = cos_sin_table(cfg, pos[rows])
        ck, sk = cos_sin_table(cfg, pos[kr])
        qs = rotate(qs, cq[:, None, :], sq[:, None, :])
        ks = rotate(ks, ck[:, None, :], sk[:, None, :])
    return sink_attention(qs, ks, vs, sinks, scale, pos[rows], pos[kr], window, row_block=16)


def decode(q, k_cache, v_cache, cache_seqlens, sinks, scale, window, cfg: RopeConfig = RopeConfig(), rotate_q=True):
    """One new token per sequence against a KV cache.

    q [N,Hq,D] (un-rotated when rotate_q); k_cache / v_cache [N,Lmax,Hkv,D] with K
    already rotated; cache_seqlens [N] counts the cached rows including the new
    token's own, so the query sits at position L_n - 1 and sees rows 0..L_n-1
    (the last min(L_n, W) of them on a window layer). Returns fp64 [N,Hq,D].
    """
    L = np.asarray(cache_seqlens, dtype=np.int64)
    N = q.shape[0]
    out = np.zeros(q.shape[:2] + (v_cache.shape[-1],), dtype=np.float64)
    for n in range(N):
        Ln = int(L[n])
        if Ln <= 0:
            continue
        qn = q[n][None]                                          # [1,Hq,D]
        if rotate_q:
            c, s = cos_sin_table(cfg, [Ln - 1])
            qn = rotate(qn, c[:, None, :], s[:, None, :])
        lo = 0 if window <= 0 else max(0, Ln - window)
        kp = np.arange(lo, Ln)
        out[n] = sink_attention(qn, k_cache[n, lo:Ln], v_cache[n, lo:Ln], sinks, scale,
                                np.array([Ln - 1]), kp, window)[0]
    return out
