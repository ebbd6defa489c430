"""Gradients of the sink + GQA + sliding-window attention, and its log-sum-exp (oracle).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``.

The forward is the definition in ``oracle.attention`` (pages
"nemo_automodel.components.models.gpt_oss.layers", GptOssAttention: sinks,
sliding_window, softmax_scale; Transformers v4.55.0 release notes,
"Architecture": a learned per-head sink adds a term to the softmax
denominator). No page prints a backward pass; the pages describe a training
framework (the same docs' model and FSDP pages), so the gradients here are the
plain derivatives of that forward definition, written out:

For one query row i of head h (group g), visible keys j, tau = softmax_scale:
  s_ij  = tau <q~_i, k~_j>
  lse_i = log( exp(sigma_h) + sum_j exp(s_ij) )          (natural log)
  p_ij  = exp(s_ij - lse_i),   o_i = sum_j p_ij v_j
Given dO = dL/do:
  dv_j      += sum_i p_ij dO_i                       (over the 8 heads of the group)
  dP_ij      = <dO_i, v_j>
  D_i        = <dO_i, o_i>  = sum_j p_ij dP_ij
  dS_ij      = p_ij (dP_ij - D_i)
  dq~_i      = tau sum_j dS_ij k~_j
  dk~_j     += tau sum_i dS_ij q~_i
  dsigma_h   = - sum_i exp(sigma_h - lse_i) D_i      (the sink's probability times -D_i)
A row with nothing visible and sigma = -inf has lse = -inf, o = 0 and no gradient.

RoPE: q~ = R q and k~ = R k with the dtype-rounded cos/sin table as constants
(page "nemo_automodel.components.models.gpt_oss.rope_utils",
_apply_rotary_emb_qk). The rounding of the rotated values to bf16 is taken as
the identity for the gradient (a dtype cast passes the gradient through), so
dq = R^T dq~ and dk = R^T dk~, with R^T the rotation by the opposite angle:
  dx1 = dy1 C + dy2 S,   dx2 = dy2 C - dy1 S.

Everything is fp64 and unrounded. Pinned by tests/test_oracle_backward.py
(finite differences of the forward, torch autograd of an independently written
forward, closed forms). The tolerance a bf16 implementation is held to is not
part of the definition and lives with the GPU tests.
"""

import numpy as np

from .attention import _visible
from .rope import rotate, rope_qk_bshd, rope_qk_thd, thd_positions
from .yarn import RopeConfig, cos_sin_table


def rotate_transpose(dy, cos, sin):
    """R^T applied to dy[..., D] (the first rotary_dim dims; the rest pass through)."""
    dy = np.asarray(dy, dtype=np.float64)
    half = cos.shape[-1]
    rd = 2 * half
    d1 = dy[..., :half]
    d2 = dy[..., half:rd]
    return np.concatenate([d1 * cos + d2 * sin, d2 * cos - d1 * sin, dy[..., rd:]], axis=-1)


def sink_attention_backward(q, k, v, sinks, scale, q_pos, k_pos, window, dout):
    """One sequence, q [Tq,Hq,D] and k/v [Tk,Hkv,D] already rotated, dout [Tq,Hq,D].

    Returns (o, lse, dq~, dk~, dv, dsinks): fp64, lse [Tq,Hq] natural log.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    sinks = np.asarray(sinks, dtype=np.float64)
    Tq, Hq, D = q.shape
    Tk, Hkv, _ = k.shape
    G = Hq // Hkv
    vis = _visible(np.asarray(q_pos, dtype=np.int64), np.asarray(k_pos, dtype=np.int64), window)  # [Tq,Tk]
    o = np.zeros((Tq, Hq, v.shape[-1]))
    lse = np.full((Tq, Hq), -np.inf)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsinks = np.zeros(Hq)
    for h in range(Hq):
        g = h // G
        Q, K, V, dO = q[:, h], k[:, g], v[:, g], dout[:, h]
        s = np.where(vis, scale * (Q @ K.T), -np.inf)             # [Tq,Tk]
        m = np.maximum(sinks[h], s.max(axis=1, initial=-np.inf))  # per-row max for a stable log-sum-exp
        live = np.isfinite(m)
        mz = np.where(live, m, 0.0)
        z = np.exp(sinks[h] - mz) + np.exp(s - mz[:, None]).sum(axis=1)
        l = np.where(live, mz + np.log(np.where(live, z, 1.0)), -np.inf)
        p = np.where(live[:, None], np.exp(s - np.where(live, l, 0.0)[:, None]), 0.0)
        oh = p @ V
        dP = dO @ V.T
        Dr = (dO * oh).sum(axis=1)
        dS = p * (dP - Dr[:, None])
        dq[:, h] = scale * (dS @ K)
        dk[:, g] += scale * (dS.T @ Q)
        dv[:, g] += p.T @ dO
        psink = np.where(live, np.exp(sinks[h] - np.where(live, l, 0.0)), 0.0)
        dsinks[h] = -(psink * Dr).sum()
        o[:, h] = oh
        lse[:, h] = l
    return o, lse, dq, dk, dv, dsinks


def prefill_bshd_backward(q, k, v, sinks, scale, window, dout, cfg: RopeConfig = RopeConfig(),
                          rotate_qk=True, round_rotation=True):
    """BSHD: q [B,S,Hq,D], k/v [B,S,Hkv,D], dout [B,S,Hq,D] (fp64 holding bf16 values).

    With rotate_qk, q and k are rotated as in the forward (rounded to bf16 unless
    round_rotation is False) and the gradients are rotated back with R^T.
    Returns dict(o, lse [B,S,Hq], dq, dk, dv, dsinks [Hq]).
    """
    B, S = q.shape[:2]
    if rotate_qk:
        qr, kr = rope_qk_bshd(q, k, cfg, round_output=round_rotation)
    else:
        qr, kr = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
    pos = np.arange(S)
    out = {n: [] for n in ("o", "lse", "dq", "dk", "dv")}
    dsinks = np.zeros(q.shape[2])
    for b in range(B):
        r = sink_attention_backward(qr[b], kr[b], v[b], sinks, scale, pos, pos, window, dout[b])
        for n, x in zip(("o", "lse", "dq", "dk", "dv"), r[:5]):
            out[n].append(x)
        dsinks += r[5]
    res = {n: np.stack(x) for n, x in out.items()}
    if rotate_qk:
        cos, sin = cos_sin_table(cfg, pos)
        rot = (cos[None, :, None, :], sin[None, :, None, :])
        res["dq"] = rotate_transpose(res["dq"], *rot)
        res["dk"] = rotate_transpose(res["dk"], *rot)
    res["dsinks"] = dsinks
    return res


def prefill_thd_backward(q, k, v, cu_seqlens, sinks, scale, window, dout, cfg: RopeConfig = RopeConfig(),
                         rotate_qk=True, round_rotation=True):
    """Packed THD: q [T,Hq,D], k/v [T,Hkv,D], dout [T,Hq,D], cu_seqlens [N+1]; positions restart per sequence."""
    T = q.shape[0]
    if rotate_qk:
        qr, kr = rope_qk_thd(q, k, cu_seqlens, cfg, round_output=round_rotation)
    else:
        qr, kr = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    res = {"o": np.zeros(q.shape[:2] + (v.shape[-1],)), "lse": np.full(q.shape[:2], -np.inf),
           "dq": np.zeros(q.shape), "dk": np.zeros(k.shape), "dv": np.zeros(v.shape),
           "dsinks": np.zeros(q.shape[1])}
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b <= a:
            continue
        pos = np.arange(b - a)
        r = sink_attention_backward(qr[a:b], kr[a:b], v[a:b], sinks, scale, pos, pos, window, dout[a:b])
        res["o"][a:b], res["lse"][a:b], res["dq"][a:b], res["dk"][a:b], res["dv"][a:b] = r[:5]
        res["dsinks"] += r[5]
    if rotate_qk:
        pos = thd_positions(cu, T)
        cos, sin = cos_sin_table(cfg, pos)
        rot = (cos[:, None, :], sin[:, None, :])
        res["dq"] = rotate_transpose(res["dq"], *rot)
        res["dk"] = rotate_transpose(res["dk"], *rot)
    return res


def prefill_backward_rows(q, k, v, sinks, scale, window, dout, q_rows, key_lo, key_hi,
                          cfg: RopeConfig = RopeConfig()):
    """Selected gradients of one sequence: q [S,Hq,D], k/v [S,Hkv,D] un-rotated
    (fp64 holding bf16 values), dout [S,Hq,D]; positions 0..S-1.

    Returns dq for the query rows q_rows and dk, dv for the keys key_lo..key_hi-1.
    Each equals the matching entry of
    prefill_bshd_backward: dq of a row depends on that row's visible keys only,
    and every query that sees one of the keys is included for dk and dv (the
    queries before key_lo cannot see them), so leaving the rest out changes nothing.
    """
    q_rows = np.asarray(q_rows, dtype=np.int64)
    S = q.shape[0]
    out = {}
    # dq: the rows and every key they see
    klo = 0 if window <= 0 else max(0, int(q_rows.min()) - window + 1)
    kr = np.arange(klo, int(q_rows.max()) + 1)
    cq, sq = cos_sin_table(cfg, q_rows)
    ck, sk = cos_sin_table(cfg, kr)
    qs = rotate(q[q_rows], cq[:, None, :], sq[:, None, :])
    ks = rotate(k[kr], ck[:, None, :], sk[:, None, :])
    r = sink_attention_backward(qs, ks, v[kr], sinks, scale, q_rows, kr, window, dout[q_rows])
    out["dq"] = rotate_transpose(r[2], cq[:, None, :], sq[:, None, :])
    # dk, dv: every query that sees a key in [key_lo, key_hi), each with all keys it sees
    q_hi = S - 1 if window <= 0 else min(S - 1, key_hi - 1 + window - 1)
    qr = np.arange(key_lo, q_hi + 1)
    klo = 0 if window <= 0 else max(0, key_lo - window + 1)
    kr = np.arange(klo, q_hi + 1)
    cq, sq = cos_sin_table(cfg, qr)
    ck, sk = cos_sin_table(cfg, kr)
    qs = rotate(q[qr], cq[:, None, :], sq[:, None, :])
    ks = rotate(k[kr], ck[:, None, :], sk[:, None, :])
    r = sink_attention_backward(qs, ks, v[kr], sinks, scale, qr, kr, window, dout[qr])
    sel = slice(key_lo - klo, key_hi - klo)
    ck, sk = ck[sel], sk[sel]
    out["dk"] = rotate_transpose(r[3][sel], ck[:, None, :], sk[:, None, :])
    out["dv"] = r[4][sel]
    return out
