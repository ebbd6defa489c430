"""Error model of a bf16 / fp32 backward kernel, for the tolerance of the GPU backward tests.

TEST INFRASTRUCTURE. This is not part of the oracle: the oracle (oracle.backward)
holds only the exact fp64 gradients of the attention's definition. What a kernel
that takes its matrix-core operands in bf16 and accumulates in fp32 may differ
from them by is a property of the arithmetic, stated and derived here.

The kernels round to bf16 (8 significant bits, nearest): dS = p (dP - D) as the
operand of dq~ = tau dS k~ and dk~ = tau dS^T q~, p as the operand of
dv = p^T dO, and the forward's output o inside D = <dO, o>. Each such rounding
errs by at most U = 2^-8 relative, with a standard deviation of at most
U / sqrt(3); independent errors add in quadrature. The noise scale n of an
output element is therefore the root-sum-square of the terms whose rounding it
inherits (E_i = sum_d (dO_id o_id)^2 carries the rounding of o into D):

  n_dq~_id^2 = tau^2 [ sum_j dS_ij^2 k~_jd^2 + E_i (sum_j p_ij k~_jd)^2 ]
  n_dk~_jd^2 = tau^2 sum_i [ dS_ij^2 q~_id^2 + p_ij^2 E_i q~_id^2 ]
  n_dv_jd^2  = sum_i p_ij^2 dO_id^2
  n_dsigma_h^2 = sum_i exp(sigma_h - lse_i)^2 E_i,   m_dsigma_h = sum_i |exp(sigma_h - lse_i) D_i|

dq and dk are rotated back with R^T, so their squares combine with cos^2 and
sin^2. An element passes when

  |gpu - oracle| <= 4 U n + 2 U |oracle| + 1e-6

(dsigma: 2 U m_dsigma in place of 2 U |oracle|). 4 U n is about seven standard
deviations of the accumulated rounding noise; 2 U |oracle| covers the rounding of
the result itself (U) and the forward's log-sum-exp, whose row sum adds
bf16-rounded p (U). tests/test_backward_tolerance.py shows on the CPU that a
bf16 emulation of a correct kernel passes this bound and that plausible kernel
mistakes (a dropped term, a shifted key tile, a missing scale, a wrong rotation
sign, the sink left out of the normaliser, a window one key wider) fail it.
"""

import numpy as np

import oracle
from helpers import say

U = 2.0 ** -8


def _visible(q_pos, k_pos, window):
    vis = k_pos[None, :] <= q_pos[:, None]
    if window > 0:
        vis &= (q_pos[:, None] - k_pos[None, :]) < window
    return vis


def sequence_noise2(q, k, v, sinks, tau, q_pos, k_pos, window, dout):
    """Squared noise scales of one sequence, q [Tq,Hq,D] and k [Tk,Hkv,D] already rotated.

    Returns dict dq [Tq,Hq,D], dk / dv [Tk,Hkv,D], dsinks [Hq] (squares) and m_dsinks [Hq]."""
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    sinks = np.asarray(sinks, dtype=np.float64)
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    vis = _visible(np.asarray(q_pos, dtype=np.int64), np.asarray(k_pos, dtype=np.int64), window)
    out = {"dq": np.zeros(q.shape), "dk": np.zeros(k.shape), "dv": np.zeros(v.shape),
           "dsinks": np.zeros(Hq), "m_dsinks": np.zeros(Hq)}
    for h in range(Hq):
        g = h // G
        Q, K, V, dO = q[:, h], k[:, g], v[:, g], dout[:, h]
        s = np.where(vis, tau * (Q @ K.T), -np.inf)
        m = np.maximum(sinks[h], s.max(axis=1, initial=-np.inf))
        live = np.isfinite(m)
        mz = np.where(live, m, 0.0)
        lse = mz + np.log(np.exp(sinks[h] - mz) + np.exp(s - mz[:, None]).sum(axis=1))
        p = np.where(live[:, None], np.exp(s - np.where(live, lse, 0.0)[:, None]), 0.0)
        o = p @ V
        D = (dO * o).sum(axis=1)
        dS = p * (dO @ V.T - D[:, None])
        E = ((dO * o) ** 2).sum(axis=1)
        psink = np.where(live, np.exp(sinks[h] - np.where(live, lse, 0.0)), 0.0)
        out["dq"][:, h] = tau ** 2 * ((dS ** 2) @ (K ** 2) + E[:, None] * (p @ K) ** 2)
        out["dk"][:, g] += tau ** 2 * ((dS ** 2).T @ (Q ** 2) + (p ** 2).T @ (E[:, None] * Q ** 2))
        out["dv"][:, g] += (p ** 2).T @ (dO ** 2)
        out["dsinks"][h] = (psink ** 2 * E).sum()
        out["m_dsinks"][h] = np.abs(psink * D).sum()
    return out


def rotate_noise2(n2, cos, sin):
    """Squared noise through R^T: the squares combine with cos^2 and sin^2."""
    half = cos.shape[-1]
    a, b = n2[..., :half], n2[..., half:2 * half]
    c2, s2 = cos ** 2, sin ** 2
    return np.concatenate([c2 * a + s2 * b, c2 * b + s2 * a, n2[..., 2 * half:]], axis=-1)


def _finish(n2, rot):
    out = {}
    for name in ("dq", "dk"):
        out[name] = np.sqrt(rotate_noise2(n2[name], *rot) if rot is not None else n2[name])
    out["dv"] = np.sqrt(n2["dv"])
    out["dsinks"] = np.sqrt(n2["dsinks"])
    out["m_dsinks"] = n2["m_dsinks"]
    return out


def noise_bshd(q, k, v, sinks, tau, window, dout, cfg=oracle.RopeConfig(), rotate_qk=True):
    """Noise scales of the BSHD backward (arguments as oracle.prefill_bshd_backward)."""
    B, S = q.shape[:2]
    qr, kr = oracle.rope_qk_bshd(q, k, cfg) if rotate_qk else (np.asarray(q, float), np.asarray(k, float))
    pos = np.arange(S)
    parts = [sequence_noise2(qr[b], kr[b], v[b], sinks, tau, pos, pos, window, dout[b]) for b in range(B)]
    n2 = {n: np.stack([p[n] for p in parts]) for n in ("dq", "dk", "dv")}
    n2["dsinks"] = sum(p["dsinks"] for p in parts)
    n2["m_dsinks"] = sum(p["m_dsinks"] for p in parts)
    rot = None
    if rotate_qk:
        cos, sin = oracle.cos_sin_table(cfg, pos)
        rot = (cos[None, :, None, :], sin[None, :, None, :])
    return _finish(n2, rot)


def noise_thd(q, k, v, cu_seqlens, sinks, tau, window, dout, cfg=oracle.RopeConfig(), rotate_qk=True):
    """Noise scales of the packed THD backward (arguments as oracle.prefill_thd_backward)."""
    T = q.shape[0]
    qr, kr = oracle.rope_qk_thd(q, k, cu_seqlens, cfg) if rotate_qk else (np.asarray(q, float),
                                                                           np.asarray(k, float))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n2 = {"dq": np.zeros(q.shape), "dk": np.zeros(k.shape), "dv": np.zeros(v.shape),
          "dsinks": np.zeros(q.shape[1]), "m_dsinks": np.zeros(q.shape[1])}
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b <= a:
            continue
        pos = np.arange(b - a)
        part = sequence_noise2(qr[a:b], kr[a:b], v[a:b], sinks, tau, pos, pos, window, dout[a:b])
        for name in ("dq", "dk", "dv"):
            n2[name][a:b] = part[name]
        n2["dsinks"] += part["dsinks"]
        n2["m_dsinks"] += part["m_dsinks"]
    rot = None
    if rotate_qk:
        cos, sin = oracle.cos_sin_table(cfg, oracle.thd_positions(cu, T))
        rot = (cos[:, None, :], sin[:, None, :])
    return _finish(n2, rot)


def noise_rows(q, k, v, sinks, tau, window, dout, q_rows, key_lo, key_hi, cfg=oracle.RopeConfig()):
    """Noise scales of dq at q_rows and of dk, dv at keys key_lo .. key_hi - 1 of one sequence
    (the sub-problems of oracle.prefill_backward_rows, which leave nothing out that they depend on)."""
    q_rows = np.asarray(q_rows, dtype=np.int64)
    S = q.shape[0]
    klo = 0 if window <= 0 else max(0, int(q_rows.min()) - window + 1)
    kr = np.arange(klo, int(q_rows.max()) + 1)
    cq, sq = oracle.cos_sin_table(cfg, q_rows)
    ck, sk = oracle.cos_sin_table(cfg, kr)
    part = sequence_noise2(oracle.rotate(q[q_rows], cq[:, None, :], sq[:, None, :]),
                           oracle.rotate(k[kr], ck[:, None, :], sk[:, None, :]), v[kr], sinks, tau, q_rows, kr,
                           window, dout[q_rows])
    out = {"dq": np.sqrt(rotate_noise2(part["dq"], cq[:, None, :], sq[:, None, :]))}
    q_hi = S - 1 if window <= 0 else min(S - 1, key_hi - 1 + window - 1)
    qr = np.arange(key_lo, q_hi + 1)
    klo = 0 if window <= 0 else max(0, key_lo - window + 1)
    kr = np.arange(klo, q_hi + 1)
    cq, sq = oracle.cos_sin_table(cfg, qr)
    ck, sk = oracle.cos_sin_table(cfg, kr)
    part = sequence_noise2(oracle.rotate(q[qr], cq[:, None, :], sq[:, None, :]),
                           oracle.rotate(k[kr], ck[:, None, :], sk[:, None, :]), v[kr], sinks, tau, qr, kr,
                           window, dout[qr])
    sel = slice(key_lo - klo, key_hi - klo)
    ck, sk = ck[sel], sk[sel]
    out["dk"] = np.sqrt(rotate_noise2(part["dk"][sel], ck[:, None, :], sk[:, None, :]))
    out["dv"] = np.sqrt(part["dv"][sel])
    return out


def grad_ratio(got, ref, noise, mag=None):
    """Worst |got - ref| / (4 U n + 2 U |ref| + 1e-6) over the elements (<= 1 passes)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    bound = 4 * U * noise + 2 * U * (np.abs(r) if mag is None else mag) + 1e-6
    err = np.abs(g - r)
    return float((err / bound).max()) if err.size else 0.0


def grad_close(got, ref, noise, what, mag=None):
    """grad_ratio with a log line: max-abs, relative L2 and, as a diagnostic beside the
    bound, the worst ratio under the forward's elementwise bound 1e-2 + 2e-2 |ref|."""
    import torch
    g = got.detach().to("cpu").double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    err = np.abs(g - r)
    ratio = grad_ratio(g, r, noise, mag)
    fwd = float((err / (1e-2 + 2e-2 * np.abs(r))).max()) if err.size else 0.0
    rel_l2 = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    say(f"  {what}: max_abs={float(err.max()) if err.size else 0:.3e} rel_l2={rel_l2:.3e} "
        f"worst_ratio={ratio:.3f} (forward bound 1e-2 + 2e-2|r|: {fwd:.3f})")
    if ratio > 1.0:
        bound = 4 * U * noise + 2 * U * (np.abs(r) if mag is None else mag) + 1e-6
        w = np.unravel_index(np.argmax(err / bound), err.shape)
        say(f"    worst at {tuple(int(i) for i in w)}: gpu={g[w]:.5f} ref={r[w]:.5f} noise={noise[w]:.3e}; "
            f"{int((err > bound).sum())} of {err.size} elements out of tolerance")
    return ratio
