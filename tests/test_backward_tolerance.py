"""CPU checks of the backward tolerance (tests/backward_tolerance.py).

The bound the GPU backward tests apply is derived from the bf16 roundings a
correct kernel makes. These tests pin it from both sides, on the CPU:
  * its noise scales equal their closed forms for a single key, and the
    sub-problem form used at full size equals the whole problem;
  * a bf16 emulation of a correct kernel (p and dS rounded to bf16 as matrix
    operands, D from the bf16 forward output, results rounded to bf16) passes;
  * plausible kernel mistakes each fail it: the -D term dropped for one 64-key
    tile, one key tile read one row off, tau missing on dk, the rotation back
    applied with the wrong sign (R instead of R^T), the sink left out of the
    softmax normaliser, and (window layers) a window one key wider.
Inputs are N(0, 1) bf16 like the benchmark's, 256 positions (four 64-key tiles),
16 query heads over 2 KV heads, full-causal and window-128.
"""

import numpy as np
import pytest
import torch

import backward_tolerance as bt
import oracle

pytestmark = []
TAU = 0.125
CFG = oracle.RopeConfig()


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def _inputs(S, hq, hkv, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((1, S, hq, 64), generator=g).to(torch.bfloat16).double().numpy()
    k = torch.randn((1, S, hkv, 64), generator=g).to(torch.bfloat16).double().numpy()
    v = torch.randn((1, S, hkv, 64), generator=g).to(torch.bfloat16).double().numpy()
    sinks = torch.randn(hq, generator=g).double().numpy()
    dout = torch.randn((1, S, hq, 64), generator=g).to(torch.bfloat16).double().numpy()
    return q, k, v, sinks, dout


def kernel_model(q, k, v, sinks, window, dout, mistake=None):
    """The backward as a bf16 / fp32 kernel forms it (fp64 sums stand in for fp32 ones), with an
    optional planted mistake. q, k un-rotated [1,S,H,64]. Returns dq, dk, dv (bf16-rounded), dsinks."""
    S, hq, hkv = q.shape[1], q.shape[2], k.shape[2]
    G = hq // hkv
    qr, kr = oracle.rope_qk_bshd(q, k, CFG)
    qr, kr = qr[0], kr[0]
    pos = np.arange(S)
    vis = pos[None, :] <= pos[:, None]
    if window > 0:
        wv = window + 1 if mistake == "window_one_wider" else window
        vis &= (pos[:, None] - pos[None, :]) < wv
    dq = np.zeros((S, hq, 64))
    dk = np.zeros((S, hkv, 64))
    dv = np.zeros((S, hkv, 64))
    dsinks = np.zeros(hq)
    tile = slice(64, 128)
    for h in range(hq):
        g = h // G
        Q, K, V, dO = qr[:, h], kr[:, g], v[0, :, g], dout[0, :, h]
        s = np.where(vis, TAU * (Q @ K.T), -np.inf)
        sig = -np.inf if mistake == "sink_not_in_normaliser" else sinks[h]
        m = np.maximum(sig, s.max(axis=1))
        lse = m + np.log(np.exp(sig - m) + np.exp(s - m[:, None]).sum(axis=1))
        p = np.exp(s - lse[:, None])
        o = _bf16(p @ V)                               # the forward's bf16 output
        D = (dO * o).sum(axis=1)
        dP = dO @ V.T
        ds_full = p * (dP - D[:, None])
        if mistake == "no_minus_d_one_tile":
            ds_full[:, tile] = p[:, tile] * dP[:, tile]
        dS = _bf16(ds_full)                            # bf16 matrix-core operand
        Kq = K.copy()
        if mistake == "key_tile_off_by_one":
            Kq[128:192] = K[129:193]
        dq[:, h] = TAU * (dS @ Kq)
        dk[:, g] += (1.0 if mistake == "no_tau_on_dk" else TAU) * (dS.T @ Q)
        dv[:, g] += _bf16(p).T @ dO
        dsinks[h] = -(np.exp(sinks[h] - lse) * D).sum()
    cos, sin = oracle.cos_sin_table(CFG, pos)
    c, sn = cos[:, None, :], sin[:, None, :]
    if mistake == "rotation_back_with_r":
        back = lambda y: oracle.rotate(y, c, sn, round_output=False)   # noqa: E731
    else:
        back = lambda y: oracle.rotate_transpose(y, c, sn)             # noqa: E731
    return _bf16(back(dq))[None], _bf16(back(dk))[None], _bf16(dv)[None], dsinks


MISTAKES = ["no_minus_d_one_tile", "key_tile_off_by_one", "no_tau_on_dk", "rotation_back_with_r",
            "sink_not_in_normaliser", "window_one_wider"]


@pytest.fixture(scope="module", params=[0, 128])
def problem(request):
    window = request.param
    q, k, v, sinks, dout = _inputs(256, 16, 2, 900 + window)
    ref = oracle.prefill_bshd_backward(q, k, v, sinks, TAU, window, dout, CFG)
    noise = bt.noise_bshd(q, k, v, sinks, TAU, window, dout, CFG)
    return window, (q, k, v, sinks, dout), ref, noise


def _ratios(got, ref, noise):
    dq, dk, dv, ds = got
    return {"dq": bt.grad_ratio(dq, ref["dq"], noise["dq"]), "dk": bt.grad_ratio(dk, ref["dk"], noise["dk"]),
            "dv": bt.grad_ratio(dv, ref["dv"], noise["dv"]),
            "dsinks": bt.grad_ratio(ds, ref["dsinks"], noise["dsinks"], mag=noise["m_dsinks"])}


def test_correct_kernel_model_passes(problem):
    window, (q, k, v, sinks, dout), ref, noise = problem
    r = _ratios(kernel_model(q, k, v, sinks, window, dout), ref, noise)
    print(f"W={window} correct: {r}")
    assert max(r.values()) <= 1.0, r
    # and it is not loose: the worst element uses a fair share of the bound
    assert max(r.values()) > 0.05, r


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_mistake_fails(problem, mistake):
    window, (q, k, v, sinks, dout), ref, noise = problem
    if mistake == "window_one_wider" and window == 0:
        pytest.skip("a full-causal layer has no window")
    r = _ratios(kernel_model(q, k, v, sinks, window, dout, mistake), ref, noise)
    print(f"W={window} {mistake}: {r}")
    assert max(r.values()) > 1.0, f"{mistake} passes the bound: {r}"


def test_noise_scales_single_key_closed_form():
    """Noise scales for one key: p = e^s / (e^sigma + e^s), o = p v, dS = p (1 - p) <dO, v>,
    E = sum_d (dO_d o_d)^2; n_dv^2 = sum_h p_h^2 dO_h^2; n_dq~^2 = tau^2 (dS^2 k^2 + E p^2 k^2);
    n_dsigma^2 = (1 - p)^2 E; m_dsigma = |(1 - p) p <dO, v>|."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 8, 64))
    k = rng.standard_normal((1, 1, 1, 64))
    v = rng.standard_normal((1, 1, 1, 64))
    dout = rng.standard_normal((1, 1, 8, 64))
    sinks = rng.standard_normal(8)
    n = bt.noise_bshd(q, k, v, sinks, TAU, 0, dout, rotate_qk=False)
    pv = np.zeros(8)
    for h in range(8):
        s = TAU * float(q[0, 0, h] @ k[0, 0, 0])
        p = np.exp(s) / (np.exp(sinks[h]) + np.exp(s))
        pv[h] = p
        dvd = float(dout[0, 0, h] @ v[0, 0, 0])
        E = float(((dout[0, 0, h] * p * v[0, 0, 0]) ** 2).sum())
        ds = p * (1 - p) * dvd
        kk = k[0, 0, 0]
        assert np.allclose(n["dq"][0, 0, h], TAU * np.sqrt(ds ** 2 * kk ** 2 + E * p ** 2 * kk ** 2), rtol=1e-11)
        assert np.isclose(n["dsinks"][h], (1 - p) * np.sqrt(E), rtol=1e-11)
        assert np.isclose(n["m_dsinks"][h], abs((1 - p) * p * dvd), rtol=1e-11)
    assert np.allclose(n["dv"][0, 0, 0], np.sqrt((pv[:, None] ** 2 * dout[0, 0] ** 2).sum(0)), rtol=1e-11)


@pytest.mark.parametrize("window", [0, 6])
def test_rows_noise_equals_the_whole_problem(window):
    """noise_rows (selected query rows and a key range, sub-problems only) equals the
    matching entries of the whole problem's noise."""
    rng = np.random.default_rng(51 + window)
    S, hq, hkv = 40, 16, 2
    r = lambda *s: oracle.round_bf16(rng.standard_normal(s))   # noqa: E731
    q, k, v, dout = r(1, S, hq, 64), r(1, S, hkv, 64), r(1, S, hkv, 64), r(1, S, hq, 64)
    sinks = rng.standard_normal(hq)
    full = bt.noise_bshd(q, k, v, sinks, TAU, window, dout, CFG)
    rows = [0, 3, 17, 39]
    part = bt.noise_rows(q[0], k[0], v[0], sinks, TAU, window, dout[0], rows, 20, 31, CFG)
    assert np.allclose(part["dq"], full["dq"][0, rows], rtol=1e-12)
    assert np.allclose(part["dk"], full["dk"][0, 20:31], rtol=1e-12)
    assert np.allclose(part["dv"], full["dv"][0, 20:31], rtol=1e-12)
