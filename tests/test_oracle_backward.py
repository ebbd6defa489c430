"""Pins for the oracle's attention gradients and log-sum-exp (oracle.backward).

Each pin comes from outside oracle.backward:
  * central finite differences of the forward oracle (oracle.attention, a separate
    code path) along random directions, with the rotation unrounded so the
    forward is smooth: checks dq and dk (rotated back with R^T), dv and dsinks;
  * torch autograd (float64) of a forward written here with torch ops, the sink as
    an extra logit column with a zero value row;
  * with sinks = -inf, torch's scaled_dot_product_attention backward (library);
  * lse against torch.logsumexp over [sigma, visible scores];
  * closed forms for a single key;
  * THD equals per-sequence BSHD; the gradients of GQA sum over the group.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

CFG = oracle.RopeConfig()
TAU = 0.125


def _inputs(B, S, hq, hkv, d, seed, sink_scale=1.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, S, hq, d), generator=g).to(torch.bfloat16).double().numpy()
    k = torch.randn((B, S, hkv, d), generator=g).to(torch.bfloat16).double().numpy()
    v = torch.randn((B, S, hkv, d), generator=g).to(torch.bfloat16).double().numpy()
    sinks = (torch.randn(hq, generator=g) * sink_scale).double().numpy()
    dout = torch.randn((B, S, hq, d), generator=g).to(torch.bfloat16).double().numpy()
    return q, k, v, sinks, dout


def _loss(q, k, v, sinks, dout, window):
    """L = <dout, o> with the unrounded rotation (a smooth function of q, k, v, sinks)."""
    qr, kr = oracle.rope_qk_bshd(q, k, CFG, round_output=False)
    o = oracle.prefill_bshd(qr, kr, v, sinks, TAU, window, rotate_qk=False)
    return float((dout * o).sum())


@pytest.mark.parametrize("window", [0, 3])
def test_finite_differences(window):
    B, S, hq, hkv, d = 1, 7, 16, 2, 64
    q, k, v, sinks, dout = _inputs(B, S, hq, hkv, d, 11 + window)
    g = oracle.prefill_bshd_backward(q, k, v, sinks, TAU, window, dout, CFG, round_rotation=False)
    rng = np.random.default_rng(5)
    h = 1e-5
    for name, x in (("q", q), ("k", k), ("v", v), ("sinks", sinks)):
        e = rng.standard_normal(x.shape)
        args = {"q": q, "k": k, "v": v, "sinks": sinks}
        args[name] = x + h * e
        lp = _loss(args["q"], args["k"], args["v"], args["sinks"], dout, window)
        args[name] = x - h * e
        lm = _loss(args["q"], args["k"], args["v"], args["sinks"], dout, window)
        fd = (lp - lm) / (2 * h)
        an = float((g["d" + name] * e).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), f"d{name}: finite difference {fd} vs analytic {an}"


def _torch_forward(q, k, v, sinks, window):
    """Independent torch forward for one batch: q [S,Hq,D], k/v [S,Hkv,D] (rotated), sinks [Hq]."""
    S, hq, d = q.shape
    G = hq // k.shape[1]
    K = k.repeat_interleave(G, dim=1)
    V = v.repeat_interleave(G, dim=1)
    s = TAU * torch.einsum("ihd,jhd->hij", q, K)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    m = j <= i
    if window > 0:
        m = m & ((i - j) < window)
    s = s.masked_fill(~m[None], float("-inf"))
    logits = torch.cat([sinks[:, None, None].expand(hq, S, 1), s], dim=-1)
    p = torch.softmax(logits, dim=-1)[..., 1:]
    return torch.einsum("hij,jhd->ihd", p, V), torch.logsumexp(logits, dim=-1).T


@pytest.mark.parametrize("window", [0, 5])
def test_torch_autograd(window):
    B, S, hq, hkv, d = 2, 19, 16, 2, 64
    q, k, v, sinks, dout = _inputs(B, S, hq, hkv, d, 21 + window, sink_scale=2.0)
    g = oracle.prefill_bshd_backward(q, k, v, sinks, TAU, window, dout, rotate_qk=False)
    ds = torch.zeros(hq, dtype=torch.float64)
    for b in range(B):
        Q = torch.tensor(q[b], requires_grad=True)
        K = torch.tensor(k[b], requires_grad=True)
        V = torch.tensor(v[b], requires_grad=True)
        sg = torch.tensor(sinks, requires_grad=True)
        o, lse = _torch_forward(Q, K, V, sg, window)
        (o * torch.tensor(dout[b])).sum().backward()
        assert np.allclose(g["o"][b], o.detach().numpy(), rtol=1e-12, atol=1e-13)
        assert np.allclose(g["lse"][b], lse.detach().numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(g["dq"][b], Q.grad.numpy(), rtol=1e-10, atol=1e-12)
        assert np.allclose(g["dk"][b], K.grad.numpy(), rtol=1e-10, atol=1e-12)
        assert np.allclose(g["dv"][b], V.grad.numpy(), rtol=1e-10, atol=1e-12)
        ds += sg.grad
    assert np.allclose(g["dsinks"], ds.numpy(), rtol=1e-10, atol=1e-12)


def test_no_sink_is_sdpa_backward():
    B, S, hq, hkv, d = 1, 33, 16, 2, 64
    q, k, v, _, dout = _inputs(B, S, hq, hkv, d, 31)
    sinks = np.full(hq, -np.inf)
    g = oracle.prefill_bshd_backward(q, k, v, sinks, TAU, 0, dout, rotate_qk=False)
    G = hq // hkv
    Q = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_()
    K = torch.tensor(k).permute(0, 2, 1, 3).requires_grad_()
    V = torch.tensor(v).permute(0, 2, 1, 3).requires_grad_()
    o = F.scaled_dot_product_attention(Q, K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1),
                                       is_causal=True, scale=TAU)
    (o * torch.tensor(dout).permute(0, 2, 1, 3)).sum().backward()
    assert np.allclose(g["dq"], Q.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(g["dk"], K.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(g["dv"], V.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)
    assert np.all(g["dsinks"] == 0.0)


def test_single_key_closed_form():
    """Position 0 sees only itself: p = e^s / (e^sigma + e^s); o = p v; dv = p dO;
    dq~ = tau p (1 - p) <dO, v> k~; dsigma = -(1 - p) p <dO, v>; lse = log(e^sigma + e^s)."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 8, 64))
    k = rng.standard_normal((1, 1, 1, 64))
    v = rng.standard_normal((1, 1, 1, 64))
    dout = rng.standard_normal((1, 1, 8, 64))
    sinks = rng.standard_normal(8)
    g = oracle.prefill_bshd_backward(q, k, v, sinks, TAU, 0, dout, rotate_qk=False)
    for h in range(8):
        s = TAU * float(q[0, 0, h] @ k[0, 0, 0])
        p = np.exp(s) / (np.exp(sinks[h]) + np.exp(s))
        dv_dot = float(dout[0, 0, h] @ v[0, 0, 0])
        assert np.isclose(g["lse"][0, 0, h], np.log(np.exp(sinks[h]) + np.exp(s)), rtol=1e-13)
        assert np.allclose(g["dq"][0, 0, h], TAU * p * (1 - p) * dv_dot * k[0, 0, 0], rtol=1e-11, atol=1e-14)
        assert np.isclose(g["dsinks"][h], -(1 - p) * p * dv_dot, rtol=1e-11, atol=1e-15)
    p_all = np.array([np.exp(TAU * q[0, 0, h] @ k[0, 0, 0]) / (np.exp(sinks[h]) + np.exp(TAU * q[0, 0, h] @ k[0, 0, 0]))
                      for h in range(8)])
    assert np.allclose(g["dv"][0, 0, 0], (p_all[:, None] * dout[0, 0]).sum(0), rtol=1e-12)


def test_dead_rows_have_no_gradient():
    """sigma = -inf on a window of 0 visible keys cannot happen (the query sees itself), so
    build it with a key at a later position only: the row has nothing visible."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 8, 64))
    k = rng.standard_normal((1, 1, 64))
    v = rng.standard_normal((1, 1, 64))
    dout = rng.standard_normal((1, 8, 64))
    sinks = np.full(8, -np.inf)
    o, lse, dq, dk, dv, ds = oracle.sink_attention_backward(q, k, v, sinks, TAU, [0], [5], 0, dout)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0) and np.all(ds == 0)


def test_thd_equals_per_sequence_bshd():
    lengths = [5, 0, 17, 1]
    T = sum(lengths)
    g = torch.Generator().manual_seed(41)
    q = torch.randn((T, 16, 64), generator=g).to(torch.bfloat16).double().numpy()
    k = torch.randn((T, 2, 64), generator=g).to(torch.bfloat16).double().numpy()
    v = torch.randn((T, 2, 64), generator=g).to(torch.bfloat16).double().numpy()
    dout = torch.randn((T, 16, 64), generator=g).to(torch.bfloat16).double().numpy()
    sinks = torch.randn(16, generator=g).double().numpy()
    cu = np.concatenate([[0], np.cumsum(lengths)])
    got = oracle.prefill_thd_backward(q, k, v, cu, sinks, TAU, 4, dout)
    ds = np.zeros(16)
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        if b == a:
            continue
        ref = oracle.prefill_bshd_backward(q[None, a:b], k[None, a:b], v[None, a:b], sinks, TAU, 4, dout[None, a:b])
        for name in ("o", "lse", "dq", "dk", "dv"):
            assert np.allclose(got[name][a:b], ref[name][0], rtol=1e-12, atol=1e-13), name
        ds += ref["dsinks"]
    assert np.allclose(got["dsinks"], ds, rtol=1e-12, atol=1e-13)


def test_rotate_transpose_is_the_adjoint():
    """<R x, y> = <x, R^T y> for the YaRN table's rows (and R^T R = I up to the table's rounding)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, 3, 64))
    y = rng.standard_normal((50, 3, 64))
    cos, sin = oracle.cos_sin_table(CFG, np.arange(1000, 1050))
    c, s = cos[:, None, :], sin[:, None, :]
    rx = oracle.rotate(x, c, s, round_output=False)
    rty = oracle.rotate_transpose(y, c, s)
    assert np.isclose((rx * y).sum(), (x * rty).sum(), rtol=1e-12)


@pytest.mark.parametrize("window", [0, 6])
def test_rows_equal_the_whole_problem(window):
    """prefill_backward_rows (selected query rows and a key range, sub-problems only)
    equals the matching entries of the full backward."""
    B, S, hq, hkv, d = 1, 40, 16, 2, 64
    q, k, v, sinks, dout = _inputs(B, S, hq, hkv, d, 51 + window)
    full = oracle.prefill_bshd_backward(q, k, v, sinks, TAU, window, dout, CFG)
    rows = [0, 3, 17, 39]
    part = oracle.prefill_backward_rows(q[0], k[0], v[0], sinks, TAU, window, dout[0], rows, 20, 31, CFG)
    assert np.allclose(part["dq"], full["dq"][0, rows], rtol=1e-12, atol=1e-13)
    assert np.allclose(part["dk"], full["dk"][0, 20:31], rtol=1e-12, atol=1e-13)
    assert np.allclose(part["dv"], full["dv"][0, 20:31], rtol=1e-12, atol=1e-13)
