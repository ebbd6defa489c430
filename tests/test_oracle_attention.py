"""Pins for the oracle's sink + GQA + sliding-window attention.

Each pin comes from outside the oracle's own code:
  * sink = -inf reduces to standard causal attention: torch's
    scaled_dot_product_attention in fp64 (a library routine), with K/V
    repeat-interleaved so each query head h reads KV head h // 8;
  * the sink is an extra logit with a zero value vector: torch.softmax over
    [sigma, masked scores] then a matmul (library routines), with masks built
    from the window definition;
  * a window at least as long as the sequence equals full causal;
  * with v == 1 the output is the probability row sum, which equals
    Z / (Z + e^sigma) < 1 (Z from torch.logsumexp of the visible scores);
  * a window of 1 has the closed form v_i / (1 + e^(sigma - s_ii));
  * pure-Python loops with math.exp on tiny shapes;
  * GQA equals MHA with repeat-interleaved K/V; packed THD equals per-sequence
    BSHD; decode equals the last prefill row; permuting keys changes nothing.
"""

import math

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
    return q, k, v, sinks


def _mask(S, window):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = j <= i
    if window > 0:
        m &= (i - j) < window
    return torch.from_numpy(m)


def test_sink_minus_inf_is_sdpa_causal():
    B, S, hq, hkv, d = 2, 77, 16, 2, 64
    q, k, v, _ = _inputs(B, S, hq, hkv, d, 0)
    sinks = np.full(hq, -np.inf)
    got = oracle.prefill_bshd(q, k, v, sinks, TAU, 0, rotate_qk=False)
    G = hq // hkv
    Q = torch.from_numpy(q).permute(0, 2, 1, 3)
    K = torch.from_numpy(k).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    V = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    ref = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=TAU).permute(0, 2, 1, 3)
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("window", [0, 1, 5, 33, 200])
def test_sink_is_an_extra_logit(window):
    B, S, hq, hkv, d = 1, 90, 8, 2, 64
    q, k, v, sinks = _inputs(B, S, hq, hkv, d, 1, sink_scale=2.0)
    got = oracle.prefill_bshd(q, k, v, sinks, TAU, window, rotate_qk=False)[0]
    G = hq // hkv
    Q = torch.from_numpy(q[0]).permute(1, 0, 2)                                    # [H,S,D]
    K = torch.from_numpy(k[0]).repeat_interleave(G, dim=1).permute(1, 0, 2)
    V = torch.from_numpy(v[0]).repeat_interleave(G, dim=1).permute(1, 0, 2)
    s = TAU * torch.matmul(Q, K.transpose(1, 2))
    s = s.masked_fill(~_mask(S, window)[None], float("-inf"))
    sig = torch.from_numpy(sinks)[:, None, None].expand(hq, S, 1)
    p = torch.softmax(torch.cat([sig, s], dim=-1), dim=-1)[..., 1:]
    ref = torch.matmul(p, V).permute(1, 0, 2).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_window_at_least_length_is_full_causal():
    q, k, v, sinks = _inputs(2, 50, 8, 2, 64, 2)
    full = oracle.prefill_bshd(q, k, v, sinks, TAU, 0, CFG)
    for w in (50, 51, 128):
        assert np.array_equal(oracle.prefill_bshd(q, k, v, sinks, TAU, w, CFG), full)
    assert not np.allclose(oracle.prefill_bshd(q, k, v, sinks, TAU, 49, CFG), full)


@pytest.mark.parametrize("window", [0, 16])
def test_row_sums_fall_below_one(window):
    S, hq, hkv = 60, 8, 2
    q, k, v, sinks = _inputs(1, S, hq, hkv, 64, 3)
    ones = np.ones_like(v)
    got = oracle.prefill_bshd(q, k, ones, sinks, TAU, window, rotate_qk=False)[0]  # [S,H,D]
    G = hq // hkv
    Q = torch.from_numpy(q[0]).permute(1, 0, 2)
    K = torch.from_numpy(k[0]).repeat_interleave(G, dim=1).permute(1, 0, 2)
    s = (TAU * torch.matmul(Q, K.transpose(1, 2))).masked_fill(~_mask(S, window)[None], float("-inf"))
    lse = torch.logsumexp(s, dim=-1).numpy().T                                       # [S,H]
    expect = 1.0 / (1.0 + np.exp(sinks[None, :] - lse))
    assert np.allclose(got[..., 0], expect, rtol=1e-12)
    assert np.all(got < 1.0) and np.all(got > 0.0)
    no_sink = oracle.prefill_bshd(q, k, ones, np.full(hq, -np.inf), TAU, window, rotate_qk=False)
    assert np.allclose(no_sink, 1.0, rtol=1e-14)


def test_window_one_closed_form():
    q, k, v, sinks = _inputs(1, 40, 8, 4, 64, 4, sink_scale=3.0)
    got = oracle.prefill_bshd(q, k, v, sinks, TAU, 1, rotate_qk=False)[0]
    G = 2
    for i in range(40):
        for h in range(8):
            s_ii = TAU * float(q[0, i, h] @ k[0, i, h // G])
            w = 1.0 / (1.0 + math.exp(sinks[h] - s_ii))
            assert np.allclose(got[i, h], w * v[0, i, h // G], rtol=1e-12, atol=1e-14)


def _brute(q, k, v, sinks, window):
    """Pure-Python loops over one BSHD sequence: q [S,Hq,D], k/v [S,Hkv,D]."""
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(S)]
    for i in range(S):
        for h in range(Hq):
            g = h // G
            vis = [j for j in range(S) if j <= i and (window == 0 or i - j < window)]
            sc = {}
            for j in vis:
                acc = 0.0
                for x in range(D):
                    acc += float(q[i, h, x]) * float(k[j, g, x])
                sc[j] = TAU * acc
            sig = float(sinks[h])
            m = max([sig] + list(sc.values()))
            if m == -math.inf:
                continue
            z = math.exp(sig - m) + sum(math.exp(sc[j] - m) for j in vis)
            for x in range(D):
                out[i][h][x] = sum(math.exp(sc[j] - m) * float(v[j, g, x]) for j in vis) / z
    return np.array(out)


@pytest.mark.parametrize("S", [1, 2, 6])
@pytest.mark.parametrize("window", [0, 1, 2, 7])
@pytest.mark.parametrize("sink", [-math.inf, 0.0, 3.0])
def test_brute_force_tiny(S, window, sink):
    q, k, v, _ = _inputs(1, S, 4, 2, 64, 10 + S)
    sinks = np.full(4, sink)
    sinks[1] = sink if sink == -math.inf else -sink
    qr, kr = oracle.rope_qk_bshd(q, k, CFG)
    got = oracle.prefill_bshd(q, k, v, sinks, TAU, window, CFG)[0]
    ref = _brute(qr[0], kr[0], v[0], sinks, window)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v, sinks = _inputs(1, 70, 16, 2, 64, 5)
    got = oracle.prefill_bshd(q, k, v, sinks, TAU, 20, rotate_qk=False)
    kk = np.repeat(k, 8, axis=2)
    vv = np.repeat(v, 8, axis=2)
    ref = oracle.prefill_bshd(q, kk, vv, sinks, TAU, 20, rotate_qk=False)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("window", [0, 8])
def test_thd_equals_per_sequence_bshd(window):
    lengths = [13, 0, 1, 40, 7]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    q, k, v, sinks = _inputs(1, T, 8, 2, 64, 6)
    got = oracle.prefill_thd(q[0], k[0], v[0], cu, sinks, TAU, window, CFG)
    for n, L in enumerate(lengths):
        if L == 0:
            continue
        a, b = cu[n], cu[n + 1]
        ref = oracle.prefill_bshd(q[:, a:b], k[:, a:b], v[:, a:b], sinks, TAU, window, CFG)[0]
        assert np.array_equal(got[a:b], ref)


@pytest.mark.parametrize("window", [0, 5])
def test_decode_equals_last_prefill_row(window):
    S = 33
    q, k, v, sinks = _inputs(2, S, 8, 2, 64, 7)
    lens = [S, 20]
    qr, kr = oracle.rope_qk_bshd(q, k, CFG)
    kc = np.zeros((2, 40, 2, 64))
    vc = np.zeros((2, 40, 2, 64))
    qd = np.zeros((2, 8, 64))
    for n, L in enumerate(lens):
        kc[n, :L] = kr[n, :L]
        vc[n, :L] = v[n, :L]
        qd[n] = q[n, L - 1]
    got = oracle.decode(qd, kc, vc, lens, sinks, TAU, window, CFG)
    for n, L in enumerate(lens):
        ref = oracle.prefill_bshd(q[n:n + 1, :L], k[n:n + 1, :L], v[n:n + 1, :L], sinks, TAU, window, CFG)
        assert np.allclose(got[n], ref[0, L - 1], rtol=1e-13, atol=1e-15)


def test_key_permutation_invariance():
    S = 50
    q, k, v, sinks = _inputs(1, S, 8, 2, 64, 8)
    pos = np.arange(S)
    ref = oracle.sink_attention(q[0], k[0], v[0], sinks, TAU, pos, pos, 9)
    perm = np.random.default_rng(1).permutation(S)
    got = oracle.sink_attention(q[0], k[0][perm], v[0][perm], sinks, TAU, pos, pos[perm], 9)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("window", [0, 16])
def test_prefill_rows_match_full_prefill(window):
    S = 90
    q, k, v, sinks = _inputs(1, S, 8, 2, 64, 9)
    ref = oracle.prefill_bshd(q, k, v, sinks, TAU, window, CFG)[0]
    rows = np.array([0, 1, 15, 16, 17, 60, 89])
    got = oracle.prefill_rows(q[0], k[0], v[0], sinks, TAU, window, rows, CFG)
    assert np.allclose(got, ref[rows], rtol=1e-13, atol=1e-15)
