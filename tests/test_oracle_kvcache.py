"""Pins of oracle.kvcache (append and decode over contiguous, paged and ring caches).

The cache oracle is tied to definitions pinned elsewhere: a cache built by
appending a sequence token by token must hold exactly the keys the prefill
rotation produces at those positions, and decoding the last token from any
layout must give the last row of the prefill definition (full causal, or the
window). Layout-specific checks: one bulk append equals token-by-token appends
(a ring keeps only the last positions), a permuted page pool changes nothing,
and a paged cache whose pages are laid out in order is the contiguous cache.
"""

import numpy as np
import pytest

import oracle
from oracle import kvcache as kv

CFG = oracle.RopeConfig()
TAU = 0.125


def _bf16_randn(rng, shape):
    return oracle.round_bf16(rng.standard_normal(shape))


def _seq(seed, N=2, S=37, hq=16, hkv=2):
    rng = np.random.default_rng(seed)
    q = _bf16_randn(rng, (N, S, hq, 64))
    k = _bf16_randn(rng, (N, S, hkv, 64))
    v = _bf16_randn(rng, (N, S, hkv, 64))
    sinks = rng.standard_normal(hq)
    return q, k, v, sinks


def _empty(layout, N, hkv, max_pages=0):
    if layout.kind == kv.PAGED:
        shape = (N * max_pages + 3, layout.capacity, hkv, 64)   # spare pages stay unused
    else:
        shape = (N, layout.capacity, hkv, 64)
    return np.full(shape, np.nan), np.full(shape, np.nan)


def _layouts(N, S, seed):
    rng = np.random.default_rng(seed)
    ps = 8
    max_pages = (S + ps - 1) // ps
    perm = rng.permutation(N * max_pages + 3)[: N * max_pages].reshape(N, max_pages)
    return {
        "contiguous": (kv.KVLayout(kv.CONTIGUOUS, S + 5), 0),
        "paged": (kv.KVLayout(kv.PAGED, ps, perm), max_pages),
        "ring": (kv.KVLayout(kv.RING, 16), 0),
    }


def _fill_token_by_token(layout, max_pages, k, v):
    N, S, hkv = k.shape[:3]
    kc, vc = _empty(layout, N, hkv, max_pages)
    for t in range(S):
        kc, vc = kv.append(layout, kc, vc, k[:, t:t + 1], v[:, t:t + 1], [t + 1] * N, CFG)
    return kc, vc


@pytest.mark.parametrize("name", ["contiguous", "paged", "ring"])
def test_appended_rows_are_the_prefill_rotation(name):
    q, k, v, _ = _seq(1)
    N, S = k.shape[:2]
    layout, mp = _layouts(N, S, 2)[name]
    kc, vc = _fill_token_by_token(layout, mp, k, v)
    _, kr = oracle.rope_qk_bshd(q, k, CFG)
    lo = S - layout.capacity if name == "ring" else 0
    for n in range(N):
        ks, vs = kv.logical_rows(layout, kc, vc, n, lo, S)
        assert np.array_equal(ks, kr[n, lo:S])
        assert np.array_equal(vs, v[n, lo:S])


@pytest.mark.parametrize("name", ["contiguous", "paged", "ring"])
@pytest.mark.parametrize("T", [1, 5, 20])
def test_bulk_append_equals_token_by_token(name, T):
    """num_new tokens in one call == the same tokens one call each (T = 20 exceeds the
    ring's 16 slots: only the last 16 positions survive either way)."""
    _, k, v, _ = _seq(3, S=30)
    N, S = k.shape[:2]
    layout, mp = _layouts(N, S, 4)[name]
    kc0, vc0 = _fill_token_by_token(layout, mp, k[:, : S - T], v[:, : S - T])
    kc1, vc1 = kv.append(layout, kc0, vc0, k[:, S - T:], v[:, S - T:], [S] * N, CFG)
    kc2, vc2 = kc0, vc0
    for t in range(S - T, S):
        kc2, vc2 = kv.append(layout, kc2, vc2, k[:, t:t + 1], v[:, t:t + 1], [t + 1] * N, CFG)
    assert np.array_equal(kc1, kc2, equal_nan=True) and np.array_equal(vc1, vc2, equal_nan=True)


@pytest.mark.parametrize("name,window", [("contiguous", 0), ("contiguous", 16), ("contiguous", 5),
                                         ("paged", 0), ("paged", 16), ("paged", 5), ("ring", 16)])
def test_decode_equals_last_prefill_row(name, window):
    """Decode of the token at S - 1 from a cache filled by appends == row S - 1 of prefill."""
    q, k, v, sinks = _seq(5)
    N, S = k.shape[:2]
    layout, mp = _layouts(N, S, 6)[name]
    kc, vc = _fill_token_by_token(layout, mp, k, v)
    ref = oracle.prefill_bshd(q, k, v, sinks, TAU, window, CFG)[:, S - 1]
    got = kv.decode(layout, q[:, S - 1], kc, vc, [S] * N, sinks, TAU, window, CFG)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_decode_shorter_sequences_and_sink():
    """Different lengths per sequence (one of length 1) and sinks = -inf: decode of each
    sequence equals the last prefill row of that sequence alone."""
    q, k, v, _ = _seq(7, N=3, S=20)
    lengths = [20, 1, 13]
    sinks = np.full(16, -np.inf)
    for name in ("contiguous", "paged", "ring"):
        layout, mp = _layouts(3, 20, 8)[name]
        window = 16 if name == "ring" else 0
        kc, vc = _empty(layout, 3, 2, mp)
        for n, L in enumerate(lengths):
            for t in range(L):
                one = [t + 1 if m == n else 0 for m in range(3)]
                kc, vc = kv.append(layout, kc, vc, k[:, t:t + 1], v[:, t:t + 1], one, CFG)
        got = kv.decode(layout, np.stack([q[n, L - 1] for n, L in enumerate(lengths)]), kc, vc, lengths, sinks,
                        TAU, window, CFG)
        for n, L in enumerate(lengths):
            ref = oracle.prefill_bshd(q[n:n + 1, :L], k[n:n + 1, :L], v[n:n + 1, :L], sinks, TAU, window, CFG)
            np.testing.assert_allclose(got[n], ref[0, L - 1], rtol=1e-12, atol=1e-12)


def test_paged_pool_permutation_changes_nothing():
    q, k, v, sinks = _seq(9)
    N, S = k.shape[:2]
    layout, mp = _layouts(N, S, 10)["paged"]
    kc, vc = _fill_token_by_token(layout, mp, k, v)
    a = kv.decode(layout, q[:, S - 1], kc, vc, [S] * N, sinks, TAU, 0, CFG)
    perm = np.random.default_rng(11).permutation(kc.shape[0])   # new physical page of each old page
    kp, vp = np.empty_like(kc), np.empty_like(vc)
    kp[perm], vp[perm] = kc, vc
    moved = kv.KVLayout(kv.PAGED, layout.capacity, perm[layout.block_table])
    b = kv.decode(moved, q[:, S - 1], kp, vp, [S] * N, sinks, TAU, 0, CFG)
    assert np.array_equal(a, b)


def test_in_order_pages_are_the_contiguous_cache():
    q, k, v, sinks = _seq(12, S=32)
    N, S = k.shape[:2]
    cont = kv.KVLayout(kv.CONTIGUOUS, S)
    kc, vc = _fill_token_by_token(cont, 0, k, v)
    ps = 8
    paged = kv.KVLayout(kv.PAGED, ps, np.arange(N * S // ps).reshape(N, S // ps))
    kp, vp = kc.reshape(N * S // ps, ps, 2, 64), vc.reshape(N * S // ps, ps, 2, 64)
    for w in (0, 7):
        a = kv.decode(cont, q[:, S - 1], kc, vc, [S] * N, sinks, TAU, w, CFG)
        b = kv.decode(paged, q[:, S - 1], kp, vp, [S] * N, sinks, TAU, w, CFG)
        assert np.array_equal(a, b)


def test_ring_and_contiguous_bounds():
    ring = kv.KVLayout(kv.RING, 4)
    assert kv.row_of(ring, 1, 9) == (1, 1)
    with pytest.raises(ValueError):
        kv.logical_rows(ring, np.zeros((2, 4, 1, 64)), np.zeros((2, 4, 1, 64)), 0, 0, 5)
    with pytest.raises(ValueError):
        kv.row_of(kv.KVLayout(kv.CONTIGUOUS, 4), 0, 4)
    with pytest.raises(ValueError):
        kv.row_of(ring, 0, -1)
