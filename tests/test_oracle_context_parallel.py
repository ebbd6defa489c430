"""Pins of oracle.context_parallel (attention over key shards and the merge).

Merging the shards of a sequence must give the prefill definition of
oracle.attention (itself pinned): contiguous and zig-zag shardings, full and
window masks, shards that see no key of a query block. The log-sum-exp of one
shard covering everything equals the backward oracle's (independently
written, finite-difference pinned) with no sink. A pure-Python loop checks the
shard formulas on a tiny case, and the merge's degenerate forms are pinned.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import context_parallel as cp

CFG = oracle.RopeConfig()
TAU = 0.125


def _inputs(seed, B=2, S=48, hq=8, hkv=2):
    rng = np.random.default_rng(seed)
    bf = lambda *s: oracle.round_bf16(rng.standard_normal(s))
    return bf(B, S, hq, 64), bf(B, S, hkv, 64), bf(B, S, hkv, 64), rng.standard_normal(hq)


def _merged_rows(q, k, v, sinks, window, q_lo, q_hi, kv_bounds):
    parts = [cp.shard_attention(q[:, q_lo:q_hi], k[:, a:b], v[:, a:b], TAU, window, q_lo, a, CFG)
             for a, b in kv_bounds]
    return cp.merge(parts, sinks)


@pytest.mark.parametrize("window", [0, 7, 20])
@pytest.mark.parametrize("P", [1, 3, 4])
def test_contiguous_shards_merge_to_the_prefill(window, P):
    q, k, v, sinks = _inputs(1)
    S = q.shape[1]
    ref = oracle.prefill_bshd(q, k, v, sinks, TAU, window, CFG)
    cuts = np.linspace(0, S, P + 1).astype(int)
    bounds = list(zip(cuts[:-1], cuts[1:]))
    for lo, hi in bounds:     # every query shard against every key shard, as a ring would
        o, _ = _merged_rows(q, k, v, sinks, window, lo, hi, bounds)
        np.testing.assert_allclose(o, ref[:, lo:hi], rtol=1e-12, atol=1e-12)


def test_zigzag_shards_merge_to_the_prefill():
    """Rank r of 3 holds chunks r and 5 - r of 6 (the causal load balance of a ring)."""
    q, k, v, sinks = _inputs(2, S=60)
    ref = oracle.prefill_bshd(q, k, v, sinks, TAU, 0, CFG)
    chunks = [(10 * i, 10 * i + 10) for i in range(6)]
    for r in range(3):
        for lo, hi in (chunks[r], chunks[5 - r]):
            o, _ = _merged_rows(q, k, v, sinks, 0, lo, hi, [chunks[c] for c in (0, 5, 1, 4, 2, 3)])
            np.testing.assert_allclose(o, ref[:, lo:hi], rtol=1e-12, atol=1e-12)


def test_whole_sequence_lse_matches_the_backward_oracle():
    q, k, v, _ = _inputs(3, S=40)
    none = np.full(8, -np.inf)
    o, lse = cp.shard_attention(q, k, v, TAU, 0, 0, 0, CFG)
    ref = oracle.prefill_bshd_backward(q, k, v, none, TAU, 0, np.zeros_like(q), CFG)
    np.testing.assert_allclose(lse, ref["lse"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, oracle.prefill_bshd(q, k, v, none, TAU, 0, CFG), rtol=1e-12, atol=1e-12)


def test_shard_brute_force():
    q, k, v, _ = _inputs(4, B=1, S=6, hq=2, hkv=1)   # one KV head: k[..., 0, :] below
    qo, ko = 9, 5          # queries at 9..11, keys at 5..10
    o, lse = cp.shard_attention(q[:, :3], k, v, TAU, 4, qo, ko, CFG, rotate_qk=False)
    for i in range(3):
        for h in range(2):
            vis = [j for j in range(6) if 0 <= (qo + i) - (ko + j) < 4]
            s = [TAU * math.fsum(q[0, i, h] * k[0, j, 0]) for j in vis]
            if not vis:
                assert lse[0, i, h] == -math.inf and not o[0, i, h].any()
                continue
            ls = math.log(math.fsum(math.exp(x) for x in s))
            assert abs(lse[0, i, h] - ls) < 1e-12
            ref = sum(math.exp(x - ls) * v[0, j, 0] for x, j in zip(s, vis))
            np.testing.assert_allclose(o[0, i, h], ref, rtol=1e-12, atol=1e-12)


def test_merge_degenerate_forms():
    rng = np.random.default_rng(5)
    o1, l1 = rng.standard_normal((3, 4, 64)), rng.standard_normal((3, 4))
    empty = (np.zeros((3, 4, 64)), np.full((3, 4), -np.inf))
    sinks = rng.standard_normal(4)
    # a part with no keys changes nothing; with sink -inf one part is returned as is
    a = cp.merge([(o1, l1), empty], sinks)
    b = cp.merge([(o1, l1)], sinks)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-14)
    c = cp.merge([(o1, l1)], np.full(4, -np.inf))
    np.testing.assert_allclose(c[0], o1, rtol=1e-14)
    np.testing.assert_allclose(c[1], l1, rtol=1e-14)
    # only the sink: output 0, lse = sigma
    d = cp.merge([empty], sinks)
    assert not d[0].any() and np.allclose(d[1], np.broadcast_to(sinks, (3, 4)))
    # sink weight: lse = log(e^sigma + e^lse1)
    np.testing.assert_allclose(b[1], np.logaddexp(sinks, l1), rtol=1e-14)
