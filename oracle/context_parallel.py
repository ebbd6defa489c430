"""Attention over shards of the keys, and the merge of their partial results (oracle).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``.

The pages' attention (page "nemo_automodel.components.models.gpt_oss.layers",
GptOssAttention; Transformers v4.55.0 release notes, "Architecture": the sink
adds one term to the softmax denominator; the rope_utils page rotates q and k
at their positions, and its context-parallel arguments split a sequence over
ranks) can be computed one block of keys at a time. For a query row, a shard
of keys yields

    lse_p = log sum_j e^{s_j}          (over the shard's visible keys; -inf if none)
    o_p   = sum_j e^{s_j - lse_p} v_j  (0 if none)

and the attention over the union of the shards, with the sink sigma counted
once, is

    lse = log(e^sigma + sum_p e^{lse_p}),    o = sum_p e^{lse_p - lse} o_p.

Positions are global: query s of a shard that starts at q_offset sits at
q_offset + s, key j of a shard at kv_offset + j; the causal / window mask and
the rotations use those positions. Everything is fp64 (bf16 rounding only at
the rotated q and k, as in oracle.attention). Pinned by
tests/test_oracle_context_parallel.py.
"""

import numpy as np

from .rope import rotate
from .yarn import RopeConfig, cos_sin_table


def shard_attention(q, k, v, scale, window, q_offset, kv_offset, cfg: RopeConfig = RopeConfig(), rotate_qk=True):
    """q [B, Sq, Hq, D], k / v [B, Sk, Hkv, D] (q and k un-rotated when rotate_qk).

    Returns (o [B, Sq, Hq, D], lse [B, Sq, Hq]) without any sink term."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    qp = q_offset + np.arange(Sq)
    kp = kv_offset + np.arange(Sk)
    if rotate_qk:
        c, s = cos_sin_table(cfg, qp)
        q = rotate(q, c[None, :, None, :], s[None, :, None, :])
        c, s = cos_sin_table(cfg, kp)
        k = rotate(k, c[None, :, None, :], s[None, :, None, :])
    diff = qp[:, None] - kp[None, :]
    vis = diff >= 0
    if window > 0:
        vis &= diff < window
    o = np.zeros((B, Sq, Hq, D))
    lse = np.full((B, Sq, Hq), -np.inf)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            sc = scale * (q[b, :, h, :] @ k[b, :, h // g, :].T)
            sc = np.where(vis, sc, -np.inf)
            m = sc.max(axis=1, keepdims=True)
            has = np.isfinite(m[:, 0])
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(sc - m)
            z = e.sum(axis=1)
            lse[b, has, h] = (m[:, 0] + np.log(np.where(has, z, 1.0)))[has]
            w = e / np.where(z > 0, z, 1.0)[:, None]
            o[b, :, h, :] = w @ v[b, :, h // g, :]
    return o, lse


def merge(parts, sinks):
    """parts: list of (o [.., Hq, D], lse [.., Hq]); sinks [Hq] (-inf allowed).

    Returns (o, lse) of the attention over all the parts' keys with the sink once."""
    sinks = np.asarray(sinks, dtype=np.float64)
    if not parts:
        raise ValueError("merge needs the shape of at least one part")
    lse_all = np.stack([np.asarray(l, dtype=np.float64) for _, l in parts])      # [P, .., Hq]
    sig = np.broadcast_to(sinks, lse_all.shape[1:])
    M = np.maximum(sig, lse_all.max(axis=0))
    Mu = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(lse_all - Mu)                                                     # e^{-inf} = 0
    z = np.exp(sig - Mu) + w.sum(axis=0)
    o = sum(w[i][..., None] * np.asarray(parts[i][0], dtype=np.float64) for i in range(len(parts)))
    o = np.where(z[..., None] > 0, o / np.where(z > 0, z, 1.0)[..., None], 0.0)
    lse = np.where(z > 0, Mu + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    return o, lse
