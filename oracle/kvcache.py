"""KV caches of the decode loop: append and decode over contiguous, paged and ring caches (oracle).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``.

No page specifies a KV cache. The pages show the generation loop (the
``model.generate`` examples of the Transformers v4.55.0 release notes, "Welcome
GPT OSS"), in which every new token attends to the keys and values of all
earlier tokens of its sequence; what a token attends to is the definition in
``oracle.attention`` (page "nemo_automodel.components.models.gpt_oss.layers",
GptOssAttention; the same notes, "Architecture"). A cache is only the place
where those keys and values are kept between steps. The readings used here:

* A cache row holds k rotated at its own position (rounded once to bf16, as
  page "nemo_automodel.components.models.gpt_oss.rope_utils",
  _apply_rotary_emb_qk, rotates k) and v unchanged.
* cache_seqlens[n] counts the tokens of sequence n including the ones being
  appended; the num_new tokens appended in one call sit at positions
  L - num_new .. L - 1, and the decoded token is the one at L - 1.
* Where position p of sequence n lives:
    contiguous  row p of sequence n                    (k_cache [N, capacity, Hkv, D])
    paged       row p mod page_size of physical page   (k_cache [num_pages, page_size, Hkv, D])
                block_table[n, p div page_size]
    ring        slot p mod capacity of sequence n      (k_cache [N, capacity, Hkv, D])
  A ring keeps only the last ``capacity`` positions: exactly what a sliding-
  window layer whose window equals the capacity reads.

Everything is numpy float64 holding bf16 values, as in the rest of the oracle.
Pinned by tests/test_oracle_kvcache.py.
"""

from dataclasses import dataclass

import numpy as np

from .attention import sink_attention
from .rope import rotate
from .yarn import RopeConfig, cos_sin_table

CONTIGUOUS, PAGED, RING = "contiguous", "paged", "ring"


@dataclass
class KVLayout:
    kind: str                          # CONTIGUOUS, PAGED or RING
    capacity: int                      # rows per sequence / rows per page / slots per sequence
    block_table: np.ndarray = None     # PAGED: [N, max_pages] physical page of each logical page


def row_of(layout: KVLayout, n: int, p: int):
    """Index of position p of sequence n in the first two dims of the cache arrays."""
    if p < 0:
        raise ValueError("negative position")
    if layout.kind == CONTIGUOUS:
        if p >= layout.capacity:
            raise ValueError(f"position {p} beyond the {layout.capacity} rows of a contiguous cache")
        return n, p
    if layout.kind == PAGED:
        return int(layout.block_table[n, p // layout.capacity]), p % layout.capacity
    if layout.kind == RING:
        return n, p % layout.capacity
    raise ValueError(f"unknown cache kind {layout.kind!r}")


def append(layout: KVLayout, k_cache, v_cache, k_new, v_new, cache_seqlens, cfg: RopeConfig = RopeConfig(),
           rotate_k=True):
    """Store num_new tokens per sequence; returns updated copies of the caches.

    k_new / v_new [N, num_new, Hkv, D]; token t of sequence n has position
    L_n - num_new + t. Tokens are stored in position order, so in a ring a
    later position overwrites an earlier one that maps to the same slot.
    """
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    N, T = k_new.shape[:2]
    for n in range(N):
        L = int(cache_seqlens[n])
        for t in range(T):
            p = L - T + t
            if p < 0:
                continue
            kk = k_new[n, t]
            if rotate_k:
                c, s = cos_sin_table(cfg, [p])
                kk = rotate(kk[None], c[:, None, :], s[:, None, :])[0]
            i = row_of(layout, n, p)
            kc[i] = kk
            vc[i] = v_new[n, t]
    return kc, vc


def logical_rows(layout: KVLayout, k_cache, v_cache, n, lo, hi):
    """K and V rows of positions lo .. hi - 1 of sequence n, in position order."""
    if layout.kind == RING and hi - lo > layout.capacity:
        raise ValueError("a ring holds only its last `capacity` positions")
    idx = [row_of(layout, n, p) for p in range(lo, hi)]
    if not idx:
        shape = (0,) + tuple(np.shape(k_cache)[2:])
        return np.zeros(shape), np.zeros(shape)
    return (np.stack([np.asarray(k_cache[i], dtype=np.float64) for i in idx]),
            np.stack([np.asarray(v_cache[i], dtype=np.float64) for i in idx]))


def decode(layout: KVLayout, q, k_cache, v_cache, cache_seqlens, sinks, scale, window,
           cfg: RopeConfig = RopeConfig(), rotate_q=True):
    """The token at position L_n - 1 of every sequence against its cached keys.

    q [N, Hq, D] (un-rotated when rotate_q). The visible positions are those the
    mask allows (all of 0 .. L - 1, or the last min(L, window) of them), each
    read from wherever the layout keeps it. Returns fp64 [N, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    N = q.shape[0]
    out = np.zeros(q.shape[:2] + (np.shape(v_cache)[-1],), dtype=np.float64)
    for n in range(N):
        L = int(cache_seqlens[n])
        if L <= 0:
            continue
        qn = q[n][None]
        if rotate_q:
            c, s = cos_sin_table(cfg, [L - 1])
            qn = rotate(qn, c[:, None, :], s[:, None, :])
        lo = 0 if window <= 0 else max(0, L - window)
        ks, vs = logical_rows(layout, k_cache, v_cache, n, lo, L)
        out[n] = sink_attention(qn, ks, vs, sinks, scale, np.array([L - 1]), np.arange(lo, L), window)[0]
    return out
