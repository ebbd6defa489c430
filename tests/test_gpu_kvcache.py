"""GPU parity of the KV-cache append and of decode over paged and ring caches,
against oracle.kvcache, through the C ABI.

Append is compared bit for bit (the rotation is exact and v is copied): the
whole cache after the call, so rows that must not change are checked too.
Decode uses the elementwise tolerance of helpers.py; a paged full-layer decode
is also bit-identical to the contiguous decode of the same rows. The loop test
runs prompt appends and several decode steps over contiguous, paged and ring
caches side by side with the oracle doing the same.
"""

import numpy as np
import pytest
import torch

import attention_yarn_rope_amd as gx
import oracle
from attention_yarn_rope_amd import workloads as wl
from helpers import assert_close, np64, say
from oracle import kvcache as kv

pytestmark = pytest.mark.gpu
CFG = oracle.RopeConfig()
TAU = 0.125


@pytest.fixture(scope="module")
def table():
    return gx.rope_table(80000)


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)


def _caches(kind, N, seed, hkv=8):
    """Random initial caches (so untouched rows are checked) and the oracle layout."""
    g = torch.Generator().manual_seed(seed)
    if kind == "contiguous":
        shape, bt = (N, 160, hkv, 64), None
        lay = kv.KVLayout(kv.CONTIGUOUS, 160)
    elif kind == "ring":
        shape, bt = (N, 16, hkv, 64), None
        lay = kv.KVLayout(kv.RING, 16)
    else:
        max_pages, ps = 5, 32
        pool = N * max_pages + 2
        bt = torch.randperm(pool, generator=g)[: N * max_pages].reshape(N, max_pages).to(torch.int32)
        shape = (pool, ps, hkv, 64)
        lay = kv.KVLayout(kv.PAGED, ps, bt.numpy())
    kc = torch.randn(shape, generator=g).to(torch.bfloat16)
    vc = torch.randn(shape, generator=g).to(torch.bfloat16)
    return kc, vc, bt, lay


@pytest.mark.parametrize("kind", ["contiguous", "paged", "ring"])
@pytest.mark.parametrize("T", [1, 7, 20])
def test_append_bit_exact(table, kind, T):
    """Ragged lengths: L = 0 and L < T skip the tokens without a position; a ring of
    16 slots receives T = 20 tokens in one call (only the last 16 land)."""
    N = 6
    lengths = [0, 3, T, 40, 100, 150]
    kc, vc, bt, lay = _caches(kind, N, 100 + T)
    kn, vn = wl.new_tokens(N, T, 200 + T)
    say(f"[gpu] kv append kind={kind} T={T}")
    kg, vg = kc.cuda(), vc.cuda()
    gx.kv_append(kg, vg, kn.cuda(), vn.cuda(), torch.tensor(lengths, dtype=torch.int32).cuda(), kind=kind,
                 block_table=bt.cuda() if bt is not None else None, table=table)
    rk, rv = kv.append(lay, np64(kc), np64(vc), np64(kn), np64(vn), lengths, CFG)
    assert torch.equal(kg.cpu(), _bf16(rk)), "k cache differs from the oracle"
    assert torch.equal(vg.cpu(), _bf16(rv)), "v cache differs from the oracle"


def test_append_without_table_stores_k_as_given():
    N, T = 3, 4
    kc, vc, _, lay = _caches("contiguous", N, 7)
    kn, vn = wl.new_tokens(N, T, 8)
    kg, vg = kc.cuda(), vc.cuda()
    gx.kv_append(kg, vg, kn.cuda(), vn.cuda(), torch.tensor([4, 9, 17], dtype=torch.int32).cuda())
    rk, rv = kv.append(lay, np64(kc), np64(vc), np64(kn), np64(vn), [4, 9, 17], CFG, rotate_k=False)
    assert torch.equal(kg.cpu(), _bf16(rk)) and torch.equal(vg.cpu(), _bf16(rv))


def test_append_equals_rope_qk(table):
    """A whole prompt appended in one call holds exactly the keys gptoss_rope_qk produces."""
    inp = wl.prefill_bshd(2, 150, seed=31)
    k = inp.k.cuda()
    kc = torch.zeros((2, 160, 8, 64), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    gx.kv_append(kc, vc, k, inp.v.cuda(), torch.tensor([150, 150], dtype=torch.int32).cuda(), table=table)
    _, kr = gx.rope_qk(inp.q.cuda(), k, table)
    assert torch.equal(kc[:, :150], kr)
    assert torch.equal(vc[:, :150].cpu(), inp.v)


def _paged_ref(w, window):
    lay = kv.KVLayout(kv.PAGED, w.k_pool.shape[1], w.block_table.numpy())
    # the pools as float32 (exact for bf16): the oracle reads only the rows it needs
    return kv.decode(lay, np64(w.q), w.k_pool.float().numpy(), w.v_pool.float().numpy(), w.lengths, np64(w.sinks),
                     TAU, window, CFG)


@pytest.mark.parametrize("page_size", [32, 64, 256])
@pytest.mark.parametrize("window", [0, 128, 5])
def test_decode_paged(table, page_size, window):
    w = wl.paged_decode([1, 31, 32, 33, 300, 1000, 1500], page_size, seed=40 + page_size + window)
    say(f"[gpu] paged decode page={page_size} window={window}")
    out = gx.attn_decode_kv(w.q.cuda(), w.k_pool.cuda(), w.v_pool.cuda(), w.cache_seqlens.cuda(), w.sinks.cuda(),
                            kind="paged", block_table=w.block_table.cuda(), window=window, table=table,
                            max_seqlen=1500)
    assert_close(out, _paged_ref(w, window), f"paged P={page_size} W={window}")


def _gather(w):
    """The contiguous cache holding the same rows as a paged pool (test-side indexing)."""
    N, ps = len(w.lengths), w.k_pool.shape[1]
    Lmax = max(w.lengths)
    kc = torch.zeros((N, Lmax, 8, 64), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    for n, L in enumerate(w.lengths):
        p = torch.arange(L)
        pages = w.block_table[n, p // ps].long()
        kc[n, :L] = w.k_pool[pages, p % ps]
        vc[n, :L] = w.v_pool[pages, p % ps]
    return kc, vc


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_paged_equals_contiguous_full_layer(table, splits):
    """Full layers read the same keys in the same 32-key steps from either layout."""
    w = wl.paged_decode([1, 33, 700, 2000, 4096], 64, seed=50 + splits)
    kc, vc = _gather(w)
    q, lens, s = w.q.cuda(), w.cache_seqlens.cuda(), w.sinks.cuda()
    a = gx.attn_decode_kv(q, w.k_pool.cuda(), w.v_pool.cuda(), lens, s, kind="paged",
                          block_table=w.block_table.cuda(), table=table, max_seqlen=4096, num_splits=splits)
    b = gx.attn_decode(q, kc.cuda(), vc.cuda(), lens, s, table=table, num_splits=splits)
    c = gx.attn_decode_kv(q, kc.cuda(), vc.cuda(), lens, s, kind="contiguous", table=table, num_splits=splits)
    assert torch.equal(a, b) and torch.equal(b, c)


@pytest.mark.parametrize("lengths", [[1, 50, 127, 128, 129, 1000], [70000, 3, 128 * 300 + 17]])
def test_decode_ring(table, lengths):
    w = wl.ring_decode(lengths, 128, seed=60 + len(lengths))
    say(f"[gpu] ring decode lengths={lengths}")
    out = gx.attn_decode_kv(w.q.cuda(), w.k_cache.cuda(), w.v_cache.cuda(), w.cache_seqlens.cuda(), w.sinks.cuda(),
                            kind="ring", window=128, table=table, max_seqlen=max(lengths))
    lay = kv.KVLayout(kv.RING, 128)
    ref = kv.decode(lay, np64(w.q), np64(w.k_cache), np64(w.v_cache), lengths, np64(w.sinks), TAU, 128, CFG)
    assert_close(out, ref, f"ring lengths={lengths}")


def test_generation_loop(table):
    """Ragged prompts written by one bulk append, then decode steps that append one
    token each: full layer on contiguous and paged caches, window-128 layer on a ring."""
    N, prompt = 3, [5, 40, 130]
    Tp = max(prompt)
    g = torch.Generator().manual_seed(70)
    sinks = torch.randn(64, generator=g)
    lens = list(prompt)
    kn, vn = wl.new_tokens(N, Tp, 71)
    cont = kv.KVLayout(kv.CONTIGUOUS, 256)
    ring = kv.KVLayout(kv.RING, 128)
    bt = torch.randperm(3 * 8 + 1, generator=g)[:24].reshape(3, 8).to(torch.int32)
    paged = kv.KVLayout(kv.PAGED, 32, bt.numpy())
    caches = {
        "contiguous": (cont, torch.zeros((N, 256, 8, 64), dtype=torch.bfloat16), None),
        "paged": (paged, torch.zeros((25, 32, 8, 64), dtype=torch.bfloat16), bt),
        "ring": (ring, torch.zeros((N, 128, 8, 64), dtype=torch.bfloat16), None),
    }
    gpu = {k: (c.cuda(), c.clone().cuda()) for k, (_, c, _) in caches.items()}
    ref = {k: (np64(c), np64(c)) for k, (_, c, _) in caches.items()}

    def append_all(kn_, vn_, lens_):
        L = torch.tensor(lens_, dtype=torch.int32).cuda()
        for k, (lay, _, b) in caches.items():
            gx.kv_append(gpu[k][0], gpu[k][1], kn_.cuda(), vn_.cuda(), L, kind=k,
                         block_table=b.cuda() if b is not None else None, table=table, max_seqlen=256)
            ref[k] = kv.append(lay, ref[k][0], ref[k][1], np64(kn_), np64(vn_), lens_, CFG)

    append_all(kn, vn, lens)
    for step in range(4):
        lens = [L + 1 for L in lens]
        k1, v1 = wl.new_tokens(N, 1, 80 + step)
        append_all(k1, v1, lens)
        q = wl.new_tokens(N, 8, 90 + step)[0].reshape(N, 64, 64)   # any bf16 [N, Hq, D]
        L = torch.tensor(lens, dtype=torch.int32).cuda()
        say(f"[gpu] generation loop step {step} lengths={lens}")
        for k, window in (("contiguous", 0), ("paged", 0), ("ring", 128)):
            lay, _, b = caches[k]
            out = gx.attn_decode_kv(q.cuda(), gpu[k][0], gpu[k][1], L, sinks.cuda(), kind=k,
                                    block_table=b.cuda() if b is not None else None, window=window, table=table,
                                    max_seqlen=256)
            r = kv.decode(lay, np64(q), ref[k][0], ref[k][1], lens, np64(sinks), TAU, window, CFG)
            assert_close(out, r, f"loop step {step} {k}")
    for k in caches:
        assert torch.equal(gpu[k][0].cpu(), _bf16(ref[k][0])) and torch.equal(gpu[k][1].cpu(), _bf16(ref[k][1]))


@pytest.fixture(scope="module")
def paged64():
    return wl.paged_decode(wl.decode64_lengths(), 64, seed=44)


@pytest.mark.parametrize("window", [0, 128])
def test_decode64_paged_full_size(table, paged64, window):
    """The 64-sequence decode's lengths (uniform in [1024, 32768]) over a paged pool of
    64-row pages: the full layer is bit-identical to the contiguous decode of the same
    rows, the window layer matches the oracle on every output."""
    w = paged64
    say(f"[gpu] decode64 paged window={window}")
    q, lens, s = w.q.cuda(), w.cache_seqlens.cuda(), w.sinks.cuda()
    out = gx.attn_decode_kv(q, w.k_pool.cuda(), w.v_pool.cuda(), lens, s, kind="paged",
                            block_table=w.block_table.cuda(), window=window, table=table, max_seqlen=32768)
    if window == 0:
        kc, vc = _gather(w)
        ref = gx.attn_decode(q, kc.cuda(), vc.cuda(), lens, s, table=table)
        assert torch.equal(out, ref)
    else:
        assert_close(out, _paged_ref(w, window), "decode64 paged W=128")


def test_decode64_ring_window(table):
    lengths = wl.decode64_lengths()
    w = wl.ring_decode(lengths, 128, seed=45)
    out = gx.attn_decode_kv(w.q.cuda(), w.k_cache.cuda(), w.v_cache.cuda(), w.cache_seqlens.cuda(), w.sinks.cuda(),
                            kind="ring", window=128, table=table, max_seqlen=32768)
    ref = kv.decode(kv.KVLayout(kv.RING, 128), np64(w.q), np64(w.k_cache), np64(w.v_cache), lengths,
                    np64(w.sinks), TAU, 128, CFG)
    assert_close(out, ref, "decode64 ring W=128")
