"""Seeded synthetic workloads: input tensors and work counts.

This module draws random inputs and counts work; it holds none of the
attention or RoPE arithmetic. The HIP path (via the binding) and the CPU oracle
consume the very same CPU tensors it returns.

Generation recipe (one torch.Generator per workload, seeded, in this order):
  1. sequence lengths, if the workload has any: torch.randint(lo, hi + 1, (n,));
  2. q, then k, then v: torch.randn(shape, dtype=float32) rounded to bfloat16;
     for a decode KV cache, sequence by sequence, K rows then V rows of the
     valid length only (rows past the length stay zero);
  3. sinks: torch.randn(num_q_heads, dtype=float32).
Paged pools, ring caches and appended tokens have their own draw orders (see
paged_decode, ring_decode, new_tokens).

The shapes follow GPT-OSS's attention: 64 query heads and 8 KV heads of width
64 (q_proj 2880->4096, k_proj / v_proj 2880->512 in the gpt-oss-20b module
print-out), scale 64 ** -0.5.
"""

from dataclasses import dataclass, field

import torch

HQ, HKV, HEAD_DIM = 64, 8, 64
SCALE = HEAD_DIM ** -0.5
WINDOW = 128


@dataclass
class Prefill:
    name: str
    layout: str                      # "bshd" or "thd"
    q: torch.Tensor                  # bshd [B,S,Hq,D] / thd [T,Hq,D], bf16, CPU
    k: torch.Tensor
    v: torch.Tensor
    sinks: torch.Tensor              # fp32 [Hq]
    cu_seqlens: torch.Tensor = None  # int32 [N+1] (thd only)
    lengths: list = field(default_factory=list)

    @property
    def seq_lengths(self):
        if self.layout == "thd":
            return list(self.lengths)
        return [self.q.shape[1]] * self.q.shape[0]

    @property
    def max_seqlen(self):
        return max(self.seq_lengths) if self.seq_lengths else 0


@dataclass
class Decode:
    name: str
    q: torch.Tensor                  # [N,Hq,D] bf16, un-rotated
    k_cache: torch.Tensor            # [N,Lmax,Hkv,D] bf16, K taken as already rotated
    v_cache: torch.Tensor
    cache_seqlens: torch.Tensor      # int32 [N], includes the new token
    sinks: torch.Tensor
    lengths: list = field(default_factory=list)


def _randn_bf16(shape, g):
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def prefill_bshd(B, S, seed, hq=HQ, hkv=HKV, d=HEAD_DIM, name=None):
    g = torch.Generator().manual_seed(seed)
    q = _randn_bf16((B, S, hq, d), g)
    k = _randn_bf16((B, S, hkv, d), g)
    v = _randn_bf16((B, S, hkv, d), g)
    sinks = torch.randn(hq, generator=g, dtype=torch.float32)
    return Prefill(name or f"bshd_B{B}_S{S}", "bshd", q, k, v, sinks)


def prefill_thd(num_seqs, lo, hi, seed, hq=HQ, hkv=HKV, d=HEAD_DIM, lengths=None, name=None):
    """Packed sequences with lengths uniform in [lo, hi] (or the given lengths)."""
    g = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = torch.randint(lo, hi + 1, (num_seqs,), generator=g).tolist()
    lengths = [int(x) for x in lengths]
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    T = cu[-1]
    q = _randn_bf16((T, hq, d), g)
    k = _randn_bf16((T, hkv, d), g)
    v = _randn_bf16((T, hkv, d), g)
    sinks = torch.randn(hq, generator=g, dtype=torch.float32)
    return Prefill(name or f"thd_N{len(lengths)}_T{T}", "thd", q, k, v, sinks,
                   cu_seqlens=torch.tensor(cu, dtype=torch.int32), lengths=lengths)


def decode(num_seqs, lo, hi, seed, max_len=None, hq=HQ, hkv=HKV, d=HEAD_DIM, lengths=None, name=None):
    """One query token per sequence, cache lengths uniform in [lo, hi] (incl. the new token)."""
    g = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = torch.randint(lo, hi + 1, (num_seqs,), generator=g).tolist()
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    Lmax = max_len if max_len is not None else hi
    q = _randn_bf16((N, hq, d), g)
    kc = torch.zeros((N, Lmax, hkv, d), dtype=torch.bfloat16)
    vc = torch.zeros((N, Lmax, hkv, d), dtype=torch.bfloat16)
    for n, L in enumerate(lengths):
        kc[n, :L] = _randn_bf16((L, hkv, d), g)
        vc[n, :L] = _randn_bf16((L, hkv, d), g)
    sinks = torch.randn(hq, generator=g, dtype=torch.float32)
    return Decode(name or f"decode_N{N}", q, kc, vc, torch.tensor(lengths, dtype=torch.int32), sinks,
                  lengths=lengths)


@dataclass
class PagedDecode:
    name: str
    q: torch.Tensor                  # [N,Hq,D] bf16, un-rotated
    k_pool: torch.Tensor             # [num_pages, page_size, Hkv, D] bf16, every row random
    v_pool: torch.Tensor
    block_table: torch.Tensor        # int32 [N, max_pages]: a random permutation of the used pages
    cache_seqlens: torch.Tensor      # int32 [N]
    sinks: torch.Tensor
    lengths: list = field(default_factory=list)


def paged_decode(lengths, page_size, seed, spare_pages=3, hq=HQ, hkv=HKV, d=HEAD_DIM, name=None):
    """A decode batch over a paged KV pool. Sequence n owns ceil(L_n / page_size)
    pages (at least one); the pool holds those plus `spare_pages` unused ones, in
    an order drawn by torch.randperm, and block-table entries past a sequence's
    pages name page 0. Draw order: q, the K pool, the V pool, the permutation, sinks."""
    g = torch.Generator().manual_seed(seed)
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    pages = [max(1, -(-L // page_size)) for L in lengths]
    total = sum(pages) + spare_pages
    q = _randn_bf16((N, hq, d), g)
    kp = _randn_bf16((total, page_size, hkv, d), g)
    vp = _randn_bf16((total, page_size, hkv, d), g)
    perm = torch.randperm(total, generator=g)
    bt = torch.zeros((N, max(pages)), dtype=torch.int32)
    at = 0
    for n, c in enumerate(pages):
        bt[n, :c] = perm[at:at + c].to(torch.int32)
        at += c
    sinks = torch.randn(hq, generator=g, dtype=torch.float32)
    return PagedDecode(name or f"paged_N{N}_P{page_size}", q, kp, vp, bt, torch.tensor(lengths, dtype=torch.int32),
                       sinks, lengths=lengths)


def ring_decode(lengths, slots, seed, hq=HQ, hkv=HKV, d=HEAD_DIM, name=None):
    """A decode batch over ring caches of `slots` rows per sequence (all rows
    random); lengths are logical and may exceed the slot count. Draw order: q,
    K rings, V rings, sinks."""
    g = torch.Generator().manual_seed(seed)
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    q = _randn_bf16((N, hq, d), g)
    kc = _randn_bf16((N, slots, hkv, d), g)
    vc = _randn_bf16((N, slots, hkv, d), g)
    sinks = torch.randn(hq, generator=g, dtype=torch.float32)
    return Decode(name or f"ring_N{N}_W{slots}", q, kc, vc, torch.tensor(lengths, dtype=torch.int32), sinks,
                  lengths=lengths)


def far_below(lead_q, lead_k, spread, seed, hq=HQ, hkv=HKV, d=HEAD_DIM):
    """Already-rotated q, k whose scaled dot products all lie near -512, and v.

    q = -8 + spread * N(0, 1) and k = +8 + spread * N(0, 1) in every dimension,
    v ~ N(0, 1), all rounded to bf16: with scale 1/8 and width 64 every logit is
    -512 plus a spread of a few units (exactly -512 for spread 0). Draw order:
    q, k, v. Returns (q [lead_q, Hq, D], k [lead_k, Hkv, D], v [lead_k, Hkv, D])."""
    g = torch.Generator().manual_seed(seed)
    q = (-8.0 + spread * torch.randn(tuple(lead_q) + (hq, d), generator=g)).to(torch.bfloat16)
    k = (8.0 + spread * torch.randn(tuple(lead_k) + (hkv, d), generator=g)).to(torch.bfloat16)
    v = _randn_bf16(tuple(lead_k) + (hkv, d), g)
    return q, k, v


def new_tokens(num_seqs, num_new, seed, hkv=HKV, d=HEAD_DIM):
    """k and v of the newest tokens [N, num_new, Hkv, D] (un-rotated k), bf16."""
    g = torch.Generator().manual_seed(seed)
    return _randn_bf16((num_seqs, num_new, hkv, d), g), _randn_bf16((num_seqs, num_new, hkv, d), g)


@dataclass
class Projection:
    name: str
    x: torch.Tensor                  # [tokens, hidden] bf16
    wq: torch.Tensor                 # [Hq*64, hidden] bf16 (Linear weight layout)
    bq: torch.Tensor                 # [Hq*64] bf16
    wk: torch.Tensor
    bk: torch.Tensor
    wv: torch.Tensor
    bv: torch.Tensor


def projection(tokens, seed, hidden=2880, hq=HQ, hkv=HKV, d=HEAD_DIM, name=None):
    """Inputs of the q/k/v projections (gpt-oss-20b print-out: hidden 2880, q 2880 -> 4096,
    k / v 2880 -> 512, Linear with bias): x ~ N(0, 1); weights ~ N(0, 1 / hidden), the scale of
    a Linear initialisation; biases ~ N(0, 0.1^2); all rounded to bf16. Draw order: x, wq, bq,
    wk, bk, wv, bv."""
    g = torch.Generator().manual_seed(seed)
    x = _randn_bf16((tokens, hidden), g)
    ws = []
    for out in (hq * d, hkv * d, hkv * d):
        w = (torch.randn((out, hidden), generator=g, dtype=torch.float32) * hidden ** -0.5).to(torch.bfloat16)
        b = (torch.randn(out, generator=g, dtype=torch.float32) * 0.1).to(torch.bfloat16)
        ws += [w, b]
    return Projection(name or f"proj_T{tokens}", x, *ws)


def projection_flops(tokens, hidden=2880, hq=HQ, hkv=HKV, d=HEAD_DIM):
    """2 * hidden FLOPs per output element of x W^T (the bias adds and the rotation are not counted)."""
    return 2 * tokens * hidden * (hq + 2 * hkv) * d


def grad_out(shape, seed):
    """Gradient of the loss with respect to the attention output for the
    backward pass: torch.randn(shape) rounded to bfloat16, its own generator."""
    g = torch.Generator().manual_seed(seed)
    return _randn_bf16(tuple(shape), g)


# The five workloads of this attention path: a tiny prefill, a dense 4K BSHD
# prefill, packed THD sequences, a 128K-token prefill and a 64-sequence decode.
def tiny(seed=0):
    return prefill_bshd(1, 256, seed, name="tiny_B1_S256")


def dense(seed=1):
    return prefill_bshd(4, 4096, seed, name="dense_B4_S4096")


def thd(seed=2):
    return prefill_thd(16, 128, 8192, seed, name="thd_16seq")


def long_context(seed=3):
    return prefill_bshd(1, 131072, seed, name="long_B1_S131072")


def long_context_rows():
    """The 512 sampled query rows of the 131072-token sequence: 0, 1, 127, 128, 131071
    and the first 507 other entries of torch.randperm(131072) after manual_seed(5), sorted."""
    special = [0, 1, 127, 128, 131071]
    perm = torch.randperm(131072, generator=torch.Generator().manual_seed(5)).tolist()
    extra = [r for r in perm if r not in special][:507]
    return sorted(special + extra)


def decode64(seed=4):
    return decode(64, 1024, 32768, seed, max_len=32768, name="decode_64seq")


def decode64_lengths(seed=4):
    """The cache lengths of decode64 (its generator's first draw) without its caches."""
    g = torch.Generator().manual_seed(seed)
    return [int(x) for x in torch.randint(1024, 32768 + 1, (64,), generator=g).tolist()]


# ---- work counts (what the throughput figures divide by) ----

def visible_pairs(length, window):
    """Number of (query, key) position pairs with j <= i and (window == 0 or i - j < window)."""
    n = int(length)
    if window <= 0 or window >= n:
        return n * (n + 1) // 2
    w = int(window)
    return w * (w + 1) // 2 + (n - w) * w


def prefill_flops(lengths, window, hq=HQ, d=HEAD_DIM):
    """Unmasked FLOPs: 2*D for q.k plus 2*D for p*v per visible pair and query head."""
    return 4 * d * hq * sum(visible_pairs(n, window) for n in lengths)


def prefill_bytes(total_tokens, table_rows, hq=HQ, hkv=HKV, d=HEAD_DIM, rotary_dim=HEAD_DIM):
    """Read q, k, v once, write o once (bf16), read the sinks (fp32) and the bf16 table rows."""
    return (total_tokens * (2 * hq * d * 2 + 2 * hkv * d * 2)
            + hq * 4 + table_rows * rotary_dim * 2)


def decode_bytes(lengths, window, hq=HQ, hkv=HKV, d=HEAD_DIM, rotary_dim=HEAD_DIM):
    """Visible K/V rows + q in + o out + sinks + one table row and one length per sequence."""
    kv_rows = sum(min(L, window) if window > 0 else L for L in lengths)
    N = len(lengths)
    return (kv_rows * hkv * d * 2 * 2 + N * hq * d * 2 * 2 + hq * 4
            + N * rotary_dim * 2 + N * 4)


def decode_flops(lengths, window, hq=HQ, d=HEAD_DIM):
    kv_rows = sum(min(L, window) if window > 0 else L for L in lengths)
    return 4 * d * hq * kv_rows
