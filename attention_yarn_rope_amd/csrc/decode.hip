// Split-KV decode attention for GPT-OSS on gfx950: one new query token per
// sequence against a bf16 KV cache, with the per-head sink, GQA and the
// causal / sliding-window mask of prefill (page
// "nemo_automodel.components.models.gpt_oss.layers", GptOssAttention;
// Transformers v4.55.0 release notes, "Architecture").
//
// Split kernel: one work group per (key chunk, sequence, group of 8 KV heads);
// the chunk length comes from the plan kernel below;
// wave w takes KV head w, so the group streams whole 1 KB cache rows (8 heads
// x 128 B) and each K/V row of a head is read from HBM exactly once for the 8
// query heads that share it. Rows are fetched with non-temporal loads
// (read-once data) in whole 128-byte rows, 32 keys per step, the next step's
// loads in flight while the current one computes. K and V pass
// through one per-wave LDS block: K is read back as MFMA A fragments for
// S^T = K Q^T (v_mfma_f32_16x16x32_bf16, 8 heads padded to 16 columns), V
// transposed with ds_read_b64_tr_b16 for O^T = V^T P^T. Exact online softmax per step; each
// wave writes one unnormalised partial (m, l, acc[64]) per query head.
// Combine kernel: per (sequence, query head) it merges the partials and adds
// the sink exactly once: M = max(sigma, m_s), l = exp(sigma - M) + sum l_s
// exp(m_s - M), o = sum acc_s exp(m_s - M) / l (all in log2 units). With one
// split per sequence (window layers, short caches) the split kernel applies
// the same formula to its single partial itself, in the same operation order,
// and no combine kernel runs.
#include <mutex>

#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

constexpr int NW = 8;          // waves per work group: one KV head each
constexpr int NT = 64 * NW;
constexpr int NTC = 256;       // combine kernel block
constexpr int SUB = 32;        // keys per wave step
constexpr int DVS = 80;        // LDS row stride of a wave's K / V block (160 B)

// max / sum over lanes l, l^16, l^32, l^48 (the 4 lanes of one MFMA column)
__device__ __forceinline__ float col_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The keys of sequence n: the query sits at position L - 1 (L = its clamped
// length); keys [start, end) are read and those before lo are masked. A
// contiguous cache reads exactly the visible positions. A paged cache starts at
// the 32-key boundary at or before lo, so that every 32-key step lies inside
// one page (pages hold a power of two >= 32 rows). A ring holds the last
// ring_slots positions in slots 0 .. min(L, ring_slots) - 1, all visible (the
// window equals the slot count), and the order of keys does not change the
// result.
struct KeySpan { int L, lo, start, end; };
__device__ __forceinline__ KeySpan key_span(const DecodeParams& p, int n) {
  KeySpan r;
  r.L = min(max(__ldg(p.cache_seqlens + n), 0), p.max_cache_len);
  if (p.kind == kCacheRing) {
    r.lo = r.start = 0;
    r.end = min(r.L, p.ring_slots);
  } else {
    r.lo = (p.window > 0) ? max(0, r.L - p.window) : 0;
    r.start = (p.kind == kCachePaged) ? (r.lo & ~(SUB - 1)) : r.lo;
    r.end = r.L;
  }
  return r;
}

template <bool ROTQ, bool PAGED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void decode_split_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t lds_v[NW][SUB * DVS];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.z * NW + wave;
  const int col = lane & 15, grp = lane >> 4;
  if (g >= p.num_kv_heads) return;
  const bool direct = p.direct_chunk > 0;
  const int chunk = direct ? p.direct_chunk : __builtin_amdgcn_readfirstlane(p.plan[0]);
  const int items = direct ? p.num_seqs : __builtin_amdgcn_readfirstlane(p.plan[1]);
  const int2* work = reinterpret_cast<const int2*>(p.plan + 2);
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
  const int2 w = direct ? make_int2(it, 0) : work[it];
  const int n = __builtin_amdgcn_readfirstlane(w.x);
  const int split = __builtin_amdgcn_readfirstlane(w.y);
  const KeySpan span = key_span(p, n);
  const int L = span.L, lo = span.lo;
  const int c0 = span.start + split * chunk;
  const int c1 = min(c0 + chunk, span.end);
  const float sl = p.scale_log2;

  const char* kbase = reinterpret_cast<const char*>(p.k + (int64_t)n * p.kv_sn + (int64_t)g * p.kv_sh);
  const char* vbase = reinterpret_cast<const char*>(p.v + (int64_t)n * p.kv_sn + (int64_t)g * p.kv_sh);
  bf16_t* vl = lds_v[wave];
  const int32_t row_bytes = (int32_t)p.kv_sp * 2;   // < 2^31 over a whole sequence (host check)
  // per-lane byte offset inside a step: row (lane >> 3) + 8 i, 16-byte chunk lane & 7,
  // so one load instruction moves 8 whole 128-byte rows of this head
  const uint32_t roff = (uint32_t)((lane >> 3) * row_bytes + 16 * (lane & 7));

  // The rows of step s + 1 are requested as soon as step s has moved its rows
  // into LDS. The buffer range ends after key c1 - 1, so rows past the chunk
  // read as zeros.
  uint4 kr[4], vr[4];
  auto load_block = [&](int s0) __attribute__((always_inline)) {
    if (PAGED) {
      // the step lies inside one page: its rows start at row s0 mod page_size of
      // the page the block table names; rows past c1 and rows before lo (the
      // 32-key boundary below a window's first key) read as zeros
      const int lp = s0 >> p.page_log2;
      const int pid = min(max(__ldg(p.block_table + (int64_t)n * p.max_pages + min(lp, p.max_pages - 1)), 0),
                          p.num_pages - 1);
      const int64_t at = (int64_t)pid * p.kv_sn + (int64_t)(s0 - (lp << p.page_log2)) * p.kv_sp;
      const int32_t bytes = (c1 > s0) ? (min(c1 - s0, SUB) - 1) * row_bytes + 2 * kHeadDim : 0;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + at + (int64_t)g * p.kv_sh, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + at + (int64_t)g * p.kv_sh, bytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = (s0 + (lane >> 3) + 8 * i < lo) ? 0x80000000u : roff + (uint32_t)(i * 8 * row_bytes);
        kr[i] = ldb16_nt(rk, off);
        vr[i] = ldb16_nt(rv, off);
      }
    } else {
      const int64_t start = (int64_t)s0 * row_bytes;
      const int32_t bytes = (c1 > s0) ? (c1 - s0 - 1) * row_bytes + 2 * kHeadDim : 0;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + start, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + start, bytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kr[i] = ldb16_nt(rk, roff + (uint32_t)(i * 8 * row_bytes));
        vr[i] = ldb16_nt(rv, roff + (uint32_t)(i * 8 * row_bytes));
      }
    }
  };
  // the first step's rows are requested before q, so both latencies overlap
  if (c0 < c1) load_block(c0);

  // Q fragments (B operand, 8 query heads in columns 0..7; columns 8..15 are
  // zero padding). Every lane loads a valid row so the loads need no branch.
  bf16x8_t qf[2];
  {
    const bf16_t* qp = p.q + (int64_t)n * p.q_sn + (int64_t)(g * kGroup + (col & (kGroup - 1))) * p.q_sh;
    const uint4 x1 = ldg16(qp + 8 * grp), x2 = ldg16(qp + 32 + 8 * grp);
    uint4 y1 = x1, y2 = x2;
    if (ROTQ) {
      const bf16_t* tp = p.table + (int64_t)min(max(L - 1, 0), p.table_rows - 1) * (16 * p.rot_chunks);
      if (p.rot_chunks == kHeadDim / 16) {
        rope8(x1, x2, ldg16(tp + 8 * grp), ldg16(tp + 32 + 8 * grp), y1, y2);
      } else {   // partial rotary: each chunk with its pair partner
        y1 = rope_chunk_partial(qp, tp, grp, p.rot_chunks, x1);
        y2 = rope_chunk_partial(qp, tp, grp + 4, p.rot_chunks, x2);
      }
    }
    const uint4 zero = make_uint4(0, 0, 0, 0);
    qf[0] = as_bf16x8(col < kGroup ? y1 : zero);
    qf[1] = as_bf16x8(col < kGroup ? y2 : zero);
  }

  float m = -INFINITY, lsum = 0.0f;
  f32x4_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int s0) __attribute__((always_inline)) {
    // K rows -> LDS -> MFMA A fragments
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(vl + ((lane >> 3) + 8 * i) * DVS + 8 * (lane & 7)) = kr[i];
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    bf16x8_t ka[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      ka[kb][0] = *reinterpret_cast<const bf16x8_t*>(vl + (kb * 16 + col) * DVS + 8 * grp);
      ka[kb][1] = *reinterpret_cast<const bf16x8_t*>(vl + (kb * 16 + col) * DVS + 32 + 8 * grp);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // V rows -> the same LDS block (the K fragments are in registers now), read back
    // transposed below; the staging registers are then free for the next step's rows
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(vl + ((lane >> 3) + 8 * i) * DVS + 8 * (lane & 7)) = vr[i];
    if (s0 + SUB < c1) load_block(s0 + SUB);
    f32x4_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      z = mfma16(ka[kb][0], qf[0], z);
      sacc[kb] = mfma16(ka[kb][1], qf[1], z);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = s0 + kb * 16 + 4 * grp + r;
        sacc[kb][r] = ((uint32_t)(key - lo) < (uint32_t)(c1 - lo)) ? sacc[kb][r] : -INFINITY;
        mx = fmaxf(mx, sacc[kb][r]);
      }
    mx = col_max(mx);
    const float mnew = fmaxf(m, mx * sl);
    const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
    const float f = __builtin_amdgcn_exp2f(m - mu);
    uint32_t w[4];
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      w[2 * kb] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][0], sl, -mu)),
                              __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][1], sl, -mu)));
      w[2 * kb + 1] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][2], sl, -mu)),
                                  __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][3], sl, -mu)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) psum = add_bf16x2(w[i], psum);
    lsum = lsum * f + psum;
    m = mnew;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= f;
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const bf16_t* vb = vl + (4 * grp + (col >> 2)) * DVS + 16 * db + 4 * (col & 3);
      const uint2 a_lo = lds_read_tr16(vb);
      const uint2 a_hi = lds_read_tr16(vb + 16 * DVS);
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(a_lo.x, a_lo.y, a_hi.x, a_hi.y));
      oacc[db] = mfma16(a, pf, oacc[db]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  };
  for (int s0 = c0; s0 < c1; s0 += SUB) step(s0);
  lsum = col_sum(lsum);
  if (direct) {
    // the only split of the sequence: add the sink and normalise here
    if (col < kGroup) {
      const int h = g * kGroup + col;
      const float sig = __ldg(p.sinks + h) * kLog2e;
      const float M = fmaxf(sig, m);
      const float Mu = (M == -INFINITY) ? 0.0f : M;
      const float wgt = __builtin_amdgcn_exp2f(m - Mu);
      float l = 0.0f;
      l += lsum * wgt;
      l += __builtin_amdgcn_exp2f(sig - Mu);
      bf16_t* op = p.o + (int64_t)n * p.o_sn + (int64_t)h * p.o_sh + 4 * grp;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float o = 0.0f;
          o += oacc[db][e] * wgt;
          r[e] = (l > 0.0f) ? o / l : 0.0f;
        }
        // out is only 4-byte aligned (even strides): two 32-bit stores
        uint32_t* o32 = reinterpret_cast<uint32_t*>(op + 16 * db);
        o32[0] = pack_bf16x2(r[0], r[1]);
        o32[1] = pack_bf16x2(r[2], r[3]);
      }
    }
  } else if (col < kGroup) {
    const int64_t slot = (((int64_t)n * p.num_kv_heads + g) * p.num_splits + split) * kGroup + col;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      *reinterpret_cast<f32x4_t*>(p.part_o + slot * kHeadDim + 16 * db + 4 * grp) = oacc[db];
    if (grp == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(m, lsum);
  }
  }   // work items
}

// Split planning. Every work group ends with stores of its partials, whose
// completion it waits for; thousands of small splits pay that wait thousands
// of times, a few hundred large ones leave the machine idle at the end. The
// plan kernel reads the cache lengths and picks the split length so that the
// call has about target_chunks (sequence, split) items: total visible keys /
// target_chunks, rounded up to a multiple of 128, at least min_chunk (so the
// partial buffers sized on the host always suffice). A caller-given split
// count is used as is. It then writes the list of items, the full-length
// splits first and each sequence's shorter last split after them, so the split
// kernel's work groups take real work only and the short items run last.
// plan[0] = keys per split, plan[1] = item count, plan[2..] = int2 (sequence, split).
constexpr int kPlanThreads = 256;
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodeParams p) {
  __shared__ long long part[kPlanThreads];
  __shared__ int scan_full[kPlanThreads], scan_part[kPlanThreads];
  __shared__ int chunk_s;
  const int t = threadIdx.x;
  auto eff_len = [&](int n) {
    const KeySpan r = key_span(p, n);
    return r.end - r.start;
  };
  long long total = 0;
  for (int n = t; n < p.num_seqs; n += kPlanThreads) total += eff_len(n);
  part[t] = total;
  __syncthreads();
  for (int off = kPlanThreads / 2; off > 0; off >>= 1) {
    if (t < off) part[t] += part[t + off];
    __syncthreads();
  }
  if (t == 0) {
    int chunk = p.chunk_fixed;
    if (chunk <= 0) {
      const long long want = (part[0] + p.target_chunks - 1) / max(p.target_chunks, 1);
      long long c = (want + 127) / 128 * 128;
      c = c < p.min_chunk ? p.min_chunk : c;
      const long long cap = ((long long)p.max_cache_len + 127) / 128 * 128;
      chunk = (int)(c > cap ? (cap > p.min_chunk ? cap : p.min_chunk) : c);
    }
    chunk_s = chunk;
    p.plan[0] = chunk;
  }
  __syncthreads();
  const int chunk = chunk_s;
  // thread t owns sequences [n0, n1)
  const int per = (p.num_seqs + kPlanThreads - 1) / kPlanThreads;
  const int n0 = min(t * per, p.num_seqs), n1 = min(n0 + per, p.num_seqs);
  int nf = 0, np = 0;
  for (int n = n0; n < n1; ++n) {
    const int e = eff_len(n);
    nf += e / chunk;
    np += (e % chunk) != 0;
  }
  scan_full[t] = nf;
  scan_part[t] = np;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {   // inclusive scans
    const int a = (t >= off) ? scan_full[t - off] : 0;
    const int b = (t >= off) ? scan_part[t - off] : 0;
    __syncthreads();
    scan_full[t] += a;
    scan_part[t] += b;
    __syncthreads();
  }
  const int total_full = scan_full[kPlanThreads - 1];
  int pf = scan_full[t] - nf;                 // exclusive prefix: first slot of this thread
  int pp = total_full + scan_part[t] - np;
  int2* work = reinterpret_cast<int2*>(p.plan + 2);
  for (int n = n0; n < n1; ++n) {
    const int e = eff_len(n);
    const int full = e / chunk;
    for (int s = 0; s < full; ++s) work[pf++] = make_int2(n, s);
    if (e % chunk) work[pp++] = make_int2(n, full);
  }
  if (t == kPlanThreads - 1) p.plan[1] = total_full + scan_part[kPlanThreads - 1];
}

// One wave per (sequence, query head). Splits across lanes for the max and the
// weights, then lane = head dim for the weighted sum of the partial outputs.
__global__ __launch_bounds__(NTC) void decode_combine_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * (NTC / 64) + (threadIdx.x >> 6);
  const int Hq = p.num_kv_heads * kGroup;
  if (idx >= p.num_seqs * Hq) return;
  const int n = idx / Hq;
  const int h = idx - n * Hq;
  const int g = h / kGroup, c = h - g * kGroup;
  const KeySpan span = key_span(p, n);
  const int chunk = p.direct_chunk > 0 ? p.direct_chunk : *p.plan;
  const int nsplit = min((span.end - span.start + chunk - 1) / chunk, p.num_splits);
  const float sig = __ldg(p.sinks + h) * kLog2e;
  const int64_t base = ((int64_t)n * p.num_kv_heads + g) * p.num_splits;
  float M = sig;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int s = s0 + lane;
    if (s < nsplit) M = fmaxf(M, p.part_ml[((base + s) * kGroup + c) * 2]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float Mu = (M == -INFINITY) ? 0.0f : M;
  float l = 0.0f, o = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int s = s0 + lane;
    float wgt = 0.0f;
    if (s < nsplit) {
      const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + ((base + s) * kGroup + c) * 2);
      wgt = __builtin_amdgcn_exp2f(ml.x - Mu);
      l += ml.y * wgt;
    }
    const int cnt = min(64, nsplit - s0);
    const float* po = p.part_o + ((base + s0) * kGroup + c) * kHeadDim + lane;
    int j = 0;
    for (; j + 4 <= cnt; j += 4) {
      const float a0 = po[(int64_t)(j + 0) * kGroup * kHeadDim], a1 = po[(int64_t)(j + 1) * kGroup * kHeadDim];
      const float a2 = po[(int64_t)(j + 2) * kGroup * kHeadDim], a3 = po[(int64_t)(j + 3) * kGroup * kHeadDim];
      o += a0 * __shfl(wgt, j) + a1 * __shfl(wgt, j + 1) + a2 * __shfl(wgt, j + 2) + a3 * __shfl(wgt, j + 3);
    }
    for (; j < cnt; ++j) o += po[(int64_t)j * kGroup * kHeadDim] * __shfl(wgt, j);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
  l += __builtin_amdgcn_exp2f(sig - Mu);
  const float r = (l > 0.0f) ? o / l : 0.0f;
  // two lanes per bf16 pair: even lane stores the pair
  const float r_next = __shfl_down(r, 1);
  if ((lane & 1) == 0) {
    bf16_t* op = p.o + (int64_t)n * p.o_sn + (int64_t)h * p.o_sh + lane;
    *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(r, r_next);
  }
}

// Scratch of the allocation-free decode entry point (partials and plan of one
// call), one copy per GPU, held until the process ends. Calls that overlap on
// one GPU share it and race; nothing in it needs to start at zero (the plan
// kernel writes the plan, the split kernel every partial the combine reads).
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

// Device address of `scratch` on the current device. In host code the array's
// name stands for a host-side shadow, not device memory, so kernels are handed
// this address, looked up once per device.
hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  hipError_t e;
  if (p.direct_chunk <= 0) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // one work group per planned item (at most max_items of them), looping if there are more
  dim3 grid((unsigned)p.max_items, 1, (p.num_kv_heads + NW - 1) / NW);
  const bool paged = p.kind == kCachePaged;
  if (p.table)
    hipLaunchKernelGGL((paged ? decode_split_kernel<true, true> : decode_split_kernel<true, false>), grid, dim3(NT),
                       0, stream, p);
  else
    hipLaunchKernelGGL((paged ? decode_split_kernel<false, true> : decode_split_kernel<false, false>), grid,
                       dim3(NT), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.direct_chunk > 0) return e;   // one split: the split kernel wrote o
  const int waves = p.num_seqs * p.num_kv_heads * kGroup;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((waves + 3) / 4), dim3(NTC), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gptoss
