// Split-KV decode attention for GPT-OSS on gfx950: one new query token per
// sequence against a bf16 KV cache, with the per-head sink, GQA and the
// causal / sliding-window mask of prefill (page
// "nemo_automodel.components.models.gpt_oss.layers", GptOssAttention;
// Transformers v4.55.0 release notes, "Architecture").
//
// Split kernel: one work group per (key chunk, sequence, group of 8 KV heads);
// wave w takes KV head w, so the group streams whole 1 KB cache rows (8 heads
// x 128 B) and each K/V row of a head is read from HBM exactly once for the 8
// query heads that share it. Rows are fetched in full 128 B lines with
// non-temporal loads (read-once data), 32 keys per step, the next step's loads
// in flight while the current one computes. K and V pass through one per-wave
// LDS block: K is read back as MFMA A fragments for S^T = K Q^T
// (v_mfma_f32_16x16x32_bf16, 8 heads padded to 16 columns), V transposed with
// ds_read_b64_tr_b16 for O^T = V^T P^T. Exact online softmax per step; each
// wave writes one unnormalised partial (m, l, acc[64]) per query head.
// Combine kernel: per (sequence, query head) it merges the partials and adds
// the sink exactly once: M = max(sigma, m_s), l = exp(sigma - M) + sum l_s
// exp(m_s - M), o = sum acc_s exp(m_s - M) / l (all in log2 units).
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

// 16-byte non-temporal load (global_load_dwordx4 ... nt): streamed once, kept out of the caches
__device__ __forceinline__ uint4 ldg16_nt(const bf16_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool ROTQ>
__global__ __launch_bounds__(NT) void decode_split_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t lds_v[NW][SUB * DVS];

  const int split = blockIdx.x;
  const int n = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.z * NW + wave;
  const int col = lane & 15, grp = lane >> 4;
  if (g >= p.num_kv_heads) return;

  const int L = min(max(__ldg(p.cache_seqlens + n), 0), p.max_cache_len);
  const int lo = (p.window > 0) ? max(0, L - p.window) : 0;
  const int nsplit = (L - lo + p.chunk - 1) / p.chunk;
  if (split >= nsplit) return;
  const int c0 = lo + split * p.chunk;
  const int c1 = min(c0 + p.chunk, L);
  const float sl = p.scale_log2;

  bf16x8_t qf[2];
  {
    uint4 y1 = make_uint4(0, 0, 0, 0), y2 = make_uint4(0, 0, 0, 0);
    if (col < kGroup) {
      const bf16_t* qp = p.q + (int64_t)n * p.q_sn + (int64_t)(g * kGroup + col) * p.q_sh;
      uint4 x1 = ldg16(qp + 8 * grp), x2 = ldg16(qp + 32 + 8 * grp);
      if (ROTQ) {
        const bf16_t* tp = p.table + (int64_t)min(max(L - 1, 0), p.table_rows - 1) * kHeadDim + 8 * grp;
        rope8(x1, x2, ldg16(tp), ldg16(tp + 32), y1, y2);
      } else {
        y1 = x1; y2 = x2;
      }
    }
    qf[0] = as_bf16x8(y1);
    qf[1] = as_bf16x8(y2);
  }

  const bf16_t* kbase = p.k + (int64_t)n * p.kv_sn + (int64_t)g * p.kv_sh;
  const bf16_t* vbase = p.v + (int64_t)n * p.kv_sn + (int64_t)g * p.kv_sh;
  bf16_t* vl = lds_v[wave];

  float m = -INFINITY, lsum = 0.0f;
  f32x4_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 kr[4], vr[4];
  auto load_block = [&](int s0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = s0 + (lane >> 3) + 8 * i;
      kr[i] = make_uint4(0, 0, 0, 0);
      vr[i] = make_uint4(0, 0, 0, 0);
      if (key < c1) {
        kr[i] = ldg16_nt(kbase + (int64_t)key * p.kv_sp + 8 * (lane & 7));
        vr[i] = ldg16_nt(vbase + (int64_t)key * p.kv_sp + 8 * (lane & 7));
      }
    }
  };
  if (c0 < c1) load_block(c0);
  for (int s0 = c0; s0 < c1; s0 += SUB) {
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
    // V rows -> the same LDS block (the K fragments are in registers now), read back transposed
    // below; the staging registers are then free for the next step's loads
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
        sacc[kb][r] = (key < c1) ? sacc[kb][r] : -INFINITY;
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
  }
  lsum = col_sum(lsum);
  if (col < kGroup) {
    const int64_t slot = (((int64_t)n * p.num_kv_heads + g) * p.num_splits + split) * kGroup + col;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      *reinterpret_cast<f32x4_t*>(p.part_o + slot * kHeadDim + 16 * db + 4 * grp) = oacc[db];
    if (grp == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(m, lsum);
  }
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
  const int L = min(max(__ldg(p.cache_seqlens + n), 0), p.max_cache_len);
  const int lo = (p.window > 0) ? max(0, L - p.window) : 0;
  const int nsplit = min((L - lo + p.chunk - 1) / p.chunk, p.num_splits);
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

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  dim3 grid(p.num_splits, p.num_seqs, (p.num_kv_heads + NW - 1) / NW);
  if (p.table)
    hipLaunchKernelGGL(decode_split_kernel<true>, grid, dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_split_kernel<false>, grid, dim3(NT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = p.num_seqs * p.num_kv_heads * kGroup;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((waves + 3) / 4), dim3(NTC), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gptoss
