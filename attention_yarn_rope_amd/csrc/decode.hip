// Split-KV decode attention for GPT-OSS on gfx950: one new query token per
// sequence against a bf16 KV cache, with the per-head sink, GQA and the
// causal / sliding-window mask of prefill (page
// "nemo_automodel.components.models.gpt_oss.layers", GptOssAttention;
// Transformers v4.55.0 release notes, "Architecture").
//
// Split kernel: one work group per (key chunk, KV head, sequence). The 8 query
// heads of the KV head's group share every K/V row, which is streamed from HBM
// exactly once: K goes straight from global memory into the MFMA A operand
// (16 B per lane), V is staged through LDS and read transposed with
// ds_read_b64_tr_b16. Each wave covers a quarter of the chunk in blocks of 32
// keys with an exact online softmax; the 4 waves merge in LDS and write one
// unnormalised partial (m, l, acc[64]) per query head.
// Combine kernel: per (sequence, query head) it merges the partials and adds
// the sink exactly once: M = max(sigma, m_s), l = exp(sigma - M) + sum l_s
// exp(m_s - M), o = sum acc_s exp(m_s - M) / l (all in log2 units).
#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

constexpr int NT = 256;
constexpr int SUB = 32;     // keys per wave step
constexpr int DVS = 80;     // LDS row stride of a wave's V block (160 B)

template <bool ROTQ>
__global__ __launch_bounds__(NT) void decode_split_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t lds_v[4][SUB * DVS];
  __shared__ float red_m[4][8];
  __shared__ float red_l[4][8];
  __shared__ float red_o[4][8][kHeadDim];

  const int g = blockIdx.x;       // KV heads fastest: the 8 groups reading the same cache rows run together
  const int split = blockIdx.y;
  const int n = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;

  const int L = min(max(__ldg(p.cache_seqlens + n), 0), p.max_cache_len);
  const int lo = (p.window > 0) ? max(0, L - p.window) : 0;
  const int nsplit = (L - lo + p.chunk - 1) / p.chunk;
  if (split >= nsplit) return;
  const int c0 = lo + split * p.chunk;
  const int c1 = min(c0 + p.chunk, L);
  const int per_wave = p.chunk / 4;
  const int w0 = c0 + wave * per_wave;
  const float sl = p.scale_log2;

  // q fragment (B operand): column col = query head 8g + col for col < 8
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

  // K (A operand: rows = keys, k = d) and V rows for the 32 keys at s0; rows
  // at or beyond c1 read as zero
  bf16x8_t ka[2][2];
  uint4 vr[4];
  auto load_block = [&](int s0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = s0 + kb * 16 + col;
      uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
      if (key < c1) {
        const bf16_t* kp = kbase + (int64_t)key * p.kv_sp + 8 * grp;
        a0 = ldg16(kp);
        a1 = ldg16(kp + 32);
      }
      ka[kb][0] = as_bf16x8(a0);
      ka[kb][1] = as_bf16x8(a1);
    }
    // V rows s0 .. s0+31: lane -> rows (lane>>3) + 8i, 16 B chunk lane&7
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = s0 + (lane >> 3) + 8 * i;
      vr[i] = make_uint4(0, 0, 0, 0);
      if (key < c1) vr[i] = ldg16(vbase + (int64_t)key * p.kv_sp + 8 * (lane & 7));
    }
  };
  const int w1 = min(w0 + per_wave, c1);   // this wave's keys: [w0, w1)
  if (w0 < w1) load_block(w0);
  for (int s0 = w0; s0 < w1; s0 += SUB) {
    const bf16x8_t k00 = ka[0][0], k01 = ka[0][1], k10 = ka[1][0], k11 = ka[1][1];
    const uint4 v0 = vr[0], v1 = vr[1], v2 = vr[2], v3 = vr[3];
    if (s0 + SUB < w1) load_block(s0 + SUB);   // next block in flight during this one
    f32x4_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      z = mfma16(kb ? k10 : k00, qf[0], z);
      sacc[kb] = mfma16(kb ? k11 : k01, qf[1], z);
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
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx * sl);
    const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
    const float f = __builtin_amdgcn_exp2f(m - mu);   // m = -inf -> 0
    uint32_t w[4];
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][0], sl, -mu));
      float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][1], sl, -mu));
      float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][2], sl, -mu));
      float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][3], sl, -mu));
      w[2 * kb] = pack_bf16x2(e0, e1);
      w[2 * kb + 1] = pack_bf16x2(e2, e3);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) psum = add_bf16x2(w[i], psum);
    lsum = lsum * f + psum;
    m = mnew;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= f;
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));

    *reinterpret_cast<uint4*>(vl + ((lane >> 3) + 0) * DVS + 8 * (lane & 7)) = v0;
    *reinterpret_cast<uint4*>(vl + ((lane >> 3) + 8) * DVS + 8 * (lane & 7)) = v1;
    *reinterpret_cast<uint4*>(vl + ((lane >> 3) + 16) * DVS + 8 * (lane & 7)) = v2;
    *reinterpret_cast<uint4*>(vl + ((lane >> 3) + 24) * DVS + 8 * (lane & 7)) = v3;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
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
    __builtin_amdgcn_wave_barrier();   // reads done before the next step overwrites the block
  }

  // ---- merge the 4 waves ----
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (col < kGroup) {
    if (grp == 0) {
      red_m[wave][col] = m;
      red_l[wave][col] = lsum;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[wave][col][16 * db + 4 * grp + r] = oacc[db][r];
  }
  __syncthreads();
  // thread -> (head c, two dims)
  const int c = tid >> 5;
  const int d0 = 2 * (tid & 31);
  float M = -INFINITY;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) M = fmaxf(M, red_m[w2][c]);
  const float Mu = (M == -INFINITY) ? 0.0f : M;
  float lt = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    const float f = __builtin_amdgcn_exp2f(red_m[w2][c] - Mu);
    lt += red_l[w2][c] * f;
    o0 += red_o[w2][c][d0] * f;
    o1 += red_o[w2][c][d0 + 1] * f;
  }
  const int64_t slot = (((int64_t)n * p.num_kv_heads + g) * p.num_splits + split) * kGroup + c;
  *reinterpret_cast<float2*>(p.part_o + slot * kHeadDim + d0) = make_float2(o0, o1);
  if ((tid & 31) == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(M, lt);
}

// One wave per (sequence, query head). Splits across lanes for the max and the
// weights, then lane = head dim for the weighted sum of the partial outputs.
__global__ __launch_bounds__(NT) void decode_combine_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
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
  dim3 grid(p.num_kv_heads, p.num_splits, p.num_seqs);
  if (p.table)
    hipLaunchKernelGGL(decode_split_kernel<true>, grid, dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_split_kernel<false>, grid, dim3(NT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = p.num_seqs * p.num_kv_heads * kGroup;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((waves + 3) / 4), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gptoss
