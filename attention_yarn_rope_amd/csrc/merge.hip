// Merge of partial attention outputs computed over disjoint sets of keys (the
// shards of a context-parallel prefill, or the splits of a decode), adding the
// per-head sink once (page "nemo_automodel.components.models.gpt_oss.layers",
// GptOssAttention: the sink is one more term of the softmax denominator).
//
// Part p of a row holds o_p = sum_j e^{s_j - lse_p} v_j over its keys and
// lse_p = log sum_j e^{s_j} (-inf when it has none). With the sink logit sigma:
//   lse = log(e^sigma + sum_p e^{lse_p}),   o = sum_p e^{lse_p - lse} o_p,
// which is the attention over all the parts' keys.
#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

constexpr int kPartBatch = 8;   // parts whose loads are in flight together

// 8 lanes per (token, head) row, 8 dims (16 bytes) each: a wave merges 8 rows.
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);   // token * Hq + head
  const int c = lane & 7;                                              // dims 8c .. 8c + 7
  if (row >= (int64_t)p.tokens * p.num_q_heads) return;
  const int64_t t = row / p.num_q_heads;
  const int h = (int)(row - t * p.num_q_heads);
  const float sig = p.sinks ? __ldg(p.sinks + h) * kLog2e : -INFINITY;
  // the running maximum M moves only with a larger part (then z and acc are rescaled), so
  // parts can be taken a batch at a time with every load of the batch issued first
  float M = sig, z = 0.0f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  const uint16_t* obase = p.o + t * p.o_st + (int64_t)h * p.o_sh + 8 * c;
  for (int q0 = 0; q0 < p.parts; q0 += kPartBatch) {
    float l2[kPartBatch];
    uint4 ov[kPartBatch];
#pragma unroll
    for (int i = 0; i < kPartBatch; ++i) {
      const int q = min(q0 + i, p.parts - 1);   // past the last part: load it again, weight 0 below
      l2[i] = (q0 + i < p.parts) ? __ldg(p.lse + q * p.l_sp + row) * kLog2e : -INFINITY;
      ov[i] = *reinterpret_cast<const uint4*>(obase + q * p.o_sp);
    }
    float mb = M;
#pragma unroll
    for (int i = 0; i < kPartBatch; ++i) mb = fmaxf(mb, l2[i]);
    const float mu = (mb == -INFINITY) ? 0.0f : mb;
    const float f = __builtin_amdgcn_exp2f(M - mu);   // rescale what was summed so far (M <= mb)
    z *= f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= f;
#pragma unroll
    for (int i = 0; i < kPartBatch; ++i) {
      const float w = __builtin_amdgcn_exp2f(l2[i] - mu);
      z += w;
      const uint32_t* pw = reinterpret_cast<const uint32_t*>(&ov[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += w * bf16_lo(pw[e]);
        acc[2 * e + 1] += w * bf16_hi(pw[e]);
      }
    }
    M = mb;
  }
  const float Mu = (M == -INFINITY) ? 0.0f : M;
  z += __builtin_amdgcn_exp2f(sig - Mu);
  const float rz = (z > 0.0f) ? 1.0f / z : 0.0f;
  uint4 y;
  y.x = pack_bf16x2(acc[0] * rz, acc[1] * rz);
  y.y = pack_bf16x2(acc[2] * rz, acc[3] * rz);
  y.z = pack_bf16x2(acc[4] * rz, acc[5] * rz);
  y.w = pack_bf16x2(acc[6] * rz, acc[7] * rz);
  *reinterpret_cast<uint4*>(p.out + t * p.out_st + (int64_t)h * p.out_sh + 8 * c) = y;
  if (p.lse_out && c == 0) p.lse_out[row] = (z > 0.0f) ? (Mu + __builtin_amdgcn_logf(z)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.tokens * p.num_q_heads;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((uint32_t)((rows + 31) / 32)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gptoss
