// Merge of partial attention outputs computed over disjoint sets of keys (the
// shards of a context-parallel prefill, or the splits of a decode), adding the
// per-head sink once (page "nemo_automodel.components.models.gpt_oss.layers",
// GptOssAttention: the sink is one more term of the softmax denominator).
//
// Part p of a row holds o_p = sum_j e^{s_j - lse_p} v_j over its keys and
// lse_p = log sum_j e^{s_j} (-inf when it has none). With the sink logit sigma:
//   lse = log(e^sigma + sum_p e^{lse_p}),   o = sum_p e^{lse_p - lse} o_p,
// which is the attention over all the parts' keys. One wave per (token, head);
// lane = head dimension.
#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // token * Hq + head
  if (row >= (int64_t)p.tokens * p.num_q_heads) return;
  const int64_t t = row / p.num_q_heads;
  const int h = (int)(row - t * p.num_q_heads);
  const float sig = p.sinks ? __ldg(p.sinks + h) * kLog2e : -INFINITY;
  float M = sig;
  for (int q = 0; q < p.parts; ++q) M = fmaxf(M, __ldg(p.lse + q * p.l_sp + row) * kLog2e);
  const float Mu = (M == -INFINITY) ? 0.0f : M;
  float z = __builtin_amdgcn_exp2f(sig - Mu), acc = 0.0f;
  for (int q = 0; q < p.parts; ++q) {
    const float w = __builtin_amdgcn_exp2f(__ldg(p.lse + q * p.l_sp + row) * kLog2e - Mu);
    const uint16_t* o = p.o + q * p.o_sp + t * p.o_st + (int64_t)h * p.o_sh;
    z += w;
    acc += w * bf16_lo((uint32_t)o[lane]);
  }
  const float r = (z > 0.0f) ? acc / z : 0.0f;
  const float r_next = __shfl_down(r, 1);
  if ((lane & 1) == 0)
    *reinterpret_cast<uint32_t*>(p.out + t * p.out_st + (int64_t)h * p.out_sh + lane) = pack_bf16x2(r, r_next);
  if (p.lse_out && lane == 0) p.lse_out[row] = (z > 0.0f) ? (Mu + __builtin_amdgcn_logf(z)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.tokens * p.num_q_heads;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((uint32_t)((rows + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gptoss
