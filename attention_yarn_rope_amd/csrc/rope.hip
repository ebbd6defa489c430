// YaRN cos/sin table and the standalone q/k rotation (gfx950).
//
// Table: page "nemo_automodel.components.models.gpt_oss.rope_utils",
// RotaryEmbedding._compute_cos_sin -- row p holds c*cos(p*omega_i) then
// c*sin(p*omega_i), the cosine and sine halves concatenated, rounded to the
// q/k dtype (_apply_rotary_emb_qk: shared dtype-rounded tables).
// Rotation: same page, _apply_rotary_emb_qk / apply_rotary_emb_qk -- q and k
// rotated with one table, out of place, BSHD or THD with positions restarting
// per packed sequence.
#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

// fp64 -> bf16, rounded once to nearest-even. The fp32 step rounds to odd
// (truncate, then set the last bit if anything was dropped); fp32 keeps
// 24 >= 8 + 2 significand bits, so the following nearest-even rounding to bf16
// gives the same result as rounding the fp64 value directly.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  float f = (float)x;
  uint32_t u = __float_as_uint(f);
  if ((double)f != x) {
    if (fabs((double)f) > fabs(x)) u -= 1u;  // step the magnitude down: truncation
    u |= 1u;
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void rope_table_kernel(TableParams p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.num_positions * p.half;
  if (idx >= total) return;
  const int32_t pos = (int32_t)(idx / p.half);
  const int32_t i = (int32_t)(idx - (int64_t)pos * p.half);
  const double angle = (double)pos * p.omega[i];
  double s, c;
  sincos(angle, &s, &c);
  uint16_t* row = p.table + (int64_t)pos * (2 * p.half);
  row[i] = f64_to_bf16(p.concentration * c);
  row[p.half + i] = f64_to_bf16(p.concentration * s);
}


// One thread per (token row, head, chunk pair cc in 0..3).
__global__ __launch_bounds__(256) void rope_qk_kernel(RopeQKParams p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)p.batch * p.tokens * p.heads;
  if (idx >= rows * 4) return;
  const int32_t cc = (int32_t)(idx & 3);
  const int64_t r = idx >> 2;
  const int32_t h = (int32_t)(r % p.heads);
  const int64_t bt = r / p.heads;
  const int32_t b = (int32_t)(bt / p.tokens);
  const int32_t t = (int32_t)(bt - (int64_t)b * p.tokens);
  int32_t pos = t + p.pos0;
  if (p.cu_seqlens) pos = t - __ldg(p.cu_seqlens + find_seq(p.cu_seqlens, p.num_seqs, t));
  pos = min(max(pos, 0), p.table_rows - 1);
  const uint16_t* x = p.x + b * p.s_b + t * p.s_t + h * p.s_h;
  rotate_row_chunks(x, p.y + r * kHeadDim, p.table + (int64_t)pos * (16 * p.rot_chunks), p.rot_chunks, cc);
}

}  // namespace

hipError_t launch_rope_table(const TableParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.num_positions * p.half;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_table_kernel, dim3((uint32_t)blocks), dim3(threads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_rope_qk(const RopeQKParams& p, hipStream_t stream) {
  const int64_t work = (int64_t)p.batch * p.tokens * p.heads * 4;
  if (work == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (work + threads - 1) / threads;
  hipLaunchKernelGGL(rope_qk_kernel, dim3((uint32_t)blocks), dim3(threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gptoss
