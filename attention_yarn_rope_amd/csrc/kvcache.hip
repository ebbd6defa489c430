// KV-cache append for the decode loop on gfx950: the newest tokens' k, rotated
// at their positions, and v are written into a contiguous, paged or ring cache.
//
// No page specifies a cache. The generation loop of the Transformers v4.55.0
// release notes ("Welcome GPT OSS", model.generate) re-reads the keys and
// values of earlier tokens at every step; the rotation is the one of page
// "nemo_automodel.components.models.gpt_oss.rope_utils" (_apply_rotary_emb_qk:
// half-split pairs, cos/sin from the shared dtype-rounded table), computed by
// the same rope8 as the standalone rotation, so a cached key is bit-identical
// to the key gptoss_rope_qk produces at that position.
#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

// One thread per (sequence, new token, KV head, chunk pair cc in 0..3): the
// 8-dim chunks cc and cc + 4 of v, and of k rotated by rotate_row_chunks (any
// rotary_dim that is a multiple of 16; the tail past it is copied). Four
// consecutive threads cover one 128-byte row.
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)p.num_seqs * p.num_new * p.num_kv_heads;
  if (idx >= rows * 4) return;
  const int cc = (int)(idx & 3);
  const int64_t r = idx >> 2;
  const int g = (int)(r % p.num_kv_heads);
  const int64_t nt = r / p.num_kv_heads;
  const int t = (int)(nt % p.num_new);
  const int n = (int)(nt / p.num_new);
  const int pos = __ldg(p.cache_seqlens + n) - p.num_new + t;
  if (pos < 0) return;
  int64_t row;
  if (p.kind == kCachePaged) {
    const int lp = pos >> p.page_log2;
    if (lp >= p.max_pages) return;
    const int pid = min(max(__ldg(p.block_table + (int64_t)n * p.max_pages + lp), 0), p.num_pages - 1);
    row = (int64_t)pid * p.c_s0 + (int64_t)(pos - (lp << p.page_log2)) * p.c_sr;
  } else if (p.kind == kCacheRing) {
    if (t < p.num_new - p.capacity) return;   // a later token of this call takes the slot
    row = (int64_t)n * p.c_s0 + (int64_t)(pos % p.capacity) * p.c_sr;
  } else {
    if (pos >= p.capacity) return;
    row = (int64_t)n * p.c_s0 + (int64_t)pos * p.c_sr;
  }
  row += (int64_t)g * p.c_sh;
  const uint16_t* kx = p.kn + (int64_t)n * p.kn_sn + (int64_t)t * p.kn_st + (int64_t)g * p.kn_sh;
  const uint16_t* vx = p.vn + (int64_t)n * p.vn_sn + (int64_t)t * p.vn_st + (int64_t)g * p.vn_sh;
  if (p.table) {
    rotate_row_chunks(kx, p.k + row, p.table + (int64_t)min(pos, p.table_rows - 1) * (16 * p.rot_chunks),
                      p.rot_chunks, cc);
  } else {
    stg16(p.k + row + 8 * cc, ldg16(kx + 8 * cc));
    stg16(p.k + row + 32 + 8 * cc, ldg16(kx + 32 + 8 * cc));
  }
  stg16(p.v + row + 8 * cc, ldg16(vx + 8 * cc));
  stg16(p.v + row + 32 + 8 * cc, ldg16(vx + 32 + 8 * cc));
}

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
  const int64_t work = (int64_t)p.num_seqs * p.num_new * p.num_kv_heads * 4;
  if (work == 0) return hipSuccess;
  const int threads = 256;
  hipLaunchKernelGGL(kv_append_kernel, dim3((uint32_t)((work + threads - 1) / threads)), dim3(threads), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace gptoss
