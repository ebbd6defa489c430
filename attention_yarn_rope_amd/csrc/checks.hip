// Check of the device-resident lengths that the attention calls trust: THD
// sequence offsets (cu_seqlens, the packed-sequence format of the rope_utils
// page's apply_rotary_emb_qk: offsets starting at 0, non-decreasing, ending at
// the token count) and decode cache lengths (1 .. the cache's rows). The
// kernels clamp every index derived from these values, so bad values cannot
// reach memory outside the buffers; this check tells a caller whether they
// hold. One work group: a bitmask of the broken rules and the first offending
// index of each array.
#include <climits>

#include "gptoss_attn.h"
#include "internal.h"

namespace gptoss {
namespace {

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void check_lengths_kernel(const int32_t* cu, int32_t batch,
                                                                      int32_t total, const int32_t* cl,
                                                                      int32_t n, int32_t max_len,
                                                                      int32_t* result) {
  __shared__ int32_t mask_s, first_cu_s, first_cl_s;
  const int t = threadIdx.x;
  if (t == 0) {
    mask_s = 0;
    first_cu_s = INT_MAX;
    first_cl_s = INT_MAX;
  }
  __syncthreads();
  int mask = 0, first_cu = INT_MAX, first_cl = INT_MAX;
  if (cu) {
    for (int i = t; i <= batch; i += kCheckThreads) {
      const int v = cu[i];
      int bad = 0;
      if (i == 0 && v != 0) bad |= GPTOSS_LEN_CU_START;
      if (i > 0 && v < cu[i - 1]) bad |= GPTOSS_LEN_CU_ORDER;
      if (i == batch && total >= 0 && v != total) bad |= GPTOSS_LEN_CU_TOTAL;
      if (bad) {
        mask |= bad;
        first_cu = min(first_cu, i);
      }
    }
  }
  if (cl) {
    for (int i = t; i < n; i += kCheckThreads) {
      const int v = cl[i];
      if (v < 1 || v > max_len) {
        mask |= GPTOSS_LEN_CACHE;
        first_cl = min(first_cl, i);
      }
    }
  }
  if (mask) {
    atomicOr(&mask_s, mask);
    atomicMin(&first_cu_s, first_cu);
    atomicMin(&first_cl_s, first_cl);
  }
  __syncthreads();
  if (t == 0) {
    result[0] = mask_s;
    result[1] = first_cu_s == INT_MAX ? -1 : first_cu_s;
    result[2] = first_cl_s == INT_MAX ? -1 : first_cl_s;
  }
}

}  // namespace

hipError_t launch_check_lengths(const int32_t* cu_seqlens, int32_t batch, int32_t total_tokens,
                                const int32_t* cache_seqlens, int32_t num_seqs, int32_t max_cache_len,
                                int32_t* result, hipStream_t stream) {
  hipLaunchKernelGGL(check_lengths_kernel, dim3(1), dim3(kCheckThreads), 0, stream, cu_seqlens, batch,
                     total_tokens, cache_seqlens, num_seqs, max_cache_len, result);
  return hipGetLastError();
}

}  // namespace gptoss
