// Stand-ins for the kernel launchers and the HIP queries the C ABI calls after
// its argument checks, for a host-only build of api.cpp (no GPU code). Reaching
// any of them means a call got past its checks: the program aborts.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "internal.h"

namespace {
[[noreturn]] void reached(const char* what) {
  std::fprintf(stderr, "launch path reached: %s\n", what);
  std::abort();
}
}  // namespace

namespace gptoss {
hipError_t launch_rope_table(const TableParams&, hipStream_t) { reached("launch_rope_table"); }
hipError_t launch_rope_qk(const RopeQKParams&, hipStream_t) { reached("launch_rope_qk"); }
hipError_t launch_prefill(const PrefillParams&, bool, int, hipStream_t) { reached("launch_prefill"); }
hipError_t launch_window_runs(const PrefillParams&, bool, hipStream_t) { reached("launch_window_runs"); }
hipError_t launch_thd_schedule(const int32_t*, int32_t, int32_t, int32_t, int2*, int32_t*, hipStream_t) {
  reached("launch_thd_schedule");
}
hipError_t launch_backward(const BackwardParams&, bool, hipStream_t) { reached("launch_backward"); }
hipError_t launch_fill_f32(float*, int32_t, float, hipStream_t) { reached("launch_fill_f32"); }
hipError_t launch_decode(const DecodeParams&, hipStream_t) { reached("launch_decode"); }
hipError_t launch_qkv_proj(const ProjParams&, hipStream_t) { reached("launch_qkv_proj"); }
hipError_t launch_merge(const MergeParams&, hipStream_t) { reached("launch_merge"); }
hipError_t launch_kv_append(const AppendParams&, hipStream_t) { reached("launch_kv_append"); }
hipError_t launch_check_lengths(const int32_t*, int32_t, int32_t, const int32_t*, int32_t, int32_t, int32_t*,
                                hipStream_t) {
  reached("launch_check_lengths");
}
hipError_t static_scratch(void**) { reached("static_scratch"); }
}  // namespace gptoss

extern "C" {
const char* hipGetErrorString(hipError_t) { return "hip error (host-only build)"; }
hipError_t hipGetDevice(int*) { reached("hipGetDevice"); }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { reached("hipDeviceGetAttribute"); }
}
