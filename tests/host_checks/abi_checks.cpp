// Host-only driver of the C ABI's argument checks and host computations, built
// with AddressSanitizer and UndefinedBehaviorSanitizer together with api.cpp
// and launch_stubs.cpp (no GPU code). Every call below must return before any
// launch (the stubs abort if one is reached) with the status the header
// documents; pointers are fake, non-NULL and never dereferenced by the checks.
// Exit status 0 when every expectation holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "gptoss_attn.h"

static int failures = 0;
static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    std::fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", line, what, got, want, gptoss_last_error());
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

static void* const P = reinterpret_cast<void*>(0x100000);   // aligned fake device pointer
static const int32_t* const PI = reinterpret_cast<const int32_t*>(0x100000);
static const float* const PF = reinterpret_cast<const float*>(0x100000);

static gptoss_rope_config cfg(int rd = 64) {
  gptoss_rope_config c;
  c.head_dim = 64; c.rotary_dim = rd; c.base = 150000.0; c.scaling_factor = 32.0;
  c.initial_context_length = 4096; c.ntk_alpha = 1.0; c.ntk_beta = 32.0;
  return c;
}
static gptoss_seq_desc desc(int layout = GPTOSS_BSHD, int b = 2, int s = 128, int hq = 64, int hkv = 8, int d = 64,
                            const int32_t* cu = nullptr, int max_s = -1) {
  gptoss_seq_desc x;
  x.layout = layout; x.batch = b; x.seqlen = s; x.max_seqlen = max_s < 0 ? s : max_s; x.cu_seqlens = cu;
  x.num_q_heads = hq; x.num_kv_heads = hkv; x.head_dim = d;
  return x;
}

int main() {
  // ---- host computations: YaRN parameters, sizes, status strings ----
  double omega[32], conc = 0;
  for (int rd : {16, 32, 48, 64}) {
    gptoss_rope_config c = cfg(rd);
    EXPECT(gptoss_yarn_params(&c, omega, &conc), GPTOSS_OK);
    for (int i = 0; i < rd / 2; ++i)
      if (!(omega[i] > 0.0) || !std::isfinite(omega[i])) { std::fprintf(stderr, "omega[%d] = %g\n", i, omega[i]); ++failures; }
  }
  gptoss_rope_config bad = cfg(63);
  EXPECT(gptoss_yarn_params(&bad, omega, &conc), GPTOSS_ERR_SHAPE);
  bad = cfg(); bad.base = 0.5;
  EXPECT(gptoss_yarn_params(&bad, omega, &conc), GPTOSS_ERR_SHAPE);
  EXPECT(gptoss_yarn_params(nullptr, omega, &conc), GPTOSS_ERR_NULL);
  for (int code = -1; code < 8; ++code)
    if (!gptoss_status_string(code) || !std::strlen(gptoss_status_string(code))) ++failures;
  gptoss_seq_desc d = desc();
  size_t ws = gptoss_attn_prefill_workspace_size(&d);
  if (ws == 0) ++failures;
  gptoss_seq_desc t = desc(GPTOSS_THD, 16, 65171, 64, 8, 64, PI, 8192);
  if (gptoss_attn_prefill_workspace_size(&t) <= gptoss_attn_prefill_workspace_size(&d)) ++failures;
  if (gptoss_attn_prefill_backward_workspace_size(&t) == 0) ++failures;
  if (gptoss_attn_prefill_shard_workspace_size(&d, 4096) == 0) ++failures;
  if (gptoss_attn_decode_workspace_size(64, 64, 32768, 0) == 0) ++failures;
  if (gptoss_attn_decode_workspace_size(1 << 20, 64, 1 << 20, 0) == 0) ++failures;   // large sizes: no overflow trap
  EXPECT((int)gptoss_attn_decode_workspace_size(-1, 64, 100, 0), 0);
  gptoss_seq_desc huge = desc(GPTOSS_BSHD, 1 << 20, 1 << 20);
  (void)gptoss_attn_prefill_workspace_size(&huge);
  (void)gptoss_attn_prefill_backward_workspace_size(&huge);

  // ---- rope table / rope_qk ----
  gptoss_rope_config c = cfg();
  EXPECT(gptoss_rope_table_init(nullptr, 16, P, nullptr), GPTOSS_ERR_NULL);
  EXPECT(gptoss_rope_table_init(&c, 0, P, nullptr), GPTOSS_ERR_SHAPE);
  EXPECT(gptoss_rope_table_init(&c, 16, nullptr, nullptr), GPTOSS_ERR_NULL);
  const int64_t q3[3] = {128 * 64 * 64, 64 * 64, 64}, k3[3] = {128 * 8 * 64, 8 * 64, 64};
  EXPECT(gptoss_rope_qk(nullptr, P, q3, P, k3, P, P, P, 128, 64, nullptr), GPTOSS_ERR_NULL);
  EXPECT(gptoss_rope_qk(&d, P, q3, P, k3, P, P, P, 100, 64, nullptr), GPTOSS_ERR_SHAPE);   // table too short
  EXPECT(gptoss_rope_qk(&d, P, q3, P, k3, P, P, P, 128, 24, nullptr), GPTOSS_ERR_UNSUPPORTED);

  // ---- prefill ----
  EXPECT(gptoss_attn_prefill(nullptr, P, q3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 64, P, q3, P, ws, nullptr),
         GPTOSS_ERR_NULL);
  gptoss_seq_desc d128 = desc(GPTOSS_BSHD, 2, 128, 64, 8, 128);
  EXPECT(gptoss_attn_prefill(&d128, P, q3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 64, P, q3, P, ws, nullptr),
         GPTOSS_ERR_UNSUPPORTED);
  EXPECT(gptoss_attn_prefill(&d, P, q3, P, k3, P, k3, PF, 0.125f, -1, P, 128, 64, P, q3, P, ws, nullptr),
         GPTOSS_ERR_SHAPE);
  EXPECT(gptoss_attn_prefill(&d, P, q3, P, k3, P, k3, PF, NAN, 0, P, 128, 64, P, q3, P, ws, nullptr),
         GPTOSS_ERR_SHAPE);
  EXPECT(gptoss_attn_prefill(&d, P, q3, P, k3, P, k3, PF, -1.0f, 0, P, 128, 64, P, q3, P, ws, nullptr),
         GPTOSS_ERR_SHAPE);
  EXPECT(gptoss_attn_prefill(&d, P, q3, P, k3, P, k3, PF, 0.0f, 0, P, 128, 64, P, q3, P, 16, nullptr),
         GPTOSS_ERR_WORKSPACE);   // scale 0 = head_dim ** -0.5 passes; the workspace does not
  EXPECT(gptoss_attn_prefill(&d, P, q3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 24, P, q3, P, ws, nullptr),
         GPTOSS_ERR_UNSUPPORTED);
  EXPECT(gptoss_attn_prefill(&d, P, q3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 32, P, q3, P, 16, nullptr),
         GPTOSS_ERR_WORKSPACE);   // partial rotary passes the table check
  const int64_t bad3[3] = {128 * 64 * 64, 64 * 64, 65};
  EXPECT(gptoss_attn_prefill(&d, P, bad3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 64, P, q3, P, ws, nullptr),
         GPTOSS_ERR_UNSUPPORTED);
  gptoss_seq_desc nocu = desc(GPTOSS_THD, 2, 100, 64, 8, 64, nullptr, 50);
  EXPECT(gptoss_attn_prefill(&nocu, P, q3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 64, P, q3, P, ws, nullptr),
         GPTOSS_ERR_NULL);
  EXPECT(gptoss_attn_prefill_ex(&d, P, q3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 64, P, q3, P, ws, 9, nullptr),
         GPTOSS_ERR_SHAPE);
  EXPECT(gptoss_attn_prefill_lse(&d, P, q3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 64, P, q3, nullptr, P, ws, nullptr),
         GPTOSS_ERR_NULL);
  EXPECT(gptoss_attn_prefill_shard(&d, P, q3, P, k3, P, k3, -1, 0, 0, 0.125f, 0, P, 4096, 64, P, q3,
                                   (float*)P, P, ws, nullptr), GPTOSS_ERR_SHAPE);
  EXPECT(gptoss_attn_prefill_shard(&d, P, q3, P, k3, P, k3, 128, 0x7fffff00, 0, 0.125f, 0, P, 4096, 64, P, q3,
                                   (float*)P, P, ws, nullptr), GPTOSS_ERR_SHAPE);

  // ---- backward ----
  size_t bws = gptoss_attn_prefill_backward_workspace_size(&d);
  EXPECT(gptoss_attn_prefill_backward(&d, P, q3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 64, P, q3, P, q3, PF,
                                      P, P, P, nullptr, P, bws, nullptr), GPTOSS_ERR_NULL);
  EXPECT(gptoss_attn_prefill_backward(&d, P, q3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 32, P, q3, P, q3, PF,
                                      P, P, P, (float*)P, P, bws, nullptr), GPTOSS_ERR_UNSUPPORTED);
  EXPECT(gptoss_attn_prefill_backward(&d, P, q3, P, k3, P, k3, PF, 0.125f, 0, P, 128, 64, P, q3, P, q3, PF,
                                      P, P, P, (float*)P, P, 16, nullptr), GPTOSS_ERR_WORKSPACE);

  // ---- decode ----
  const int64_t q2[2] = {64 * 64, 64}, kv3[3] = {1024 * 8 * 64, 8 * 64, 64};
  size_t dws = gptoss_attn_decode_workspace_size(4, 64, 1024, 0);
  EXPECT(gptoss_attn_decode(4, 64, 8, 64, P, q2, P, P, kv3, PI, 1024, PF, 0.125f, 0, P, 1024, 64, P, q2, P, 16, 0,
                            nullptr), GPTOSS_ERR_WORKSPACE);
  EXPECT(gptoss_attn_decode(4, 60, 8, 64, P, q2, P, P, kv3, PI, 1024, PF, 0.125f, 0, P, 1024, 64, P, q2, P, dws, 0,
                            nullptr), GPTOSS_ERR_UNSUPPORTED);
  EXPECT(gptoss_attn_decode(4, 64, 8, 64, P, q2, P, P, kv3, PI, 0, PF, 0.125f, 0, P, 1024, 64, P, q2, P, dws, 0,
                            nullptr), GPTOSS_ERR_SHAPE);
  EXPECT(gptoss_attn_decode(4, 64, 8, 64, P, q2, P, P, kv3, PI, 1024, PF, 0.125f, 0, P, 1024, 8, P, q2, P, dws, 0,
                            nullptr), GPTOSS_ERR_UNSUPPORTED);
  gptoss_kv_layout lay;
  std::memset(&lay, 0, sizeof lay);
  lay.kind = GPTOSS_CACHE_PAGED; lay.capacity = 64; lay.strides[0] = 64 * 8 * 64; lay.strides[1] = 8 * 64;
  lay.strides[2] = 64; lay.block_table = PI; lay.max_pages = 8; lay.num_pages = 100;
  EXPECT(gptoss_attn_decode_kv(&lay, 4, 64, 8, 64, P, q2, P, P, PI, 1024, PF, 0.125f, 0, P, 1024, 64, P, q2, P,
                               dws, 0, nullptr), GPTOSS_ERR_SHAPE);   // 8 pages x 64 rows < 1024
  EXPECT(gptoss_attn_decode_kv(&lay, 4, 64, 8, 64, P, q2, P, P, PI, 512, PF, 0.125f, 0, P, 1024, 64, P, q2, P,
                               16, 0, nullptr), GPTOSS_ERR_WORKSPACE);
  lay.kind = GPTOSS_CACHE_RING; lay.capacity = 128; lay.block_table = nullptr;
  EXPECT(gptoss_attn_decode_kv(&lay, 4, 64, 8, 64, P, q2, P, P, PI, 512, PF, 0.125f, 64, P, 1024, 64, P, q2, P,
                               dws, 0, nullptr), GPTOSS_ERR_UNSUPPORTED);   // ring needs window == capacity
  lay.kind = GPTOSS_CACHE_CONTIGUOUS; lay.capacity = 1;
  EXPECT(gptoss_attn_decode_kv_noalloc(&lay, 2048, 64, 8, 64, P, q2, P, P, PI, 1, PF, 0.125f, 0, P, 1, 64, P, q2,
                                       0, nullptr), GPTOSS_ERR_WORKSPACE);   // partials beyond the scratch
  EXPECT(gptoss_attn_decode_kv_noalloc(nullptr, 4, 64, 8, 64, P, q2, P, P, PI, 1, PF, 0.125f, 0, P, 1, 64, P, q2,
                                       0, nullptr), GPTOSS_ERR_NULL);

  // ---- KV append, merge, projection ----
  const int64_t kn3[3] = {8 * 8 * 64, 8 * 64, 64};
  lay.capacity = 1024;
  EXPECT(gptoss_kv_append(&lay, P, P, 4, 8, 64, 8, nullptr, kn3, P, kn3, PI, 1024, P, 1024, 64, nullptr),
         GPTOSS_ERR_NULL);
  EXPECT(gptoss_kv_append(&lay, P, P, 4, 8, 64, 8, P, kn3, P, kn3, PI, 1024, P, 100, 64, nullptr),
         GPTOSS_ERR_SHAPE);
  const int64_t p4[4] = {128 * 64 * 64, 64 * 64, 64, 1};
  EXPECT(gptoss_attn_merge(2, 128, 64, 128, P, p4, PF, PF, P, q2, nullptr, nullptr), GPTOSS_ERR_UNSUPPORTED);
  EXPECT(gptoss_attn_merge(2, 128, 64, 64, nullptr, p4, PF, PF, P, q2, nullptr, nullptr), GPTOSS_ERR_NULL);
  EXPECT(gptoss_attn_merge(2, 0, 64, 64, P, p4, PF, PF, P, q2, nullptr, nullptr), GPTOSS_OK);   // nothing to do
  EXPECT(gptoss_qkv_proj_rope(&d, P, 2880, 2880, P, P, P, P, P, P, P, 4096, 48, P, P, P, nullptr),
         GPTOSS_ERR_UNSUPPORTED);
  EXPECT(gptoss_qkv_proj_rope(&d, P, 2880, 2890, P, P, P, P, P, P, P, 4096, 64, P, P, P, nullptr),
         GPTOSS_ERR_UNSUPPORTED);

  // ---- check of device-resident lengths ----
  int32_t* const PR = reinterpret_cast<int32_t*>(0x100000);
  EXPECT(gptoss_check_lengths(PI, 4, 100, PI, 4, 1024, nullptr, nullptr), GPTOSS_ERR_NULL);
  EXPECT(gptoss_check_lengths(PI, -1, 100, nullptr, 0, 0, PR, nullptr), GPTOSS_ERR_SHAPE);
  EXPECT(gptoss_check_lengths(nullptr, 0, -1, PI, -2, 1024, PR, nullptr), GPTOSS_ERR_SHAPE);
  EXPECT(gptoss_check_lengths(nullptr, 0, -1, PI, 4, 0, PR, nullptr), GPTOSS_ERR_SHAPE);

  if (failures) std::fprintf(stderr, "%d expectation(s) failed\n", failures);
  else std::printf("all argument checks behaved as documented\n");
  return failures ? 1 : 0;
}
