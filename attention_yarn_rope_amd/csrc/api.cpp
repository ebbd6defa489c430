// C ABI of the GPT-OSS attention library: argument checks, YaRN parameters on
// the host, workspace sizing and kernel dispatch. Declared in gptoss_attn.h.
#include "gptoss_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "internal.h"

using namespace gptoss;

namespace {

thread_local std::string g_last_error;

gptoss_status fail(gptoss_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gptoss_status fail(gptoss_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

gptoss_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return GPTOSS_OK;
  return fail(GPTOSS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool strides_ok(const int64_t* s, int n) {
  for (int i = 0; i < n; ++i)
    if (s[i] < 0 || (s[i] & 7) != 0) return false;
  return true;
}
constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Compute units of the current device (256 if the query fails).
int32_t device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

// The scale of the scores (page "nemo_automodel.components.models.gpt_oss.layers",
// GptOssAttention.softmax_scale = head_dim ** -0.5): 0 selects that default,
// any other value must be finite and positive. Returns false for an invalid one.
bool resolve_scale(float& scale, int32_t head_dim) {
  if (scale == 0.0f) {
    scale = 1.0f / std::sqrt((float)head_dim);   // 0.125 exactly for head_dim 64
    return true;
  }
  return scale > 0.0f && std::isfinite(scale);
}

// YaRN (page "nemo_automodel.components.models.gpt_oss.rope_utils",
// RotaryEmbedding._compute_concentration_and_inv_freq): theta_i =
// base^(-2i/d); with s > 1 the ramp gamma_i = clamp((i - lo) / (hi - lo), 0, 1)
// between lo = (d/2) ln(L0 / (2 pi beta_fast)) / ln(base) and
// hi = (d/2) ln(L0 / (2 pi beta_slow)) / ln(base) blends theta_i (gamma = 0)
// into theta_i / s (gamma = 1); concentration 0.1 ln(s) + 1.
gptoss_status yarn(const gptoss_rope_config* cfg, double* omega, double* conc) {
  if (!cfg) return fail(GPTOSS_ERR_NULL, "rope config is NULL");
  const int d = cfg->rotary_dim;
  if (d <= 0 || (d & 1) || d > cfg->head_dim || d / 2 > kMaxPairs)
    return fail(GPTOSS_ERR_SHAPE, "rotary_dim %d must be even, in (0, head_dim=%d] and <= %d", d,
                cfg->head_dim, 2 * kMaxPairs);
  if (!(cfg->base > 1.0) || !std::isfinite(cfg->base))
    return fail(GPTOSS_ERR_SHAPE, "RoPE base must be finite and > 1");
  const int half = d / 2;
  const double s = cfg->scaling_factor;
  double c = 1.0;
  if (s > 1.0) {
    if (!(cfg->initial_context_length > 0) || !(cfg->ntk_alpha > 0.0) || !(cfg->ntk_beta > cfg->ntk_alpha))
      return fail(GPTOSS_ERR_SHAPE, "YaRN needs initial_context_length > 0 and 0 < ntk_alpha < ntk_beta");
    const double L0 = (double)cfg->initial_context_length;
    const double lb = std::log(cfg->base);
    const double lo = half * std::log(L0 / (2.0 * M_PI * cfg->ntk_beta)) / lb;
    const double hi = half * std::log(L0 / (2.0 * M_PI * cfg->ntk_alpha)) / lb;
    for (int i = 0; i < half; ++i) {
      const double theta = std::pow(cfg->base, -(2.0 * i) / d);
      double gam = (i - lo) / (hi - lo);
      gam = gam < 0.0 ? 0.0 : (gam > 1.0 ? 1.0 : gam);
      omega[i] = theta * (1.0 - gam) + (theta / s) * gam;
    }
    c = 0.1 * std::log(s) + 1.0;
  } else {
    for (int i = 0; i < half; ++i) omega[i] = std::pow(cfg->base, -(2.0 * i) / d);
  }
  *conc = c;
  return GPTOSS_OK;
}

gptoss_status check_desc(const gptoss_seq_desc* d) {
  if (!d) return fail(GPTOSS_ERR_NULL, "sequence descriptor is NULL");
  if (d->layout != GPTOSS_BSHD && d->layout != GPTOSS_THD)
    return fail(GPTOSS_ERR_SHAPE, "layout %d is neither BSHD (0) nor THD (1)", d->layout);
  if (d->batch < 0 || d->seqlen < 0) return fail(GPTOSS_ERR_SHAPE, "negative batch or seqlen");
  if (d->head_dim != kHeadDim)
    return fail(GPTOSS_ERR_UNSUPPORTED, "head_dim %d unsupported (only 64)", d->head_dim);
  if (d->num_kv_heads < 1 || d->num_q_heads != kGroup * d->num_kv_heads)
    return fail(GPTOSS_ERR_UNSUPPORTED, "num_q_heads %d must be 8 x num_kv_heads %d", d->num_q_heads,
                d->num_kv_heads);
  if (d->layout == GPTOSS_THD) {
    if (d->batch > 0 && !d->cu_seqlens) return fail(GPTOSS_ERR_NULL, "THD layout needs cu_seqlens");
    if (d->max_seqlen < 0 || d->max_seqlen > d->seqlen)
      return fail(GPTOSS_ERR_SHAPE, "max_seqlen %d must be in [0, total tokens %d]", d->max_seqlen, d->seqlen);
    if (d->batch > 4096) return fail(GPTOSS_ERR_UNSUPPORTED, "at most 4096 packed sequences");
    if (d->max_seqlen > 8192 * kPrefillBQ)
      return fail(GPTOSS_ERR_UNSUPPORTED, "packed sequences longer than %d tokens", 8192 * kPrefillBQ);
  }
  return GPTOSS_OK;
}

int32_t desc_max_len(const gptoss_seq_desc* d) { return d->layout == GPTOSS_BSHD ? d->seqlen : d->max_seqlen; }
int64_t desc_tokens(const gptoss_seq_desc* d) {
  return d->layout == GPTOSS_BSHD ? (int64_t)d->batch * d->seqlen : (int64_t)d->seqlen;
}
int32_t thd_max_items(const gptoss_seq_desc* d) {
  return (d->seqlen + kPrefillBQ - 1) / kPrefillBQ + d->batch;
}

// partial: the standalone rotations (gptoss_rope_qk, gptoss_kv_append) rotate
// the first rotary_dim dims for any multiple of 16 and copy the rest; the
// attention kernels rotate all 64 dims on their loads.
gptoss_status check_table(const void* table, int32_t table_rows, int32_t rotary_dim, int32_t need_rows,
                          bool partial = false) {
  if (!table) return GPTOSS_OK;
  if (partial) {
    if (rotary_dim < 16 || rotary_dim > kHeadDim || rotary_dim % 16 != 0)
      return fail(GPTOSS_ERR_UNSUPPORTED, "rotary_dim %d unsupported (16, 32, 48 or 64)", rotary_dim);
  } else if (rotary_dim != kHeadDim) {
    return fail(GPTOSS_ERR_UNSUPPORTED,
                "rotary_dim %d: the attention kernels rotate all 64 dims; rotate q and k with gptoss_rope_qk "
                "and pass table = NULL", rotary_dim);
  }
  if (!aligned16(table)) return fail(GPTOSS_ERR_UNSUPPORTED, "table must be 16-byte aligned");
  if (table_rows < need_rows || table_rows < 1)
    return fail(GPTOSS_ERR_SHAPE, "table has %d rows, positions up to %d are needed", table_rows, need_rows - 1);
  return GPTOSS_OK;
}

}  // namespace

extern "C" {

int gptoss_abi_version(void) { return GPTOSS_ABI_VERSION; }

const char* gptoss_status_string(int status) {
  switch (status) {
    case GPTOSS_OK: return "ok";
    case GPTOSS_ERR_NULL: return "null pointer argument";
    case GPTOSS_ERR_SHAPE: return "inconsistent shape, stride or size";
    case GPTOSS_ERR_UNSUPPORTED: return "unsupported configuration";
    case GPTOSS_ERR_WORKSPACE: return "workspace missing or too small";
    case GPTOSS_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* gptoss_last_error(void) { return g_last_error.c_str(); }

gptoss_status gptoss_yarn_params(const gptoss_rope_config* cfg, double* omega_out, double* concentration_out) {
  double omega[kMaxPairs], c;
  gptoss_status st = yarn(cfg, omega, &c);
  if (st != GPTOSS_OK) return st;
  if (omega_out) memcpy(omega_out, omega, sizeof(double) * (cfg->rotary_dim / 2));
  if (concentration_out) *concentration_out = c;
  return GPTOSS_OK;
}

gptoss_status gptoss_rope_table_init(const gptoss_rope_config* cfg, int32_t num_positions, void* table,
                                     void* stream) {
  if (!table) return fail(GPTOSS_ERR_NULL, "table is NULL");
  if (num_positions < 1) return fail(GPTOSS_ERR_SHAPE, "num_positions must be >= 1");
  TableParams p;
  gptoss_status st = yarn(cfg, p.omega, &p.concentration);
  if (st != GPTOSS_OK) return st;
  p.half = cfg->rotary_dim / 2;
  p.num_positions = num_positions;
  p.table = static_cast<uint16_t*>(table);
  return hip_status(launch_rope_table(p, static_cast<hipStream_t>(stream)), "rope table kernel");
}

}  // extern "C"

// One tensor (q or k, `heads` heads, layout strides st3) rotated into the
// contiguous y by the standalone rotation kernel (arguments checked by the caller).
static gptoss_status rotate_into(const gptoss_seq_desc* desc, const void* x, const int64_t st3[3], void* y,
                                 int32_t heads, const void* table, int32_t table_rows, int32_t rotary_dim,
                                 hipStream_t s) {
  const bool thd = desc->layout == GPTOSS_THD;
  RopeQKParams p;
  p.x = static_cast<const uint16_t*>(x);
  p.s_b = thd ? 0 : st3[0];
  p.s_t = st3[1];
  p.s_h = st3[2];
  p.y = static_cast<uint16_t*>(y);
  p.batch = thd ? 1 : desc->batch;
  p.tokens = desc->seqlen;
  p.heads = heads;
  p.cu_seqlens = thd ? desc->cu_seqlens : nullptr;
  p.num_seqs = desc->batch;
  p.table = static_cast<const uint16_t*>(table);
  p.table_rows = table_rows;
  p.rot_chunks = rotary_dim / 16;
  p.pos0 = 0;
  return hip_status(launch_rope_qk(p, s), "rope_qk kernel");
}

extern "C" {

gptoss_status gptoss_rope_qk(const gptoss_seq_desc* desc, const void* q, const int64_t q_strides[3],
                             const void* k, const int64_t k_strides[3], void* q_out, void* k_out,
                             const void* table, int32_t table_rows, int32_t rotary_dim, void* stream) {
  gptoss_status st = check_desc(desc);
  if (st != GPTOSS_OK) return st;
  if (desc_tokens(desc) == 0) return GPTOSS_OK;
  if (!q || !k || !q_out || !k_out || !q_strides || !k_strides || !table)
    return fail(GPTOSS_ERR_NULL, "q, k, q_out, k_out, strides and table are required");
  if (!strides_ok(q_strides, 3) || !strides_ok(k_strides, 3) || !aligned16(q) || !aligned16(k) ||
      !aligned16(q_out) || !aligned16(k_out))
    return fail(GPTOSS_ERR_UNSUPPORTED, "pointers must be 16-byte aligned and strides multiples of 8 elements");
  st = check_table(table, table_rows, rotary_dim, desc_max_len(desc), true);
  if (st != GPTOSS_OK) return st;
  if (desc->layout == GPTOSS_THD && desc->batch == 0) return GPTOSS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = rotate_into(desc, q, q_strides, q_out, desc->num_q_heads, table, table_rows, rotary_dim, s);
  if (st != GPTOSS_OK) return st;
  return rotate_into(desc, k, k_strides, k_out, desc->num_kv_heads, table, table_rows, rotary_dim, s);
}

}  // extern "C"

namespace {
// A BSHD query shard against a key shard of a longer sequence (NULL: whole sequences).
struct ShardArgs {
  int32_t kv_len, q_offset, kv_offset;
};

size_t prefill_ws_bytes(const gptoss_seq_desc* desc, int64_t kv_tokens) {
  size_t bytes = 0;
  if (desc->layout == GPTOSS_THD) bytes += round_up((size_t)thd_max_items(desc) * sizeof(int2)) + kAlign;
  // rotated K when k is rotated by a separate pass
  bytes += round_up((size_t)kv_tokens * desc->num_kv_heads * kHeadDim * sizeof(uint16_t));
  return bytes;
}

gptoss_status prefill_impl(const gptoss_seq_desc* desc, const void* q, const int64_t q_strides[3],
                           const void* k, const int64_t k_strides[3], const void* v,
                           const int64_t v_strides[3], const float* sinks, float softmax_scale,
                           int32_t window, const void* table, int32_t table_rows, int32_t rotary_dim,
                           void* out, const int64_t o_strides[3], float* lse, void* workspace,
                           size_t workspace_bytes, int krot, void* stream, const ShardArgs* shard = nullptr) {
  gptoss_status st = check_desc(desc);
  if (st != GPTOSS_OK) return st;
  if (desc_tokens(desc) == 0 || desc->batch == 0) return GPTOSS_OK;
  if (!q || !k || !v || !out || (!sinks && !shard) || !q_strides || !k_strides || !v_strides || !o_strides)
    return fail(GPTOSS_ERR_NULL, "q, k, v, out, sinks and all strides are required");
  if (!strides_ok(q_strides, 3) || !strides_ok(k_strides, 3) || !strides_ok(v_strides, 3) ||
      !strides_ok(o_strides, 3) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(GPTOSS_ERR_UNSUPPORTED, "pointers must be 16-byte aligned and strides multiples of 8 elements");
  if (window < 0) return fail(GPTOSS_ERR_SHAPE, "window must be >= 0 (0 = full causal)");
  if (!resolve_scale(softmax_scale, desc->head_dim))
    return fail(GPTOSS_ERR_SHAPE, "softmax_scale must be 0 (head_dim^-0.5) or finite and > 0");
  // a 64-key tile of K or V must span less than 2 GiB (32-bit buffer offsets)
  if (k_strides[1] * 2 * 64 > (int64_t)INT32_MAX || v_strides[1] * 2 * 64 > (int64_t)INT32_MAX)
    return fail(GPTOSS_ERR_UNSUPPORTED, "token strides of k and v must be below 2^24 elements");
  // rows of the table the rotations read
  const int32_t need_rows = shard ? std::max(shard->q_offset + desc->seqlen, shard->kv_offset + shard->kv_len)
                                  : desc_max_len(desc);
  st = check_table(table, table_rows, rotary_dim, need_rows, true);
  if (st != GPTOSS_OK) return st;
  if (table && rotary_dim != kHeadDim && krot == KROT_FUSED)
    return fail(GPTOSS_ERR_UNSUPPORTED, "k rotation inside the tile loads needs rotary_dim 64 (got %d)", rotary_dim);
  const int32_t kv_len = shard ? shard->kv_len : desc->seqlen;   // BSHD keys per sequence
  const size_t need = prefill_ws_bytes(desc, shard ? (int64_t)desc->batch * kv_len : desc_tokens(desc));
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return fail(GPTOSS_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  const bool thd = desc->layout == GPTOSS_THD;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int bq = kPrefillBQ;

  PrefillParams p;
  memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.q_sb = thd ? 0 : q_strides[0]; p.q_st = q_strides[1]; p.q_sh = q_strides[2];
  p.k = static_cast<const uint16_t*>(k);
  p.k_sb = thd ? 0 : k_strides[0]; p.k_st = k_strides[1]; p.k_sh = k_strides[2];
  p.v = static_cast<const uint16_t*>(v);
  p.v_sb = thd ? 0 : v_strides[0]; p.v_st = v_strides[1]; p.v_sh = v_strides[2];
  p.o = static_cast<uint16_t*>(out);
  p.o_sb = thd ? 0 : o_strides[0]; p.o_st = o_strides[1]; p.o_sh = o_strides[2];
  // without sinks the kernel still loads Hq floats, from q (any readable memory; the values are ignored)
  p.sinks = sinks ? sinks : static_cast<const float*>(q);
  p.no_sink = sinks ? 0 : 1;
  p.table = static_cast<const uint16_t*>(table);
  p.table_rows = table_rows;
  p.rot_chunks = table ? rotary_dim / 16 : kHeadDim / 16;
  p.batch = desc->batch;
  p.seqlen = desc->seqlen;
  p.num_kv_heads = desc->num_kv_heads;
  p.window = window;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.cu_seqlens = thd ? desc->cu_seqlens : nullptr;
  p.lse = lse;
  p.kv_len = kv_len;
  if (shard) {
    p.q_shift = shard->q_offset - shard->kv_offset;
    p.q_pos0 = shard->q_offset;
    p.k_pos0 = shard->kv_offset;
  }

  if (!shard && window > 0 && window % bq == 0 && window <= 4 * bq && o_strides[1] >= kHeadDim &&
      o_strides[1] * 2 * bq <= (int64_t)INT32_MAX) {
    // window layers of whole sequences: runs of consecutive query blocks, each key
    // rotated once as it enters the run's LDS ring
    if (thd) {
      // runs from the THD schedule with a run of run_len blocks as its unit
      const int32_t max_blocks = thd_max_items(desc);   // >= sum over sequences of ceil(L / 32)
      const int64_t blocks = (int64_t)max_blocks * desc->num_kv_heads;
      p.run_len = (int32_t)std::max<int64_t>(2, (blocks + kWindowRunsTargetThd - 1) / kWindowRunsTargetThd);
      const int32_t max_runs = (desc->seqlen + bq * p.run_len - 1) / (bq * p.run_len) + desc->batch;
      int2* work = reinterpret_cast<int2*>(ws);
      ws += round_up((size_t)max_runs * sizeof(int2));
      int32_t* count = reinterpret_cast<int32_t*>(ws);
      st = hip_status(launch_thd_schedule(desc->cu_seqlens, desc->batch, bq * p.run_len, max_runs, work, count, s),
                      "THD run schedule kernel");
      if (st != GPTOSS_OK) return st;
      p.work = work;
      p.work_count = count;
      p.q_blocks = max_runs;
    } else {
      const int32_t qb = (desc->seqlen + bq - 1) / bq;
      const int64_t blocks = (int64_t)qb * desc->batch * desc->num_kv_heads;
      p.run_len = (int32_t)std::max<int64_t>(2, (blocks + kWindowRunsTarget - 1) / kWindowRunsTarget);
      p.runs_per_seq = (qb + p.run_len - 1) / p.run_len;
      // every run resident at once (two work groups per CU): split neighbouring runs
      // 11 : 5 in favour of the first-dispatched one (measured best of 9 .. 12 of 16)
      const int64_t wgs = (int64_t)desc->batch * p.runs_per_seq * desc->num_kv_heads;
      if (p.runs_per_seq % 2 == 0 && wgs <= 2 * (int64_t)device_cus()) p.pair_first = (22 * p.run_len + 8) / 16;
    }
    return hip_status(launch_window_runs(p, thd, s), "window prefill kernel");
  }
  if (thd) {
    const int32_t max_items = thd_max_items(desc);
    int2* work = reinterpret_cast<int2*>(ws);
    ws += round_up((size_t)max_items * sizeof(int2));
    int32_t* count = reinterpret_cast<int32_t*>(ws);
    ws += kAlign;
    st = hip_status(launch_thd_schedule(desc->cu_seqlens, desc->batch, bq, max_items, work, count, s),
                    "THD schedule kernel");
    if (st != GPTOSS_OK) return st;
    p.work = work;
    p.work_count = count;
    p.q_blocks = max_items;
  } else {
    p.q_blocks = (desc->seqlen + bq - 1) / bq;
  }

  if (table && krot != KROT_FUSED) {
    // rotate k once into the workspace (contiguous), then attend with pre-rotated k
    uint16_t* krot_buf = reinterpret_cast<uint16_t*>(ws);
    RopeQKParams r;
    r.x = static_cast<const uint16_t*>(k);
    r.s_b = p.k_sb; r.s_t = p.k_st; r.s_h = p.k_sh;
    r.y = krot_buf;
    r.batch = thd ? 1 : desc->batch;
    r.tokens = thd ? desc->seqlen : kv_len;
    r.heads = desc->num_kv_heads;
    r.cu_seqlens = thd ? desc->cu_seqlens : nullptr;
    r.num_seqs = desc->batch;
    r.table = p.table;
    r.table_rows = table_rows;
    r.rot_chunks = rotary_dim / 16;
    r.pos0 = p.k_pos0;
    st = hip_status(launch_rope_qk(r, s), "k rotation kernel");
    if (st != GPTOSS_OK) return st;
    p.k = krot_buf;
    p.k_sh = kHeadDim;
    p.k_st = (int64_t)desc->num_kv_heads * kHeadDim;
    p.k_sb = thd ? 0 : (int64_t)kv_len * p.k_st;
  }
  return hip_status(launch_prefill(p, thd, krot, s), "prefill kernel");
}
}  // namespace

extern "C" {

gptoss_status gptoss_attn_prefill(const gptoss_seq_desc* desc, const void* q, const int64_t q_strides[3],
                                  const void* k, const int64_t k_strides[3], const void* v,
                                  const int64_t v_strides[3], const float* sinks, float softmax_scale,
                                  int32_t window, const void* table, int32_t table_rows, int32_t rotary_dim,
                                  void* out, const int64_t o_strides[3], void* workspace,
                                  size_t workspace_bytes, void* stream) {
  // K rotation: one separate pass into the workspace for both layer types.
  // Rotating inside the tile loads was measured slower on gfx950 even for
  // window layers, where each key tile is staged only about three times.
  const int krot = KROT_NONE;
  return prefill_impl(desc, q, q_strides, k, k_strides, v, v_strides, sinks, softmax_scale, window, table,
                      table_rows, rotary_dim, out, o_strides, nullptr, workspace, workspace_bytes, krot, stream);
}

gptoss_status gptoss_attn_prefill_lse(const gptoss_seq_desc* desc, const void* q, const int64_t q_strides[3],
                                      const void* k, const int64_t k_strides[3], const void* v,
                                      const int64_t v_strides[3], const float* sinks, float softmax_scale,
                                      int32_t window, const void* table, int32_t table_rows,
                                      int32_t rotary_dim, void* out, const int64_t o_strides[3], float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!lse) return fail(GPTOSS_ERR_NULL, "lse is required");
  if (!aligned16(lse)) return fail(GPTOSS_ERR_UNSUPPORTED, "lse must be 16-byte aligned");
  return prefill_impl(desc, q, q_strides, k, k_strides, v, v_strides, sinks, softmax_scale, window, table,
                      table_rows, rotary_dim, out, o_strides, lse, workspace, workspace_bytes, KROT_NONE, stream);
}

gptoss_status gptoss_attn_prefill_ex(const gptoss_seq_desc* desc, const void* q, const int64_t q_strides[3],
                                     const void* k, const int64_t k_strides[3], const void* v,
                                     const int64_t v_strides[3], const float* sinks, float softmax_scale,
                                     int32_t window, const void* table, int32_t table_rows,
                                     int32_t rotary_dim, void* out, const int64_t o_strides[3],
                                     void* workspace, size_t workspace_bytes, int32_t k_rotation,
                                     void* stream) {
  int krot;
  switch (k_rotation) {
    case GPTOSS_KROT_AUTO: krot = KROT_NONE; break;
    case GPTOSS_KROT_FUSED: krot = KROT_FUSED; break;
    case GPTOSS_KROT_SEPARATE: krot = KROT_NONE; break;
    default: return fail(GPTOSS_ERR_SHAPE, "k_rotation %d is not a gptoss_k_rotation value", k_rotation);
  }
  return prefill_impl(desc, q, q_strides, k, k_strides, v, v_strides, sinks, softmax_scale, window, table,
                      table_rows, rotary_dim, out, o_strides, nullptr, workspace, workspace_bytes, krot, stream);
}

size_t gptoss_attn_prefill_workspace_size(const gptoss_seq_desc* desc) {
  if (check_desc(desc) != GPTOSS_OK) return 0;
  return prefill_ws_bytes(desc, desc_tokens(desc));
}

size_t gptoss_attn_prefill_shard_workspace_size(const gptoss_seq_desc* desc, int32_t kv_len) {
  if (check_desc(desc) != GPTOSS_OK || desc->layout != GPTOSS_BSHD || kv_len < 0) return 0;
  return prefill_ws_bytes(desc, (int64_t)desc->batch * kv_len);
}

gptoss_status gptoss_attn_prefill_shard(const gptoss_seq_desc* desc, const void* q, const int64_t q_strides[3],
                                        const void* k, const int64_t k_strides[3], const void* v,
                                        const int64_t v_strides[3], int32_t kv_len, int32_t q_offset,
                                        int32_t kv_offset, float softmax_scale, int32_t window, const void* table,
                                        int32_t table_rows, int32_t rotary_dim, void* out,
                                        const int64_t o_strides[3], float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  gptoss_status st = check_desc(desc);
  if (st != GPTOSS_OK) return st;
  if (desc->layout != GPTOSS_BSHD) return fail(GPTOSS_ERR_UNSUPPORTED, "shards are BSHD");
  if (kv_len < 0 || q_offset < 0 || kv_offset < 0)
    return fail(GPTOSS_ERR_SHAPE, "kv_len, q_offset and kv_offset must be >= 0");
  if ((int64_t)q_offset + desc->seqlen > INT32_MAX || (int64_t)kv_offset + kv_len > INT32_MAX)
    return fail(GPTOSS_ERR_SHAPE, "positions must stay below 2^31");
  if (!lse) return fail(GPTOSS_ERR_NULL, "lse is required (the merge weights the shards by it)");
  if (reinterpret_cast<uintptr_t>(lse) & 15) return fail(GPTOSS_ERR_UNSUPPORTED, "lse must be 16-byte aligned");
  // no sink here (sinks = NULL: the shard's own softmax); the merge adds it once
  const ShardArgs sh{kv_len, q_offset, kv_offset};
  return prefill_impl(desc, q, q_strides, k, k_strides, v, v_strides, nullptr, softmax_scale,
                      window, table, table_rows, rotary_dim, out, o_strides, lse, workspace, workspace_bytes,
                      KROT_NONE, stream, &sh);
}

gptoss_status gptoss_attn_merge(int32_t num_parts, int32_t tokens, int32_t num_q_heads, int32_t head_dim,
                                const void* o_parts, const int64_t part_strides[4], const float* lse_parts,
                                const float* sinks, void* out, const int64_t o_strides[2], float* lse_out,
                                void* stream) {
  if (num_parts < 0 || tokens < 0 || num_q_heads < 1) return fail(GPTOSS_ERR_SHAPE, "negative size or no heads");
  if (head_dim != kHeadDim) return fail(GPTOSS_ERR_UNSUPPORTED, "head_dim %d unsupported (only 64)", head_dim);
  if (tokens == 0) return GPTOSS_OK;
  if (!out || !o_strides || (num_parts > 0 && (!o_parts || !part_strides || !lse_parts)))
    return fail(GPTOSS_ERR_NULL, "out, its strides and (with parts) the parts, their strides and lse are required");
  if (num_parts > 0 && (!strides_ok(part_strides, 3) || part_strides[3] != 1 || !aligned16(o_parts)))
    return fail(GPTOSS_ERR_UNSUPPORTED,
                "o_parts must be 16-byte aligned, strides multiples of 8 with the head dim contiguous");
  if (!strides_ok(o_strides, 2) || !aligned16(out))
    return fail(GPTOSS_ERR_UNSUPPORTED, "out must be 16-byte aligned with strides multiples of 8");
  MergeParams p;
  memset(&p, 0, sizeof p);
  p.o = static_cast<const uint16_t*>(o_parts);
  if (num_parts > 0) { p.o_sp = part_strides[0]; p.o_st = part_strides[1]; p.o_sh = part_strides[2]; }
  p.lse = lse_parts;
  p.l_sp = (int64_t)tokens * num_q_heads;
  p.sinks = sinks;
  p.out = static_cast<uint16_t*>(out);
  p.out_st = o_strides[0]; p.out_sh = o_strides[1];
  p.lse_out = lse_out;
  p.parts = num_parts;
  p.tokens = tokens;
  p.num_q_heads = num_q_heads;
  return hip_status(launch_merge(p, static_cast<hipStream_t>(stream)), "merge kernel");
}

// ---------------------------------------------------------------------------
// Backward of the prefill attention.
// ---------------------------------------------------------------------------
static int32_t thd_items(const gptoss_seq_desc* d, int bq) { return (d->seqlen + bq - 1) / bq + d->batch; }
// work items of the backward dq kernel (the length of each head's row of dsigma partials)
static int64_t bwd_q_items(const gptoss_seq_desc* d) {
  return d->layout == GPTOSS_THD ? (int64_t)thd_items(d, kPrefillBQ)
                                 : (int64_t)d->batch * ((d->seqlen + kPrefillBQ - 1) / kPrefillBQ);
}

size_t gptoss_attn_prefill_backward_workspace_size(const gptoss_seq_desc* desc) {
  if (check_desc(desc) != GPTOSS_OK) return 0;
  const size_t T = (size_t)desc_tokens(desc);
  const size_t hq = (size_t)desc->num_q_heads, hkv = (size_t)desc->num_kv_heads;
  size_t bytes = 0;
  if (desc->layout == GPTOSS_THD)
    bytes += round_up((size_t)thd_items(desc, kPrefillBQ) * sizeof(int2)) + kAlign +
             round_up((size_t)thd_items(desc, kBackwardKT) * sizeof(int2)) + kAlign;
  bytes += round_up(T * hq * kHeadDim * sizeof(uint16_t));    // rotated q
  bytes += round_up(T * hkv * kHeadDim * sizeof(uint16_t));   // rotated k
  bytes += round_up(T * hq * 2 * sizeof(float));              // (lse in log2 units, -<dO, o>), head-major
  bytes += round_up((size_t)bwd_q_items(desc) * hq * sizeof(float));   // dsigma partials, head-major
  return bytes;
}

gptoss_status gptoss_attn_prefill_backward(const gptoss_seq_desc* desc, const void* q, const int64_t q_strides[3],
                                           const void* k, const int64_t k_strides[3], const void* v,
                                           const int64_t v_strides[3], const float* sinks, float softmax_scale,
                                           int32_t window, const void* table, int32_t table_rows,
                                           int32_t rotary_dim, const void* out, const int64_t o_strides[3],
                                           const void* dout, const int64_t do_strides[3], const float* lse,
                                           void* dq, void* dk, void* dv, float* dsinks, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  gptoss_status st = check_desc(desc);
  if (st != GPTOSS_OK) return st;
  if (!dsinks) return fail(GPTOSS_ERR_NULL, "dsinks is required");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (desc_tokens(desc) == 0 || desc->batch == 0)
    return hip_status(launch_fill_f32(dsinks, desc->num_q_heads, 0.0f, s), "dsinks clear");
  if (!q || !k || !v || !out || !dout || !lse || !sinks || !dq || !dk || !dv || !q_strides || !k_strides ||
      !v_strides || !o_strides || !do_strides)
    return fail(GPTOSS_ERR_NULL, "q, k, v, sinks, out, dout, lse, dq, dk, dv and all strides are required");
  if (!strides_ok(q_strides, 3) || !strides_ok(k_strides, 3) || !strides_ok(v_strides, 3) ||
      !strides_ok(o_strides, 3) || !strides_ok(do_strides, 3) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
      !aligned16(out) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(lse))
    return fail(GPTOSS_ERR_UNSUPPORTED, "pointers must be 16-byte aligned and strides multiples of 8 elements");
  if (window < 0) return fail(GPTOSS_ERR_SHAPE, "window must be >= 0 (0 = full causal)");
  if (!resolve_scale(softmax_scale, desc->head_dim))
    return fail(GPTOSS_ERR_SHAPE, "softmax_scale must be 0 (head_dim^-0.5) or finite and > 0");
  if (k_strides[1] * 2 * 64 > (int64_t)INT32_MAX || v_strides[1] * 2 * 64 > (int64_t)INT32_MAX)
    return fail(GPTOSS_ERR_UNSUPPORTED, "token strides of k and v must be below 2^24 elements");
  st = check_table(table, table_rows, rotary_dim, desc_max_len(desc));
  if (st != GPTOSS_OK) return st;
  const size_t need = gptoss_attn_prefill_backward_workspace_size(desc);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return fail(GPTOSS_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  const bool thd = desc->layout == GPTOSS_THD;
  const int64_t T = desc_tokens(desc);
  const int32_t hq = desc->num_q_heads, hkv = desc->num_kv_heads;
  // one sequence's q and dO rows (plus a query block of slack) are addressed with 32-bit byte offsets
  const int64_t q_row = table ? (int64_t)hq * kHeadDim : q_strides[1];
  if (((int64_t)desc_max_len(desc) + 64) * 2 * std::max(q_row, do_strides[1]) > (int64_t)INT32_MAX)
    return fail(GPTOSS_ERR_UNSUPPORTED, "a sequence's q / dout rows must span less than 2 GiB");
  if (bwd_q_items(desc) * hkv * 2 > (int64_t)INT32_MAX)
    return fail(GPTOSS_ERR_UNSUPPORTED, "too many 32-query blocks for one launch");
  char* ws = static_cast<char*>(workspace);

  BackwardParams p;
  memset(&p, 0, sizeof p);
  if (thd) {
    const int32_t nq = thd_items(desc, kPrefillBQ), nk = thd_items(desc, kBackwardKT);
    int2* wq = reinterpret_cast<int2*>(ws);
    ws += round_up((size_t)nq * sizeof(int2));
    int32_t* cq = reinterpret_cast<int32_t*>(ws);
    ws += kAlign;
    int2* wk = reinterpret_cast<int2*>(ws);
    ws += round_up((size_t)nk * sizeof(int2));
    int32_t* ck = reinterpret_cast<int32_t*>(ws);
    ws += kAlign;
    st = hip_status(launch_thd_schedule(desc->cu_seqlens, desc->batch, kPrefillBQ, nq, wq, cq, s), "THD schedule");
    if (st != GPTOSS_OK) return st;
    st = hip_status(launch_thd_schedule(desc->cu_seqlens, desc->batch, kBackwardKT, nk, wk, ck, s), "THD schedule");
    if (st != GPTOSS_OK) return st;
    p.work_q = wq; p.count_q = cq; p.q_blocks = nq;
    p.work_k = wk; p.count_k = ck; p.k_tiles = nk;
  } else {
    p.q_blocks = (desc->seqlen + kPrefillBQ - 1) / kPrefillBQ;
    p.k_tiles = (desc->seqlen + kBackwardKT - 1) / kBackwardKT;
    // full causal, a multiple of 4 key tiles: two tiles per dk / dv work group, balanced
    p.kv_pairs = (window == 0 && p.k_tiles % 4 == 0) ? 1 : 0;
  }
  uint16_t* qrot = reinterpret_cast<uint16_t*>(ws);
  ws += round_up((size_t)T * hq * kHeadDim * sizeof(uint16_t));
  uint16_t* krot = reinterpret_cast<uint16_t*>(ws);
  ws += round_up((size_t)T * hkv * kHeadDim * sizeof(uint16_t));
  p.ld = reinterpret_cast<float*>(ws);
  ws += round_up((size_t)T * hq * 2 * sizeof(float));
  p.dsink_part = reinterpret_cast<float*>(ws);
  p.dsink_items = (int32_t)bwd_q_items(desc);
  p.tokens = T;

  if (table) {
    // k is rotated once into the workspace (contiguous) by the standalone kernel;
    // the dq kernel rotates q on load, exactly as the forward does, and writes the
    // rotated rows to the workspace for the dk / dv kernel
    st = rotate_into(desc, k, k_strides, krot, hkv, table, table_rows, rotary_dim, s);
    if (st != GPTOSS_OK) return st;
    p.q_in = static_cast<const uint16_t*>(q);
    p.qi_sb = thd ? 0 : q_strides[0]; p.qi_st = q_strides[1]; p.qi_sh = q_strides[2];
    p.q_rot = qrot;
    p.q = qrot;
    p.q_sh = kHeadDim; p.q_st = (int64_t)hq * kHeadDim; p.q_sb = thd ? 0 : (int64_t)desc->seqlen * p.q_st;
    p.k = krot;
    p.k_sh = kHeadDim; p.k_st = (int64_t)hkv * kHeadDim; p.k_sb = thd ? 0 : (int64_t)desc->seqlen * p.k_st;
  } else {
    p.q = static_cast<const uint16_t*>(q);
    p.q_sb = thd ? 0 : q_strides[0]; p.q_st = q_strides[1]; p.q_sh = q_strides[2];
    p.k = static_cast<const uint16_t*>(k);
    p.k_sb = thd ? 0 : k_strides[0]; p.k_st = k_strides[1]; p.k_sh = k_strides[2];
  }
  p.v = static_cast<const uint16_t*>(v);
  p.v_sb = thd ? 0 : v_strides[0]; p.v_st = v_strides[1]; p.v_sh = v_strides[2];
  p.o = static_cast<const uint16_t*>(out);
  p.o_sb = thd ? 0 : o_strides[0]; p.o_st = o_strides[1]; p.o_sh = o_strides[2];
  p.dout = static_cast<const uint16_t*>(dout);
  p.do_sb = thd ? 0 : do_strides[0]; p.do_st = do_strides[1]; p.do_sh = do_strides[2];
  p.lse = lse;
  p.sinks = sinks;
  p.dsinks = dsinks;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.table = static_cast<const uint16_t*>(table);
  p.table_rows = table_rows;
  p.batch = desc->batch;
  p.seqlen = desc->seqlen;
  p.num_kv_heads = hkv;
  p.window = window;
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.cu_seqlens = thd ? desc->cu_seqlens : nullptr;
  return hip_status(launch_backward(p, thd, s), "backward kernels");
}

// Keys per split when the caller fixes the number of splits: a multiple of 128.
static int32_t decode_fixed_chunk(int32_t eff_len, int32_t num_splits) {
  int32_t c = (eff_len + num_splits - 1) / num_splits;
  c = (c + 127) / 128 * 128;
  return c < 128 ? 128 : c;
}

// Upper bound of the splits any call with these sizes uses: the planned split
// length is at least min_chunk keys.
static int64_t decode_split_cap(int32_t max_cache_len, int32_t num_splits, int32_t min_chunk = kDecodeMinChunk) {
  return num_splits > 0 ? num_splits : (max_cache_len + min_chunk - 1) / min_chunk;
}

// Work-group slots of the decode split kernel on the current device (2 per CU).
static int32_t decode_slots() { return 2 * device_cus(); }

static size_t decode_ws_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_keys, int32_t num_splits,
                              int32_t min_chunk = kDecodeMinChunk) {
  const int64_t cap = decode_split_cap(max_keys, num_splits, min_chunk);
  const size_t slots = (size_t)num_seqs * num_q_heads * cap;
  // partials, then the split plan: 2 ints + one int2 per (sequence, split) item
  return round_up(slots * kHeadDim * sizeof(float)) + round_up(slots * 2 * sizeof(float)) +
         round_up(2 * sizeof(int32_t) + (size_t)num_seqs * cap * 2 * sizeof(int32_t));
}

size_t gptoss_attn_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t max_cache_len,
                                         int32_t num_splits) {
  if (num_seqs < 0 || num_q_heads < 0 || max_cache_len < 1 || num_splits < 0) return 0;
  return decode_ws_bytes(num_seqs, num_q_heads, max_cache_len, num_splits);
}

// Checks shared by both decode entry points; p gets q, sinks, table, out.
static gptoss_status decode_args(DecodeParams& p, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, const void* q, const int64_t q_strides[2], const void* k_cache,
                                 const void* v_cache, const int32_t* cache_seqlens, int32_t max_len,
                                 const float* sinks, float softmax_scale, int32_t window, const void* table,
                                 int32_t table_rows, int32_t rotary_dim, void* out, const int64_t o_strides[2],
                                 int32_t num_splits) {
  if (num_seqs < 0) return fail(GPTOSS_ERR_SHAPE, "num_seqs must be >= 0");
  if (head_dim != kHeadDim) return fail(GPTOSS_ERR_UNSUPPORTED, "head_dim %d unsupported (only 64)", head_dim);
  if (num_kv_heads < 1 || num_q_heads != kGroup * num_kv_heads)
    return fail(GPTOSS_ERR_UNSUPPORTED, "num_q_heads %d must be 8 x num_kv_heads %d", num_q_heads, num_kv_heads);
  if (max_len < 1) return fail(GPTOSS_ERR_SHAPE, "the maximum cache length must be >= 1");
  if (num_splits < 0) return fail(GPTOSS_ERR_SHAPE, "num_splits must be >= 0");
  if (window < 0) return fail(GPTOSS_ERR_SHAPE, "window must be >= 0 (0 = full causal)");
  if (!resolve_scale(softmax_scale, head_dim))
    return fail(GPTOSS_ERR_SHAPE, "softmax_scale must be 0 (head_dim^-0.5) or finite and > 0");
  if (num_seqs == 0) return GPTOSS_OK;
  if (!q || !k_cache || !v_cache || !cache_seqlens || !sinks || !out || !q_strides || !o_strides)
    return fail(GPTOSS_ERR_NULL, "q, caches, cache_seqlens, sinks, out and all strides are required");
  if (!strides_ok(q_strides, 2) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(GPTOSS_ERR_UNSUPPORTED, "pointers must be 16-byte aligned and strides multiples of 8 elements");
  if (o_strides[0] < 0 || o_strides[1] < 0 || (o_strides[0] & 1) || (o_strides[1] & 1) ||
      (reinterpret_cast<uintptr_t>(out) & 3))
    return fail(GPTOSS_ERR_UNSUPPORTED, "out must be 4-byte aligned with even strides");
  gptoss_status st = check_table(table, table_rows, rotary_dim, max_len, true);
  if (st != GPTOSS_OK) return st;
  p.q = static_cast<const uint16_t*>(q);
  p.q_sn = q_strides[0]; p.q_sh = q_strides[1];
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.cache_seqlens = cache_seqlens;
  p.max_cache_len = max_len;
  p.num_seqs = num_seqs;
  p.num_kv_heads = num_kv_heads;
  p.window = window;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.sinks = sinks;
  p.table = static_cast<const uint16_t*>(table);
  p.table_rows = table_rows;
  p.rot_chunks = table ? rotary_dim / 16 : kHeadDim / 16;
  p.o = static_cast<uint16_t*>(out);
  p.o_sn = o_strides[0]; p.o_sh = o_strides[1];
  return GPTOSS_OK;
}

// Split sizing, workspace carving and launch. eff: most keys one sequence reads
// (the workspace was sized for ws_keys >= eff).
static gptoss_status decode_run(DecodeParams& p, int32_t num_q_heads, int32_t eff, int32_t ws_keys,
                                void* workspace, size_t workspace_bytes, int32_t num_splits, void* stream,
                                int32_t min_chunk = kDecodeMinChunk) {
  const size_t need = decode_ws_bytes(p.num_seqs, num_q_heads, ws_keys, num_splits, min_chunk);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return fail(GPTOSS_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  p.min_chunk = min_chunk;
  if (num_splits == 1 || (num_splits == 0 && eff <= min_chunk)) {
    // one split per sequence (e.g. window layers): no plan, work item = sequence
    p.direct_chunk = (eff + 127) / 128 * 128;
    p.num_splits = 1;
  } else if (num_splits > 0) {
    p.chunk_fixed = decode_fixed_chunk(eff, num_splits);
    p.num_splits = (eff + p.chunk_fixed - 1) / p.chunk_fixed;
  } else {
    // planned on the device from the cache lengths: about 1.3 work items per slot
    p.chunk_fixed = 0;
    p.target_chunks = decode_slots() * 13 / 10;
    p.num_splits = (eff + min_chunk - 1) / min_chunk;
  }
  // p.num_splits <= decode_split_cap(ws_keys): the partial buffers fit the workspace
  char* ws = static_cast<char*>(workspace);
  const size_t cap = (size_t)p.num_seqs * num_q_heads * decode_split_cap(ws_keys, num_splits, min_chunk);
  p.part_o = reinterpret_cast<float*>(ws);
  p.part_ml = reinterpret_cast<float*>(ws + round_up(cap * kHeadDim * sizeof(float)));
  p.plan = reinterpret_cast<int32_t*>(ws + round_up(cap * kHeadDim * sizeof(float)) + round_up(cap * 2 * sizeof(float)));
  // work groups: enough for every item of the largest plan, at most two per slot (they loop)
  const int64_t max_items = (int64_t)p.num_seqs * p.num_splits;
  const int64_t groups = (int64_t)decode_slots() * 2;
  p.max_items = (int32_t)(max_items < groups ? max_items : groups);
  return hip_status(launch_decode(p, static_cast<hipStream_t>(stream)), "decode kernels");
}

gptoss_status gptoss_attn_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 const void* q, const int64_t q_strides[2], const void* k_cache,
                                 const void* v_cache, const int64_t kv_strides[3],
                                 const int32_t* cache_seqlens, int32_t max_cache_len, const float* sinks,
                                 float softmax_scale, int32_t window, const void* table, int32_t table_rows,
                                 int32_t rotary_dim, void* out, const int64_t o_strides[2], void* workspace,
                                 size_t workspace_bytes, int32_t num_splits, void* stream) {
  DecodeParams p;
  memset(&p, 0, sizeof p);
  gptoss_status st = decode_args(p, num_seqs, num_q_heads, num_kv_heads, head_dim, q, q_strides, k_cache, v_cache,
                                 cache_seqlens, max_cache_len, sinks, softmax_scale, window, table, table_rows,
                                 rotary_dim, out, o_strides, num_splits);
  if (st != GPTOSS_OK || num_seqs == 0) return st;
  if (!kv_strides) return fail(GPTOSS_ERR_NULL, "kv_strides are required");
  if (!strides_ok(kv_strides, 3))
    return fail(GPTOSS_ERR_UNSUPPORTED, "pointers must be 16-byte aligned and strides multiples of 8 elements");
  if (kv_strides[1] < kHeadDim || (int64_t)max_cache_len * kv_strides[1] * 2 > (int64_t)INT32_MAX)
    return fail(GPTOSS_ERR_UNSUPPORTED,
                "kv_strides[1] must be >= 64 and one sequence's rows must span less than 2 GiB");
  p.kind = kCacheContiguous;
  p.kv_sn = kv_strides[0]; p.kv_sp = kv_strides[1]; p.kv_sh = kv_strides[2];
  // window layers only ever read the last `window` rows: fewer splits
  const int32_t eff = (window > 0 && window < max_cache_len) ? window : max_cache_len;
  return decode_run(p, num_q_heads, eff, max_cache_len, workspace, workspace_bytes, num_splits, stream);
}

static int ilog2_pow2(int32_t x) {   // log2 of a power of two, else -1
  if (x <= 0 || (x & (x - 1))) return -1;
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// Checks of a cache layout shared by append and decode.
static gptoss_status check_layout(const gptoss_kv_layout* lay, int32_t max_seqlen, bool for_decode,
                                  int32_t window) {
  if (!lay) return fail(GPTOSS_ERR_NULL, "cache layout is NULL");
  if (lay->kind != GPTOSS_CACHE_CONTIGUOUS && lay->kind != GPTOSS_CACHE_PAGED && lay->kind != GPTOSS_CACHE_RING)
    return fail(GPTOSS_ERR_SHAPE, "cache kind %d is not CONTIGUOUS (0), PAGED (1) or RING (2)", lay->kind);
  if (lay->capacity < 1) return fail(GPTOSS_ERR_SHAPE, "cache capacity must be >= 1");
  if (!strides_ok(lay->strides, 3) || lay->strides[1] < kHeadDim)
    return fail(GPTOSS_ERR_UNSUPPORTED, "cache strides must be multiples of 8 elements, the row stride >= 64");
  if ((int64_t)lay->capacity * lay->strides[1] * 2 > (int64_t)INT32_MAX)
    return fail(GPTOSS_ERR_UNSUPPORTED, "one sequence's (or page's) rows must span less than 2 GiB");
  if (lay->kind == GPTOSS_CACHE_PAGED) {
    if (ilog2_pow2(lay->capacity) < 5)
      return fail(GPTOSS_ERR_UNSUPPORTED, "page size %d must be a power of two >= 32", lay->capacity);
    if (!lay->block_table) return fail(GPTOSS_ERR_NULL, "a paged cache needs its block table");
    if (lay->max_pages < 1 || lay->num_pages < 1)
      return fail(GPTOSS_ERR_SHAPE, "a paged cache needs max_pages >= 1 and num_pages >= 1");
    if (for_decode && (int64_t)max_seqlen > (int64_t)lay->max_pages * lay->capacity)
      return fail(GPTOSS_ERR_SHAPE, "max_seqlen %d exceeds max_pages x page size", max_seqlen);
  } else if (lay->kind == GPTOSS_CACHE_CONTIGUOUS) {
    if (for_decode && max_seqlen > lay->capacity)
      return fail(GPTOSS_ERR_SHAPE, "max_seqlen %d exceeds the cache's %d rows", max_seqlen, lay->capacity);
  } else if (for_decode && window != lay->capacity) {
    return fail(GPTOSS_ERR_UNSUPPORTED, "a ring cache serves a window layer with window == capacity (%d, got %d)",
                lay->capacity, window);
  }
  return GPTOSS_OK;
}

// Most keys one sequence's decode reads from a cache of this layout.
static int32_t decode_max_keys(const gptoss_kv_layout* lay, int32_t max_seqlen, int32_t window) {
  if (lay->kind == GPTOSS_CACHE_RING) return std::min(lay->capacity, max_seqlen);
  if (lay->kind == GPTOSS_CACHE_PAGED) return window > 0 ? std::min(window + 31, max_seqlen) : max_seqlen;
  return (window > 0 && window < max_seqlen) ? window : max_seqlen;
}

size_t gptoss_attn_decode_kv_workspace_size(const gptoss_kv_layout* layout, int32_t num_seqs, int32_t num_q_heads,
                                            int32_t max_seqlen, int32_t window, int32_t num_splits) {
  if (!layout || num_seqs < 0 || num_q_heads < 0 || max_seqlen < 1 || num_splits < 0 || window < 0) return 0;
  return decode_ws_bytes(num_seqs, num_q_heads, decode_max_keys(layout, max_seqlen, window), num_splits);
}

gptoss_status gptoss_attn_decode_kv(const gptoss_kv_layout* layout, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, const void* q,
                                    const int64_t q_strides[2], const void* k_cache, const void* v_cache,
                                    const int32_t* cache_seqlens, int32_t max_seqlen, const float* sinks,
                                    float softmax_scale, int32_t window, const void* table, int32_t table_rows,
                                    int32_t rotary_dim, void* out, const int64_t o_strides[2], void* workspace,
                                    size_t workspace_bytes, int32_t num_splits, void* stream) {
  DecodeParams p;
  memset(&p, 0, sizeof p);
  gptoss_status st = decode_args(p, num_seqs, num_q_heads, num_kv_heads, head_dim, q, q_strides, k_cache, v_cache,
                                 cache_seqlens, max_seqlen, sinks, softmax_scale, window, table, table_rows,
                                 rotary_dim, out, o_strides, num_splits);
  if (st != GPTOSS_OK) return st;
  st = check_layout(layout, max_seqlen, true, window);
  if (st != GPTOSS_OK || num_seqs == 0) return st;
  p.kind = layout->kind;
  p.kv_sn = layout->strides[0]; p.kv_sp = layout->strides[1]; p.kv_sh = layout->strides[2];
  if (layout->kind == GPTOSS_CACHE_PAGED) {
    p.page_log2 = ilog2_pow2(layout->capacity);
    p.block_table = layout->block_table;
    p.max_pages = layout->max_pages;
    p.num_pages = layout->num_pages;
  } else if (layout->kind == GPTOSS_CACHE_RING) {
    p.ring_slots = layout->capacity;
  }
  const int32_t keys = decode_max_keys(layout, max_seqlen, window);
  return decode_run(p, num_q_heads, keys, keys, workspace, workspace_bytes, num_splits, stream);
}

static_assert(GPTOSS_DECODE_SCRATCH_BYTES == kStaticScratchBytes, "scratch size in the header and the library");

gptoss_status gptoss_attn_decode_kv_noalloc(const gptoss_kv_layout* layout, int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim, const void* q,
                                            const int64_t q_strides[2], const void* k_cache, const void* v_cache,
                                            const int32_t* cache_seqlens, int32_t max_seqlen, const float* sinks,
                                            float softmax_scale, int32_t window, const void* table,
                                            int32_t table_rows, int32_t rotary_dim, void* out,
                                            const int64_t o_strides[2], int32_t num_splits, void* stream) {
  DecodeParams p;
  memset(&p, 0, sizeof p);
  gptoss_status st = decode_args(p, num_seqs, num_q_heads, num_kv_heads, head_dim, q, q_strides, k_cache, v_cache,
                                 cache_seqlens, max_seqlen, sinks, softmax_scale, window, table, table_rows,
                                 rotary_dim, out, o_strides, num_splits);
  if (st != GPTOSS_OK) return st;
  st = check_layout(layout, max_seqlen, true, window);
  if (st != GPTOSS_OK || num_seqs == 0) return st;
  const int32_t keys = decode_max_keys(layout, max_seqlen, window);
  // The partials must fit the fixed scratch: with a planned split count, the
  // shortest split grows (a multiple of 128 keys) until the most splits a
  // sequence can take fit; a caller-given count must fit as it is.
  // bytes per split a sequence may take: partials (acc[64], m, l) of every query
  // head and one plan entry; the three regions round up by at most 3 * kAlign
  const size_t per_split = (size_t)num_seqs * num_q_heads * (kHeadDim + 2) * sizeof(float) +
                           (size_t)num_seqs * 2 * sizeof(int32_t);
  int32_t min_chunk = kDecodeMinChunk;
  if (num_splits == 0 && decode_ws_bytes(num_seqs, num_q_heads, keys, 0, min_chunk) > kStaticScratchBytes) {
    const int64_t most = (int64_t)((kStaticScratchBytes - 4 * kAlign) / per_split);
    if (most >= 1) {
      const int64_t c = ((keys + most - 1) / most + 127) / 128 * 128;
      min_chunk = (int32_t)std::max<int64_t>(c, kDecodeMinChunk);
    }
  }
  const size_t need = decode_ws_bytes(num_seqs, num_q_heads, keys, num_splits, min_chunk);
  if (need > kStaticScratchBytes)
    return fail(GPTOSS_ERR_WORKSPACE,
                "the allocation-free decode holds at most %zu bytes of partials; this call needs %zu "
                "(fewer sequences or splits, or gptoss_attn_decode_kv with a workspace)",
                kStaticScratchBytes, need);
  void* ws = nullptr;
  st = hip_status(static_scratch(&ws), "scratch address");
  if (st != GPTOSS_OK) return st;
  p.kind = layout->kind;
  p.kv_sn = layout->strides[0]; p.kv_sp = layout->strides[1]; p.kv_sh = layout->strides[2];
  if (layout->kind == GPTOSS_CACHE_PAGED) {
    p.page_log2 = ilog2_pow2(layout->capacity);
    p.block_table = layout->block_table;
    p.max_pages = layout->max_pages;
    p.num_pages = layout->num_pages;
  } else if (layout->kind == GPTOSS_CACHE_RING) {
    p.ring_slots = layout->capacity;
  }
  return decode_run(p, num_q_heads, keys, keys, ws, kStaticScratchBytes, num_splits, stream, min_chunk);
}

gptoss_status gptoss_qkv_proj_rope(const gptoss_seq_desc* desc, const void* x, int64_t x_row_stride,
                                   int32_t hidden, const void* wq, const void* bq, const void* wk, const void* bk,
                                   const void* wv, const void* bv, const void* table, int32_t table_rows,
                                   int32_t rotary_dim, void* q_out, void* k_out, void* v_out, void* stream) {
  gptoss_status st = check_desc(desc);
  if (st != GPTOSS_OK) return st;
  if (hidden < 64 || hidden % 64 != 0)
    return fail(GPTOSS_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 64", hidden);
  if (desc->num_kv_heads % 4 != 0)
    return fail(GPTOSS_ERR_UNSUPPORTED, "num_kv_heads %d must be a multiple of 4", desc->num_kv_heads);
  const int64_t T = desc_tokens(desc);
  if (T == 0) return GPTOSS_OK;
  if (!x || !wq || !wk || !wv || !q_out || !k_out || !v_out)
    return fail(GPTOSS_ERR_NULL, "x, the weights and the outputs are required");
  if (x_row_stride < hidden || (x_row_stride & 7) || !aligned16(x) || !aligned16(wq) || !aligned16(wk) ||
      !aligned16(wv) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(v_out))
    return fail(GPTOSS_ERR_UNSUPPORTED, "pointers must be 16-byte aligned, x_row_stride >= hidden and a multiple of 8");
  for (const void* b : {bq, bk, bv})
    if (reinterpret_cast<uintptr_t>(b) & 1) return fail(GPTOSS_ERR_UNSUPPORTED, "biases must be 2-byte aligned");
  if ((int64_t)kProjTile * x_row_stride * 2 > (int64_t)INT32_MAX ||
      (int64_t)kProjTile * hidden * 2 > (int64_t)INT32_MAX)
    return fail(GPTOSS_ERR_UNSUPPORTED, "one tile's rows of x or W must span less than 2 GiB");
  if (table) {
    if (rotary_dim != 64 && rotary_dim != 32)
      return fail(GPTOSS_ERR_UNSUPPORTED, "rotary_dim %d: the projection epilogue rotates 64 or 32 dims", rotary_dim);
    if (!aligned16(table)) return fail(GPTOSS_ERR_UNSUPPORTED, "table must be 16-byte aligned");
    if (table_rows < std::max(desc_max_len(desc), 1))
      return fail(GPTOSS_ERR_SHAPE, "table has %d rows, positions up to %d are needed", table_rows,
                  desc_max_len(desc) - 1);
  }
  ProjParams p;
  memset(&p, 0, sizeof p);
  p.x = static_cast<const uint16_t*>(x);
  p.x_st = x_row_stride;
  p.w[0] = static_cast<const uint16_t*>(wq); p.w[1] = static_cast<const uint16_t*>(wk);
  p.w[2] = static_cast<const uint16_t*>(wv);
  p.b[0] = static_cast<const uint16_t*>(bq); p.b[1] = static_cast<const uint16_t*>(bk);
  p.b[2] = static_cast<const uint16_t*>(bv);
  p.out[0] = static_cast<uint16_t*>(q_out); p.out[1] = static_cast<uint16_t*>(k_out);
  p.out[2] = static_cast<uint16_t*>(v_out);
  p.nq = desc->num_q_heads * kHeadDim;
  p.nkv = desc->num_kv_heads * kHeadDim;
  p.tokens = (int32_t)T;
  p.hidden = hidden;
  p.m_tiles = (int32_t)((T + kProjTile - 1) / kProjTile);
  p.n_tiles = (p.nq + 2 * p.nkv) / kProjTile;
  p.batch = desc->batch;
  p.seqlen = desc->seqlen;
  p.cu_seqlens = desc->layout == GPTOSS_THD ? desc->cu_seqlens : nullptr;
  p.table = static_cast<const uint16_t*>(table);
  p.table_rows = table_rows;
  p.rot_half = rotary_dim / 2;
  return hip_status(launch_qkv_proj(p, static_cast<hipStream_t>(stream)), "projection kernel");
}

gptoss_status gptoss_kv_append(const gptoss_kv_layout* layout, void* k_cache, void* v_cache, int32_t num_seqs,
                               int32_t num_kv_heads, int32_t head_dim, int32_t num_new, const void* k_new,
                               const int64_t kn_strides[3], const void* v_new, const int64_t vn_strides[3],
                               const int32_t* cache_seqlens, int32_t max_seqlen, const void* table,
                               int32_t table_rows, int32_t rotary_dim, void* stream) {
  if (num_seqs < 0 || num_new < 0 || max_seqlen < 0) return fail(GPTOSS_ERR_SHAPE, "negative size");
  if (head_dim != kHeadDim) return fail(GPTOSS_ERR_UNSUPPORTED, "head_dim %d unsupported (only 64)", head_dim);
  if (num_kv_heads < 1) return fail(GPTOSS_ERR_SHAPE, "num_kv_heads must be >= 1");
  gptoss_status st = check_layout(layout, max_seqlen, false, 0);
  if (st != GPTOSS_OK) return st;
  if (num_seqs == 0 || num_new == 0) return GPTOSS_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !kn_strides || !vn_strides || !cache_seqlens)
    return fail(GPTOSS_ERR_NULL, "caches, new k / v, their strides and cache_seqlens are required");
  if (!strides_ok(kn_strides, 3) || !strides_ok(vn_strides, 3) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(k_new) || !aligned16(v_new))
    return fail(GPTOSS_ERR_UNSUPPORTED, "pointers must be 16-byte aligned and strides multiples of 8 elements");
  st = check_table(table, table_rows, rotary_dim, std::max(max_seqlen, 1), true);
  if (st != GPTOSS_OK) return st;
  AppendParams p;
  memset(&p, 0, sizeof p);
  p.k = static_cast<uint16_t*>(k_cache);
  p.v = static_cast<uint16_t*>(v_cache);
  p.c_s0 = layout->strides[0]; p.c_sr = layout->strides[1]; p.c_sh = layout->strides[2];
  p.kind = layout->kind;
  p.capacity = layout->capacity;
  if (layout->kind == GPTOSS_CACHE_PAGED) {
    p.page_log2 = ilog2_pow2(layout->capacity);
    p.block_table = layout->block_table;
    p.max_pages = layout->max_pages;
    p.num_pages = layout->num_pages;
  }
  p.kn = static_cast<const uint16_t*>(k_new);
  p.kn_sn = kn_strides[0]; p.kn_st = kn_strides[1]; p.kn_sh = kn_strides[2];
  p.vn = static_cast<const uint16_t*>(v_new);
  p.vn_sn = vn_strides[0]; p.vn_st = vn_strides[1]; p.vn_sh = vn_strides[2];
  p.cache_seqlens = cache_seqlens;
  p.num_seqs = num_seqs;
  p.num_new = num_new;
  p.num_kv_heads = num_kv_heads;
  p.table = static_cast<const uint16_t*>(table);
  p.table_rows = table_rows;
  p.rot_chunks = rotary_dim / 16;
  return hip_status(launch_kv_append(p, static_cast<hipStream_t>(stream)), "KV append kernel");
}

gptoss_status gptoss_check_lengths(const int32_t* cu_seqlens, int32_t batch, int32_t total_tokens,
                                   const int32_t* cache_seqlens, int32_t num_seqs, int32_t max_cache_len,
                                   int32_t* result, void* stream) {
  if (!result) return fail(GPTOSS_ERR_NULL, "result (3 device int32) is required");
  if (cu_seqlens && batch < 0) return fail(GPTOSS_ERR_SHAPE, "batch must be >= 0");
  if (cache_seqlens && (num_seqs < 0 || max_cache_len < 1))
    return fail(GPTOSS_ERR_SHAPE, "num_seqs must be >= 0 and max_cache_len >= 1");
  return hip_status(launch_check_lengths(cu_seqlens, cu_seqlens ? batch : 0, total_tokens, cache_seqlens,
                                         cache_seqlens ? num_seqs : 0, max_cache_len, result,
                                         static_cast<hipStream_t>(stream)),
                    "length check kernel");
}

}  // extern "C"
