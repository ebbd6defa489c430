// Internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptoss {

constexpr int kHeadDim = 64;     // D: the only head width the kernels are built for
constexpr int kGroup = 8;        // query heads per KV head (64 / 8 in GPT-OSS)
constexpr int kMaxPairs = 32;    // rotary_dim / 2

// ---- RoPE table ----
struct TableParams {
  double omega[kMaxPairs];
  double concentration;
  int32_t half;                  // rotary_dim / 2
  int32_t num_positions;
  uint16_t* table;               // [num_positions, 2*half]
};
hipError_t launch_rope_table(const TableParams& p, hipStream_t stream);

// ---- standalone q/k rotation ----
struct RopeQKParams {
  const uint16_t* x;             // one tensor (q or k)
  int64_t s_b, s_t, s_h;         // element strides of batch, token, head
  uint16_t* y;                   // contiguous output [.., tokens, heads, 64]
  int32_t batch, tokens, heads;  // BSHD: batch x seqlen; THD: batch = 1, tokens = T
  const int32_t* cu_seqlens;     // THD positions (NULL for BSHD)
  int32_t num_seqs;
  const uint16_t* table;         // [table_rows, rotary_dim]: cos of the rotary_dim / 2 pairs, then sin
  int32_t table_rows;
  int32_t rot_chunks;            // rotary_dim / 16: 8-dim chunks in each half of the rotated part
  int32_t pos0;                  // BSHD: token s is at position pos0 + s (a shard of a longer sequence)
};
hipError_t launch_rope_qk(const RopeQKParams& p, hipStream_t stream);

// ---- prefill ----
struct PrefillParams {
  const uint16_t* q; int64_t q_sb, q_st, q_sh;
  const uint16_t* k; int64_t k_sb, k_st, k_sh;
  const uint16_t* v; int64_t v_sb, v_st, v_sh;
  uint16_t* o; int64_t o_sb, o_st, o_sh;
  const float* sinks;            // always a readable [Hq] array (see no_sink)
  int32_t no_sink;               // 1: no sink term (the sinks are loaded and ignored)
  const uint16_t* table;         // NULL: q (and k) already rotated
  int32_t table_rows;
  int32_t rot_chunks;            // rotary_dim / 16: 4 rotates all 64 dims, 1..3 the first 16, 32, 48
  int32_t batch;                 // BSHD batch, or number of THD sequences
  int32_t seqlen;                // BSHD S, or THD total tokens
  int32_t num_kv_heads;
  int32_t window;
  float scale_log2;              // softmax_scale * log2(e)
  int32_t q_blocks;              // BSHD: ceil(S / BQ); THD: max work items per KV head
  const int32_t* cu_seqlens;     // THD
  const int2* work;              // THD work list (seq, q block), longest first
  const int32_t* work_count;     // THD: number of valid entries in `work`
  float* lse;                    // optional fp32 [tokens, num_q_heads] log-sum-exp per row (NULL: none)
  // BSHD shards of a longer sequence (whole sequences: 0, seqlen, 0, 0): query s
  // sits at position s + q_shift of the keys' coordinates; kv_len keys per
  // sequence; q and k rotated with table rows offset by q_pos0 and k_pos0
  int32_t q_shift;
  int32_t kv_len;
  int32_t q_pos0, k_pos0;
  // window runs (launch_window_runs): query blocks per work group and runs per sequence
  int32_t run_len, runs_per_seq;
  int32_t pair_first;            // BSHD window runs: > 0 splits each two neighbouring runs unevenly (below)
};
enum KRotation { KROT_NONE = 0, KROT_FUSED = 1 };
hipError_t launch_prefill(const PrefillParams& p, bool thd, int krot, hipStream_t stream);
// THD work list of (sequence, block of bq query positions), longest first
hipError_t launch_thd_schedule(const int32_t* cu_seqlens, int32_t num_seqs, int32_t bq, int32_t max_items,
                               int2* work, int32_t* work_count, hipStream_t stream);
constexpr int kPrefillBQ = 32;   // query positions per work item
// Window layers of whole sequences (BSHD or THD), window a multiple of 32 and at
// most 128: one work group of 8 waves per run of run_len consecutive 32-position
// query blocks of one (sequence, KV head); k is rotated as it enters the work
// group's LDS (no separate K pass). BSHD: batch * runs_per_seq runs. THD: the runs
// come from launch_thd_schedule's list built with bq = 32 * run_len (work,
// work_count; q_blocks = its capacity).
hipError_t launch_window_runs(const PrefillParams& p, bool thd, hipStream_t stream);
constexpr int kWindowRunsTarget = 512;      // BSHD work groups to aim for (two per CU, resident together)
constexpr int kWindowRunsTargetThd = 1024;  // THD: two rounds, so unequal runs can balance

// ---- prefill backward ----
struct BackwardParams {
  const uint16_t* q; int64_t q_sb, q_st, q_sh;     // rotated q (bf16)
  // Non-NULL: the dq kernel reads the caller's un-rotated q here, rotates it on
  // load (all 64 dims) and writes the rotated rows to q_rot (= q above,
  // contiguous) for the dk / dv kernel after it.
  const uint16_t* q_in; int64_t qi_sb, qi_st, qi_sh;
  uint16_t* q_rot;
  const uint16_t* k; int64_t k_sb, k_st, k_sh;     // rotated k
  const uint16_t* v; int64_t v_sb, v_st, v_sh;
  const uint16_t* o; int64_t o_sb, o_st, o_sh;     // forward output
  const uint16_t* dout; int64_t do_sb, do_st, do_sh;
  const float* lse;              // [tokens, Hq] natural log, from the forward
  float* ld;                     // workspace [Hq, tokens, 2]: per row lse in log2 units (+inf for a row
                                 // without any term) and -D = -<dO, o>
  int64_t tokens;                // rows of the token-major tensors (BSHD batch * seqlen, THD seqlen)
  const float* sinks;
  float* dsinks;                 // [Hq]
  float* dsink_part;             // workspace [Hq, dsink_items]: each dq work item's share of dsigma per head
  int32_t dsink_items;           // dq work items (BSHD batch * q_blocks, THD max entries of work_q)
  uint16_t* dq; uint16_t* dk; uint16_t* dv;   // contiguous [tokens, H, 64]
  const uint16_t* table;         // NULL: q and k were given already rotated (no rotation back)
  int32_t table_rows;
  int32_t batch;                 // BSHD batch, or number of THD sequences
  int32_t seqlen;                // BSHD S, or THD total tokens
  int32_t num_kv_heads;
  int32_t window;
  float scale;                   // softmax_scale
  float scale_log2;              // softmax_scale * log2(e)
  const int32_t* cu_seqlens;     // THD
  int32_t q_blocks;              // BSHD: ceil(S / 32); THD: max entries of work_q
  int32_t k_tiles;               // BSHD: ceil(S / 128) key tiles; THD: max entries of work_k
  int32_t kv_pairs;              // BSHD full causal: each dk / dv work group takes two key tiles (below)
  const int2* work_q; const int32_t* count_q;   // THD: (sequence, query block), most keys first
  const int2* work_k; const int32_t* count_k;   // THD: (sequence, key tile counted from the end), most queries first
};
hipError_t launch_backward(const BackwardParams& p, bool thd, hipStream_t stream);
// x[0 .. n) = value (a kernel, not a memset: safe inside captured graphs)
hipError_t launch_fill_f32(float* x, int32_t n, float value, hipStream_t stream);
constexpr int kBackwardNK = 64;   // keys per K / V tile of the backward dq kernel
constexpr int kBackwardKT = 128;  // keys per work item of the backward dk / dv kernel

// ---- decode ----
struct DecodeParams {
  const uint16_t* q; int64_t q_sn, q_sh;
  const uint16_t* k; const uint16_t* v; int64_t kv_sn, kv_sp, kv_sh;
  const int32_t* cache_seqlens;
  int32_t max_cache_len;
  int32_t num_seqs, num_kv_heads;
  int32_t window;
  float scale_log2;
  const float* sinks;
  const uint16_t* table;
  int32_t table_rows;
  int32_t rot_chunks;            // rotary_dim / 16 (4: all 64 dims)
  int32_t num_splits;            // split slots per (sequence, KV head) in the partial buffers
  int32_t chunk_fixed;           // > 0: keys per split given by the caller; 0: planned on the device
  int32_t target_chunks;         // planned: aim for about this many (sequence, split) work items
  int32_t min_chunk;             // planned: fewest keys per split (a multiple of 128, >= kDecodeMinChunk)
  int32_t* plan;                 // device: keys per split, item count, then int2 (sequence, split) items
  int32_t max_items;             // work groups launched for the split kernel
  int32_t direct_chunk;          // > 0: one split of this many keys per sequence, no plan (item = sequence)
  float* part_o;                 // [N, Hkv, splits, 8, 64]
  float* part_ml;                // [N, Hkv, splits, 8, 2]
  uint16_t* o; int64_t o_sn, o_sh;
  // cache layout (kCacheContiguous: kv_sn = sequence stride; kCachePaged: kv_sn =
  // page stride, rows per page = 1 << page_log2; kCacheRing: ring_slots rows per
  // sequence, the visible positions of a window layer with window == ring_slots)
  int32_t kind;
  int32_t page_log2;
  int32_t ring_slots;
  const int32_t* block_table;    // [num_seqs, max_pages]
  int32_t max_pages, num_pages;
};
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
constexpr int kCacheContiguous = 0, kCachePaged = 1, kCacheRing = 2;   // gptoss_cache_kind

// ---- q/k/v projection with the RoPE in its epilogue ----
struct ProjParams {
  const uint16_t* x; int64_t x_st;           // [tokens, hidden], row stride (elements)
  const uint16_t* w[3];                      // q, k, v weights [out, hidden], rows contiguous
  const uint16_t* b[3];                      // bf16 biases [out] (NULL: none)
  uint16_t* out[3];                          // [tokens, out] contiguous
  int32_t nq, nkv;                           // out widths: Hq * 64 and Hkv * 64
  int32_t tokens, hidden;
  int32_t m_tiles, n_tiles;
  int32_t batch, seqlen;                     // positions: BSHD p = t mod seqlen; THD p = t - cu[n]
  const int32_t* cu_seqlens;
  const uint16_t* table;                     // NULL: no rotation
  int32_t table_rows;
  int32_t rot_half;                          // rotary_dim / 2 (16 or 32)
};
hipError_t launch_qkv_proj(const ProjParams& p, hipStream_t stream);

// ---- merge of partial attention outputs (shards of the keys) ----
struct MergeParams {
  const uint16_t* o; int64_t o_sp, o_st, o_sh;   // bf16 partial outputs [parts, tokens, Hq, 64]
  const float* lse; int64_t l_sp;                // fp32 [parts, tokens * Hq]: natural log, -inf = no keys
  const float* sinks;                            // [Hq], -inf allowed
  uint16_t* out; int64_t out_st, out_sh;         // bf16 [tokens, Hq, 64]
  float* lse_out;                                // optional [tokens * Hq]
  int32_t parts, tokens, num_q_heads;
};
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);

// ---- check of device-resident lengths ----
hipError_t launch_check_lengths(const int32_t* cu_seqlens, int32_t batch, int32_t total_tokens,
                                const int32_t* cache_seqlens, int32_t num_seqs, int32_t max_cache_len,
                                int32_t* result, hipStream_t stream);
constexpr int kProjTile = 256;   // tokens and output features per work group

// ---- KV append ----
struct AppendParams {
  uint16_t* k; uint16_t* v; int64_t c_s0, c_sr, c_sh;   // cache strides: sequence or page, row, head
  int32_t kind, capacity, page_log2;
  const int32_t* block_table;
  int32_t max_pages, num_pages;
  const uint16_t* kn; int64_t kn_sn, kn_st, kn_sh;
  const uint16_t* vn; int64_t vn_sn, vn_st, vn_sh;
  const int32_t* cache_seqlens;
  int32_t num_seqs, num_new, num_kv_heads;
  const uint16_t* table;         // NULL: k stored as given
  int32_t table_rows;
  int32_t rot_chunks;            // rotary_dim / 16
};
hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream);
constexpr int kDecodeMinChunk = 512;   // smallest planned split (keys)

// Scratch of the allocation-free decode entry point: a file-scope __device__
// array of kStaticScratchBytes per GPU. static_scratch() returns its address on
// the current device (looked up once per device with hipGetSymbolAddress).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch(void** ptr);

}  // namespace gptoss
