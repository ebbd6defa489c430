// Flash-style prefill attention for GPT-OSS on gfx950: learned per-head sink,
// grouped-query attention (8 query heads per KV head), causal or sliding-window
// mask, YaRN RoPE applied while q and k tiles are loaded.
//
// What is computed (page "nemo_automodel.components.models.gpt_oss.layers",
// GptOssAttention: sinks, sliding_window, softmax_scale = head_dim ** -0.5;
// Transformers v4.55.0 release notes, "Architecture": alternating full-context
// and sliding 128-token-window layers, a per-head sink adding a term to the
// softmax denominator):
//   o[i,h] = sum_{j visible} exp(s_ij - M) v[j,g] / (exp(sigma_h - M) + sum_{j visible} exp(s_ij - M))
// with s_ij = tau <q~_i, k~_j>, g = h / 8, visible: j <= i and (W == 0 or i - j < W).
//
// Work item: (sequence, KV head g, block of BQ = 32 query positions). Its 256
// query rows are the 8 heads of group g x 32 positions, so every K/V tile is
// read from HBM once and staged in LDS once for the whole GQA group. Each of
// 4 waves owns 64 query rows (2 heads x 32 positions) as four 16-column blocks
// (CB = 4; window layers use 8 waves of 32 rows, CB = 2). Per KV tile of 64
// keys a CB = 4 wave runs 32 MFMAs for S^T = K Q^T and 32 for O^T = V^T P^T
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation). The softmax
// runs on S^T, whose accumulator layout is already the B-operand layout P^T
// needs (keys permuted consistently between V^T and P^T). V^T comes straight
// from the row-major V tile in LDS through ds_read_b64_tr_b16.
//
// Softmax in log2 units against a per-row reference seeded with the sink
// logit (the sink term exp(sigma - ref) = 1 starts the row sum); a row with no
// sink term (sigma = -inf, or a shard of the keys) takes the largest score of
// the first step in which it sees a key. The reference then only moves in a
// rare fallback (a tile's partial row sum beyond 2^100), so the hot loop has
// no running max and no accumulator rescale. Tiles fully visible to every
// query of the item skip the mask; tiles fully hidden are never visited.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

constexpr int BQ = kPrefillBQ;  // 32 query positions per item
constexpr int NK = 64;          // keys per KV tile
constexpr int KS = 80;          // LDS row stride of the K tile (160 B): half the bank conflicts of 144 B (measured)
constexpr int VS = 80;          // LDS row stride of the V tile (160 B): conflict-free tr16 reads
constexpr float kSumLimit = 0x1p100f;   // bound of a tile's partial row sum before the reference moves
constexpr float kRaiseGap = 8.0f;       // the reference moves to a new max more than this far above it

__device__ __forceinline__ float wave_xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_xor_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// CB = 16-column blocks per wave: 4 (2 heads x 32 positions, 4 waves of up to
// 256 VGPRs, 2 per SIMD) or 2 (1 head x 32 positions, 8 waves of up to 128
// VGPRs, 4 per SIMD: twice the waves to hide latency, for short work items).
template <int CB> struct Shape {
  static constexpr int kWaves = 16 / CB;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kThreadsPerRow = kThreads / NK;   // threads staging one 128-byte K/V row
  static constexpr int kChunks = 8 / kThreadsPerRow;     // 16-byte chunks per thread: 2 or 1
  static constexpr int kWavesPerEU = CB == 4 ? 2 : 4;
};

template <int N> struct KeyCount { static constexpr int value = N; };   // keys per compute step

// Staging: ALL = false streams the item's key tiles through two LDS buffers,
// loading tile t + 1 while tile t is computed. ALL = true (short windows: at
// most kAllTiles tiles per item) loads every tile in the prologue, together
// with q, so the item waits for memory once and then runs its tiles with no
// further loads or barriers.
constexpr int kAllTiles = 3;

template <bool ROTQ, bool ROTK, bool THD, int CB, bool ALL>
__global__ __launch_bounds__(Shape<CB>::kThreads) __attribute__((amdgpu_waves_per_eu(Shape<CB>::kWavesPerEU)))
void prefill_kernel(PrefillParams p) {
  static_assert(CB == 4 || (CB == 2 && !ROTK), "the fused K rotation needs both halves of a row in one thread");
  using SH = Shape<CB>;
  constexpr int NBUF = ALL ? kAllTiles : 2;
  __shared__ __attribute__((aligned(16))) bf16_t lds_k[NBUF * NK * KS];   // tile b at b * NK * KS
  __shared__ __attribute__((aligned(16))) bf16_t lds_v[NBUF * NK * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;   // MFMA column (query) / row (key, d) inside a 16-block
  const int grp = lane >> 4;   // 16-lane group

  // ---- work item: consecutive blocks take consecutive KV heads, so with 8 KV
  // heads every XCD (blocks are dealt round-robin over the 8 XCDs) serves one
  // KV head and keeps its K/V in its own L2.
  const int Hkv = p.num_kv_heads;
  const int item = blockIdx.x / Hkv;
  const int g = blockIdx.x - item * Hkv;
  int j, L;
  int64_t bb_off_q, bb_off_k, bb_off_v, bb_off_o;  // batch offsets
  int64_t row0;                                    // token-major row of the batch's first token (lse)
  int ts;                                          // first token of the sequence
  if (THD) {
    if (item >= __ldg(p.work_count)) return;
    const int2 w = p.work[item];
    j = w.y;
    const int n = min(max(w.x, 0), p.batch - 1);
    ts = min(max(__ldg(p.cu_seqlens + n), 0), p.seqlen);
    const int te = min(max(__ldg(p.cu_seqlens + n + 1), ts), p.seqlen);
    L = te - ts;
    bb_off_q = bb_off_k = bb_off_v = bb_off_o = 0;
    row0 = 0;
  } else {
    const int r = item / p.batch;
    const int b = item - r * p.batch;
    j = p.q_blocks - 1 - r;     // longest (most keys) first
    ts = 0;
    L = p.seqlen;
    bb_off_q = b * p.q_sb; bb_off_k = b * p.k_sb; bb_off_v = b * p.v_sb; bb_off_o = b * p.o_sb;
    row0 = (int64_t)b * p.seqlen;
  }
  const int q0 = j * BQ;
  if (j < 0 || q0 >= L) return;
  const int qlast = min(q0 + BQ, L) - 1;
  const int W = p.window;
  const uint32_t weff = (W > 0) ? (uint32_t)W : 0x7FFFFFFFu;   // keys visible: 0 <= qpos - kpos < weff
  // Query positions in the keys' coordinates: a shard of a longer sequence has
  // its queries q_shift positions after its first key (0 for a whole sequence)
  // and its own key count.
  const int qk0 = q0 + p.q_shift, qklast = qlast + p.q_shift;
  const int Lk = THD ? L : p.kv_len;
  const int kv_lo = (W > 0) ? max(0, qk0 - W + 1) : 0;
  const int kv_hi = min(qklast + 1, Lk);
  const int ntiles = (kv_hi - kv_lo + NK - 1) / NK;
  const float sl = p.scale_log2;

  // ---- K/V tile staging: thread -> (row, 8-dim chunk cc and cc + 4), read
  // with raw buffer loads: a uniform base per tile in scalar registers, one
  // 32-bit per-lane offset, and a range that ends after the item's last key,
  // so rows past it read as zeros (they lie after every query of the item; the
  // causal mask gives them weight 0). ----
  const int srow = tid / SH::kThreadsPerRow;
  const int scc = tid % SH::kThreadsPerRow;   // chunks scc (and scc + 4 when a thread stages two)
  const int32_t krow_b = (int32_t)p.k_st * 2, vrow_b = (int32_t)p.v_st * 2;   // row bytes (< 2^31 / 64: host check)
  const char* k_tile0 = reinterpret_cast<const char*>(p.k + bb_off_k + (int64_t)(ts + kv_lo) * p.k_st + (int64_t)g * p.k_sh);
  const char* v_tile0 = reinterpret_cast<const char*>(p.v + bb_off_v + (int64_t)(ts + kv_lo) * p.v_st + (int64_t)g * p.v_sh);
  const uint32_t koff = (uint32_t)(srow * krow_b + 16 * scc);
  const uint32_t voff = (uint32_t)(srow * vrow_b + 16 * scc);
  // A tile past the item's last one gets an empty range: its loads return
  // zeros without touching memory. The range covers at most the tile's own NK
  // rows, so it stays below 2^31 bytes for any sequence length.
  struct Stage { uint4 k1, k2, v1, v2, c, s; };
  auto load_tile = [&](int t, Stage& st) {
    const int rows = min(kv_hi - (kv_lo + t * NK), NK);   // keys of the item in this tile
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_tile0 + (int64_t)t * NK * krow_b, (rows - 1) * krow_b + 2 * kHeadDim);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_tile0 + (int64_t)t * NK * vrow_b, (rows - 1) * vrow_b + 2 * kHeadDim);
    st.k1 = ldb16(rk, koff); st.v1 = ldb16(rv, voff);
    if (SH::kChunks == 2) { st.k2 = ldb16(rk, koff + 64); st.v2 = ldb16(rv, voff + 64); }
    if (ROTK) {
      const int kpos = kv_lo + t * NK + srow;
      const bf16_t* tp = p.table + (int64_t)min(min(kpos, kv_hi - 1) + p.k_pos0, p.table_rows - 1) * kHeadDim + 8 * scc;
      st.c = ldg16(tp); st.s = ldg16(tp + 32);
    }
  };
  auto store_tile = [&](int buf, const Stage& st) {
    uint4 k1 = st.k1, k2 = st.k2;
    if (ROTK) rope8(st.k1, st.k2, st.c, st.s, k1, k2);
    bf16_t* kd = lds_k + buf * NK * KS + srow * KS + 8 * scc;
    bf16_t* vd = lds_v + buf * NK * VS + srow * VS + 8 * scc;
    *reinterpret_cast<uint4*>(kd) = k1;
    *reinterpret_cast<uint4*>(vd) = st.v1;
    if (SH::kChunks == 2) {
      *reinterpret_cast<uint4*>(kd + 32) = k2;
      *reinterpret_cast<uint4*>(vd + 32) = st.v2;
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T), rotated on load. Every
  // independent load (the first K/V tile or, with ALL, every tile; q, table
  // rows, sinks) is issued before any of them is used, so the work item pays
  // one memory latency, not several. Rows past the end load a valid row and are
  // never stored. ----
  Stage st[ALL ? kAllTiles : 1];
  if (ALL) {
#pragma unroll
    for (int t = 0; t < kAllTiles; ++t) load_tile(t, st[t]);
  } else if (ntiles > 0) {
    load_tile(0, st[0]);
  }
  bf16x8_t qf[CB][2];
  int qpos[2], qkp[2];   // query rows, and their positions in the keys' coordinates
  qpos[0] = q0 + col;
  qpos[1] = q0 + 16 + col;
  qkp[0] = qpos[0] + p.q_shift;
  qkp[1] = qpos[1] + p.q_shift;
  int vbase[2];
  uint32_t vlim[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int lo = max(0, qkp[c] - kv_hi + 1);
    vbase[c] = qkp[c] - lo;
    vlim[c] = (uint32_t)max((int)weff - lo, 0);
  }
  // Every load of the prologue is issued before any result is used, with no
  // branch between them: a branch between dependent loads makes the wait at its
  // join cover all loads in flight, which serialises the memory round trips.
  // The table row depends only on the position, so the lane's two query rows
  // need two table rows for all CB column blocks.
  uint4 qx[CB][2], qt[2][2];
  float sink_raw[CB];
  const bool rot_all = ROTQ && p.rot_chunks == kHeadDim / 16;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int head = g * kGroup + wave * (CB / 2) + (cb >> 1);
    const int pos = min(qpos[cb & 1], qlast);
    const bf16_t* qp = p.q + bb_off_q + (int64_t)(ts + pos) * p.q_st + (int64_t)head * p.q_sh;
    qx[cb][0] = ldg16(qp + 8 * grp);
    qx[cb][1] = ldg16(qp + 32 + 8 * grp);
    sink_raw[cb] = __ldg(p.sinks + head);
  }
  if (rot_all) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int pos = min(qpos[c], qlast);
      const bf16_t* tp = p.table + (int64_t)min(pos + p.q_pos0, p.table_rows - 1) * kHeadDim + 8 * grp;
      qt[c][0] = ldg16(tp);
      qt[c][1] = ldg16(tp + 32);
    }
  } else if (ROTQ) {
    // partial rotary: each of the lane's two chunks with its pair partner (prologue only)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int head = g * kGroup + wave * (CB / 2) + (cb >> 1);
      const int pos = min(qpos[cb & 1], qlast);
      const bf16_t* qp = p.q + bb_off_q + (int64_t)(ts + pos) * p.q_st + (int64_t)head * p.q_sh;
      const bf16_t* tp = p.table + (int64_t)min(pos + p.q_pos0, p.table_rows - 1) * (16 * p.rot_chunks);
      qx[cb][0] = rope_chunk_partial(qp, tp, grp, p.rot_chunks, qx[cb][0]);
      qx[cb][1] = rope_chunk_partial(qp, tp, grp + 4, p.rot_chunks, qx[cb][1]);
    }
  }
  float ref[CB], lsum[CB];
  bool unset[CB];        // column without a sink term whose reference is not set yet
  bool seeding = false;  // wave-uniform: some column of the wave is unset
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    uint4 y1 = qx[cb][0], y2 = qx[cb][1];
    if (rot_all) rope8(qx[cb][0], qx[cb][1], qt[cb & 1][0], qt[cb & 1][1], y1, y2);
    qf[cb][0] = as_bf16x8(y1);
    qf[cb][1] = as_bf16x8(y2);
    // reference = the sink logit (log2 units); the sink term exp2(sigma - ref) = 1
    // is counted once, in lane group 0. Without a sink term (sigma = -inf, or a
    // shard of the keys) the reference is taken from the first step holding a
    // visible key of the column: its largest score (see compute).
    const float sink = p.no_sink ? -INFINITY : sink_raw[cb] * kLog2e;
    const bool has_sink = sink > -INFINITY;
    ref[cb] = has_sink ? sink : 0.0f;
    lsum[cb] = (grp == 0 && has_sink) ? 1.0f : 0.0f;
    unset[cb] = !has_sink;
    seeding |= !has_sink;
  }
  seeding = __any(seeding);

  f32x4_t oacc[4][CB];  // [d block][column block]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < CB; ++b) oacc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (ALL) {
#pragma unroll
    for (int t = 0; t < kAllTiles; ++t) store_tile(t, st[t]);
  } else if (ntiles > 0) {
    store_tile(0, st[0]);
  }
  __syncthreads();

  // Window items whose keys start W - 1 before their first query (a multiple-of-32
  // window, not a shard): the first 32-key step holds key j visible to query row i
  // iff j >= i, and the step W / 32 later iff j < i; every step between is fully
  // visible. ge[kb][r][c] is that test for this lane's scores (key kb*16 + 4*grp + r,
  // row col + 16c), computed once instead of comparing positions in those steps.
  bool ge[2][4][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) ge[kb][r][c] = kb * 16 + 4 * grp + r >= col + 16 * c;

  // ---- one compute step over NKT keys (64: a whole tile, 32: half of one) whose
  // K and V rows start at kt and vt in LDS; tile0 = position of the first key;
  // pat: 0 = general mask, 1 / 2 = the window's first / last step (see ge) ----
  auto compute = [&](auto nkt_tag, const bf16_t* kt, const bf16_t* vt, int tile0, int pat)
      __attribute__((always_inline)) {
    constexpr int NKT = decltype(nkt_tag)::value;
    constexpr int KBN = NKT / 16;   // 16-key blocks of S^T
    constexpr int KSN = NKT / 32;   // 32-key slices of P^T (one PV MFMA each)

    // ---- S^T = K Q^T: sacc[kb][cb] element r = key (kb*16 + 4*grp + r), query col ----
    f32x4_t sacc[KBN][CB];
#pragma unroll
    for (int kb = 0; kb < KBN; ++kb) {
      const bf16_t* krow = kt + (kb * 16 + col) * KS + 8 * grp;
      const bf16x8_t a0 = as_bf16x8(*reinterpret_cast<const uint4*>(krow));
      const bf16x8_t a1 = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 32));
      // the CB first halves, then the CB second halves accumulating in place: each
      // dependent MFMA issues CB - 1 independent ones after the one it waits for
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) sacc[kb][cb] = mfma16(a0, qf[cb][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) sacc[kb][cb] = mfma16(a1, qf[cb][1], sacc[kb][cb]);
    }

    // ---- mask: only steps that are not fully visible to every query of the item.
    // visible <=> lo <= qpos - kpos < weff, one unsigned compare (branch free):
    // (qpos - lo - kpos) < (weff - lo) with the column's vbase = qpos - lo and
    // vlim = weff - lo. lo = 0 for a whole sequence; a shard of the keys can end
    // before its queries, and then lo = qpos - kv_hi + 1 hides the rows past the
    // keys (they read as zeros) ----
    const bool full = (tile0 + NKT - 1 <= qk0) && (W == 0 || qklast - tile0 < W) && (tile0 + NKT <= kv_hi);
    if constexpr (NKT == 32) {
      if (!full && pat != 0) {
        const bool first = pat == 1;
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
              sacc[kb][cb][r] = (ge[kb][r][cb & 1] == first) ? sacc[kb][cb][r] : -INFINITY;
      }
    }
    if (!full && pat == 0) {
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kpos = tile0 + kb * 16 + 4 * grp + r;
          const bool vis0 = (uint32_t)(vbase[0] - kpos) < vlim[0];
          const bool vis1 = (uint32_t)(vbase[1] - kpos) < vlim[1];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const bool vis = (cb & 1) ? vis1 : vis0;
            sacc[kb][cb][r] = vis ? sacc[kb][cb][r] : -INFINITY;
          }
        }
    }

    // ---- a column without a sink term takes its reference from the first step in
    // which it sees a key: the largest score of that step, so the step's sum is at
    // least 1 and no later exponent can underflow the whole row. Rows whose logits
    // all lie far below 0 would otherwise sum to 0 against a fixed reference. ----
    if (seeding) {   // wave-uniform; only while some column of the wave is unset
      bool left = false;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        float v = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) v = __builtin_fmaxf(v, sacc[kb][cb][r] * sl);
        const float mt = wave_xor_max(v);          // the column's max (log2 units), -inf if no key
        if (unset[cb] && mt > -INFINITY) {         // uniform across the 4 lanes of the column
          ref[cb] = mt;
          unset[cb] = false;
        }
        left |= unset[cb];
      }
      seeding = __any(left);
    }

    // ---- online softmax against a fixed reference (log2 units) ----
    // p = exp2(s*tau*log2(e) - ref). The reference starts at the sink logit and
    // only moves when a step's bf16 row sum leaves [0, 2^100] (a score that far
    // above the reference, or an overflow): then the step's true column max
    // becomes the reference, l and O are rescaled and the step is redone. Values
    // below or above the reference by up to 2^100 lose no relative precision in
    // fp32 / bf16, so the result is the same ratio as with a running max.
    bf16x8_t pf[CB][KSN];
    float tsum[CB];
    bool bad = false;
    auto exp_tile = [&](int cb) __attribute__((always_inline)) {
      uint32_t w[2 * KBN];
      const float nr = -ref[cb];
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb) {
        w[2 * kb] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][cb][0], sl, nr)),
                                __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][cb][1], sl, nr)));
        w[2 * kb + 1] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][cb][2], sl, nr)),
                                    __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][cb][3], sl, nr)));
      }
      // row sum of the bf16-rounded probabilities actually used by PV
      float ts = 0.0f;
#pragma unroll
      for (int i = 0; i < 2 * KBN; ++i) ts = add_bf16x2(w[i], ts);
      tsum[cb] = ts;
      // keys pi(grp, e) of slice ks: e < 4 -> 4*grp + e of key block 2ks, e >= 4 -> of key block 2ks+1
#pragma unroll
      for (int ks = 0; ks < KSN; ++ks)
        pf[cb][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(w[4 * ks], w[4 * ks + 1], w[4 * ks + 2], w[4 * ks + 3]));
    };
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      exp_tile(cb);
      bad |= !(tsum[cb] <= kSumLimit);
    }
    if (__any(bad)) {   // rare, wave-uniform
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        float v = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) v = __builtin_fmaxf(v, sacc[kb][cb][r]);
        const float mt = wave_xor_max(v) * sl;     // the column's max (log2 units)
        if (mt > ref[cb] + kRaiseGap) {            // uniform across the 4 lanes of the column
          const float f = __builtin_amdgcn_exp2f(ref[cb] - mt);
          lsum[cb] *= f;
#pragma unroll
          for (int db = 0; db < 4; ++db) oacc[db][cb] *= f;
          ref[cb] = mt;
        }
        exp_tile(cb);
      }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) lsum[cb] += tsum[cb];

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ks = 0; ks < KSN; ++ks) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16_t* vb = vt + (32 * ks + 4 * grp + (col >> 2)) * VS + 16 * db + 4 * (col & 3);
        const uint2 lo = lds_read_tr16(vb);
        const uint2 hi = lds_read_tr16(vb + 16 * VS);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) oacc[db][cb] = mfma16(a, pf[cb][ks], oacc[db][cb]);
      }
    }
  };

  if (ALL) {
    // every tile is in LDS, rows in key order: 32-key steps, and only the steps
    // holding keys of the item (a 159-key window span takes 5 steps, not 6)
    const int nsteps = (kv_hi - kv_lo + 31) / 32;
    const bool fixed = W > 0 && (W & 31) == 0 && p.q_shift == 0 && qk0 >= W - 1;   // kv_lo = qk0 - W + 1
    for (int u = 0; u < nsteps; ++u) {
      const int pat = fixed ? (u == 0 ? 1 : (u == W / 32 ? 2 : 0)) : 0;
      compute(KeyCount<32>(), lds_k + u * 32 * KS, lds_v + u * 32 * VS, kv_lo + 32 * u, pat);
    }
  } else {
    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      if (t + 1 < ntiles) load_tile(t + 1, st[0]);
      compute(KeyCount<NK>(), lds_k + buf * NK * KS, lds_v + buf * NK * VS, kv_lo + t * NK, 0);
      if (t + 1 < ntiles) store_tile(buf ^ 1, st[0]);
      __syncthreads();
    }
  }

  // ---- epilogue: o = acc / l, bf16 store; lane holds d = 16*db + 4*grp + r ----
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float l = wave_xor_sum(lsum[cb]);
    const int pos = qpos[cb & 1];
    if (pos > qlast) continue;
    const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
    const int head = g * kGroup + wave * (CB / 2) + (cb >> 1);
    if (p.lse && grp == 0) {
      // natural log of exp(sigma) + sum exp(s): the row sum is kept relative to
      // exp2(ref) in log2 units; -inf for a row with nothing visible and no sink
      p.lse[(row0 + ts + pos) * (Hkv * kGroup) + head] = (l > 0.0f) ? (ref[cb] + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
    }
    bf16_t* op = p.o + bb_off_o + (int64_t)(ts + pos) * p.o_st + (int64_t)head * p.o_sh + 4 * grp;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      uint2 v;
      v.x = pack_bf16x2(oacc[db][cb][0] * inv, oacc[db][cb][1] * inv);
      v.y = pack_bf16x2(oacc[db][cb][2] * inv, oacc[db][cb][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * db) = v;
    }
  }
}

// Work list for packed sequences: every (sequence n, query block jb) with
// jb < ceil(L_n / bq), ordered by jb descending (the blocks with the most keys
// first), sequences ascending within one jb. One work group of 1024 threads.
constexpr int kSchedThreads = 1024;
constexpr int kSchedMaxBlocks = 8192;   // query blocks per sequence (L <= 262144)
constexpr int kSchedMaxSeqs = 4096;

__global__ __launch_bounds__(kSchedThreads) void thd_schedule_kernel(const int32_t* cu, int32_t num_seqs, int32_t bq,
                                                                     int32_t max_items, int2* work,
                                                                     int32_t* work_count) {
  __shared__ int32_t nb[kSchedMaxSeqs];
  __shared__ int32_t cnt[kSchedMaxBlocks];
  __shared__ int32_t part[kSchedThreads];
  __shared__ int32_t jmax_s;
  const int tid = threadIdx.x;
  if (tid == 0) jmax_s = 0;
  __syncthreads();
  int local_max = 0;
  for (int n = tid; n < num_seqs; n += kSchedThreads) {
    const int a = __ldg(cu + n), b = __ldg(cu + n + 1);
    const int len = max(b - a, 0);
    const int q = min((len + bq - 1) / bq, kSchedMaxBlocks);
    nb[n] = q;
    local_max = max(local_max, q);
  }
  atomicMax(&jmax_s, local_max);
  __syncthreads();
  const int J = jmax_s;
  // count[jb] = number of sequences with more than jb blocks
  for (int jb = tid; jb < J; jb += kSchedThreads) {
    int c = 0;
    for (int n = 0; n < num_seqs; ++n) c += (nb[n] > jb);
    cnt[jb] = c;
  }
  __syncthreads();
  // start[jb] = sum of cnt[jb'] for jb' > jb: each thread owns a contiguous
  // run of jb taken from the top, then an exclusive scan over the threads.
  const int per = (J + kSchedThreads - 1) / kSchedThreads;
  const int r0 = tid * per;                 // run in "from the top" order: rank = J-1-jb
  int mysum = 0;
  for (int r = r0; r < min(r0 + per, J); ++r) mysum += cnt[J - 1 - r];
  part[tid] = mysum;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const int v = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - mysum;              // exclusive prefix
  for (int r = r0; r < min(r0 + per, J); ++r) {
    const int jb = J - 1 - r;
    const int c = cnt[jb];
    int idx = run;
    for (int n = 0; n < num_seqs; ++n) {
      if (nb[n] > jb) {
        if (idx < max_items) work[idx] = make_int2(n, jb);
        ++idx;
      }
    }
    run += c;
  }
  if (tid == kSchedThreads - 1) *work_count = min(part[kSchedThreads - 1], max_items);
}

template <bool ROTQ, bool ROTK, bool THD>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.q_blocks * (THD ? 1 : p.batch) * p.num_kv_heads;
  if (blocks == 0) return hipSuccess;
  // short work items (window layers): twice the waves per SIMD to hide their
  // load latency; windows whose items span at most kAllTiles key tiles
  // (window + BQ - 1 keys at most) stage all of them at once.
  if constexpr (!ROTK) {
    if (p.window > 0) {
      if (p.window + BQ - 1 <= kAllTiles * NK)
        hipLaunchKernelGGL((prefill_kernel<ROTQ, ROTK, THD, 2, true>), dim3((uint32_t)blocks),
                           dim3(Shape<2>::kThreads), 0, stream, p);
      else
        hipLaunchKernelGGL((prefill_kernel<ROTQ, ROTK, THD, 2, false>), dim3((uint32_t)blocks),
                           dim3(Shape<2>::kThreads), 0, stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_kernel<ROTQ, ROTK, THD, 4, false>), dim3((uint32_t)blocks), dim3(Shape<4>::kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_thd_schedule(const int32_t* cu_seqlens, int32_t num_seqs, int32_t bq, int32_t max_items,
                               int2* work, int32_t* work_count, hipStream_t stream) {
  hipLaunchKernelGGL(thd_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, cu_seqlens, num_seqs, bq,
                     max_items, work, work_count);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, bool thd, int krot, hipStream_t stream) {
  const bool rotq = p.table != nullptr;
  const bool rotk = rotq && krot == KROT_FUSED;
  if (thd) {
    if (!rotq) return launch_one<false, false, true>(p, stream);
    return rotk ? launch_one<true, true, true>(p, stream) : launch_one<true, false, true>(p, stream);
  }
  if (!rotq) return launch_one<false, false, false>(p, stream);
  return rotk ? launch_one<true, true, false>(p, stream) : launch_one<true, false, false>(p, stream);
}

}  // namespace gptoss
