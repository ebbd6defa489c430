// Sliding-window prefill as runs of consecutive query blocks (BSHD or packed
// THD; window a multiple of 32, at most 128: GPT-OSS's 128-token layers).
//
// What is computed is the prefill attention of prefill.hip (page
// "nemo_automodel.components.models.gpt_oss.layers", GptOssAttention: sinks,
// sliding_window, softmax_scale; Transformers v4.55.0 release notes,
// "Architecture": sliding 128-token-window layers, a per-head sink in the
// softmax denominator; key j visible to query i iff 0 <= i - j < W). Only the
// order of the work differs.
//
// A work group of 8 waves (wave w = query head 8 g + w, 32 positions) walks a
// run of consecutive 32-position query blocks of one (sequence b, KV head g).
// The keys of block j are the key blocks j - W/32 .. j (32 keys each); they sit
// in a ring of 6 LDS slots, slot = key block mod 6. While block j is computed,
// the work group fetches the next block's new key block into registers, and
// each wave the next block's q rows; at the end of block j the new key block is
// stored into the slot block j no longer reads (K rotated exactly as
// gptoss_rope_qk rotates it, so every key is rotated once per run and no
// separate K pass is needed) and the next q rows are rotated with table rows
// staged in LDS. One barrier per block. Each block computes W/32 + 1 steps of 32
// keys: the first with key k of the step visible to query row i iff k > i, the
// last (the diagonal block) iff k <= i, the ones between fully visible.
//
// Runs: BSHD sequences are cut into runs of run_len blocks, all resident at
// once (two work groups per CU), two neighbouring runs split unevenly (see the
// work-item mapping) so that the two work groups of a CU end together; THD runs
// come from a device-built list, longest first, in about two rounds.
#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

constexpr int SR = 32;            // key rows per ring slot = query positions per block
constexpr int SLOTS = 6;          // the W/32 + 1 <= 5 key blocks of a block and the next block's
constexpr int RS = 80;            // LDS row stride of the ring (160 B): conflict-free K and transposed V reads
constexpr int TS = 72;            // LDS row stride of the staged table rows
constexpr int NWV = 8;            // waves: one query head each
constexpr float kSumLimitW = 0x1p100f;   // a step's partial row sum beyond this moves the reference
constexpr float kRaiseGapW = 8.0f;

__device__ __forceinline__ float col_xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float col_xor_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ uint4 lds16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void stb16(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4& v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, off, 0, 0);
}
__device__ __forceinline__ void stb8(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint2& v) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, off, 0, 0);
}
__device__ __forceinline__ void stb4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
__device__ __forceinline__ uint2 ldg8(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint2 ldb8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}

// ROTM: 0 q and k given rotated, 1 all 64 dims rotated, 2 partial rotary (rotary_dim 16, 32 or 48).
// THD: packed sequences (runs from the device-built work list) instead of BSHD batches.
// Two work groups per CU (128 registers a lane, 69 KB of LDS each).
template <int ROTM, bool THD>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(4)))
void window_run_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t ring_k[SLOTS * SR * RS];
  __shared__ __attribute__((aligned(16))) bf16_t ring_v[SLOTS * SR * RS];
  __shared__ __attribute__((aligned(16))) bf16_t tab_s[2][SR * TS];   // table rows of a block's positions

  const int tid = threadIdx.x, lane = tid & 63;
  // the thread index as a value the compiler cannot move across a call site: load
  // and store offsets derived from it are recomputed where used (a few integer ops)
  // instead of being held, or spilled, across the block loop
  auto fresh_tid = [&]() __attribute__((always_inline)) {
    int t = tid;
    asm volatile("" : "+v"(t));
    return t;
  };
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int Hkv = p.num_kv_heads;
  // the KV heads of one run on one XCD (work group i runs on XCD i mod 8), one after another
  int g, r;
  const int nwg = gridDim.x;
  if (nwg % (8 * Hkv) == 0) {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    g = k % Hkv;
    r = (k / Hkv) * 8 + x;
  } else {
    g = blockIdx.x % Hkv;
    r = blockIdx.x / Hkv;
  }
  // the run: a sequence, its first query block j0 and the block after its last, j1;
  // tensor offsets of the sequence and the token-major row of its first position
  int L, j0, j1;
  int64_t off_q, off_k, off_v, off_o, row0;
  if (THD) {   // packed sequences: item r of the device-built run list (longest first)
    if (r >= __ldg(p.work_count)) return;
    const int2 w = p.work[r];
    const int n = min(max(w.x, 0), p.batch - 1);
    const int ts = min(max(__ldg(p.cu_seqlens + n), 0), p.seqlen);
    const int te = min(max(__ldg(p.cu_seqlens + n + 1), ts), p.seqlen);
    L = te - ts;
    j0 = w.y * p.run_len;
    off_q = (int64_t)ts * p.q_st; off_k = (int64_t)ts * p.k_st; off_v = (int64_t)ts * p.v_st;
    off_o = (int64_t)ts * p.o_st;
    row0 = ts;
  }
  int jend;
  if (THD) {
    jend = j0 + p.run_len;
  } else if (p.pair_first > 0) {
    // Uneven pairs: when every run is resident at once, the first half of the work
    // groups is dispatched one per CU and the second half fills the other slot; the
    // older waves win the issue arbitration, so a second-half run advances at about
    // half the speed of its neighbour until that one ends. Each two neighbouring
    // runs of a sequence therefore cover 2 run_len blocks as pair_first blocks for
    // the first-half run and the rest for the second-half run, so both end at about
    // the same time.
    const int half = p.batch * p.runs_per_seq / 2;
    const bool second = r >= half;
    const int pr = second ? r - half : r;
    const int pps = p.runs_per_seq / 2;   // pairs per sequence
    const int b = pr / pps;
    if (b >= p.batch) return;
    L = p.seqlen;
    const int base = (pr - b * pps) * 2 * p.run_len;
    j0 = second ? base + p.pair_first : base;
    jend = second ? base + 2 * p.run_len : base + p.pair_first;
    off_q = b * p.q_sb; off_k = b * p.k_sb; off_v = b * p.v_sb; off_o = b * p.o_sb;
    row0 = (int64_t)b * L;
  } else {
    const int b = r / p.runs_per_seq;
    if (b >= p.batch) return;
    L = p.seqlen;
    j0 = (r - b * p.runs_per_seq) * p.run_len;
    jend = j0 + p.run_len;
    off_q = b * p.q_sb; off_k = b * p.k_sb; off_v = b * p.v_sb; off_o = b * p.o_sb;
    row0 = (int64_t)b * L;
  }
  j1 = min(jend, (L + SR - 1) / SR);
  if (j0 < 0 || j0 >= j1) return;
  const int WS = p.window / SR;              // key blocks before the diagonal one (1 .. 4)
  const int head = g * kGroup + wave;
  const float sl = p.scale_log2;
  const bf16_t* qbase = p.q + off_q + (int64_t)head * p.q_sh;
  const char* kbase = reinterpret_cast<const char*>(p.k + off_k + (int64_t)g * p.k_sh);
  const char* vbase = reinterpret_cast<const char*>(p.v + off_v + (int64_t)g * p.v_sh);
  bf16_t* obase = p.o + off_o + (int64_t)head * p.o_sh;
  const int32_t krow_b = (int32_t)p.k_st * 2, vrow_b = (int32_t)p.v_st * 2;   // < 2^31 / 64 (host check)
  const int32_t orow_b = (int32_t)p.o_st * 2;                                 // < 2^31 / 32 (host check)
  const int Hq = Hkv * kGroup;

  // rotated 8-dim chunks in each half of the rotary part (4: all 64 dims). A K
  // thread's two 4-dim pieces start at dims kd1 and kd2: a rotation pair (i, i +
  // rotary_dim / 2) when 4 q4 < rotary_dim / 2, else two pieces of the part that
  // passes through unrotated
  constexpr bool ROT = ROTM != 0;
  const int rc = ROTM == 2 ? p.rot_chunks : 4;
  auto kd1 = [&](int q4) __attribute__((always_inline)) { return q4 < 2 * rc ? 4 * q4 : 16 * rc + 8 * (q4 - 2 * rc); };
  auto kd2 = [&](int q4) __attribute__((always_inline)) { return q4 < 2 * rc ? 4 * q4 + 8 * rc : 16 * rc + 8 * (q4 - 2 * rc) + 4; };

  // ---- staging of one key block (32 rows) by wave roles. Waves 0-3 take the K
  // rows: a thread holds 4 dims of a row and their rotation partners 32 dims on,
  // with the 4 cos / sin (8-byte pieces). Waves 4-7 take the V rows (one 16-byte
  // chunk a thread) and, for a block whose queries come next, the table rows of
  // its positions (the q rotation's cos / sin). Every thread holds 8 registers. ----
  struct St { uint4 a, b; };
  auto load_block = [&](int kb, bool qtab, St& st) __attribute__((always_inline)) {
    const int rows = min(L - kb * SR, SR);   // rows past the sequence read as zeros (causally masked)
    const int tid = fresh_tid();
    if (wave < 4) {
      const int row = tid >> 3, q4 = tid & 7;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (int64_t)kb * SR * krow_b, (rows - 1) * krow_b + 2 * kHeadDim);
      const uint2 x1 = ldb8(rk, (uint32_t)(row * krow_b + 2 * kd1(q4)));
      const uint2 x2 = ldb8(rk, (uint32_t)(row * krow_b + 2 * kd2(q4)));
      st.a = make_uint4(x1.x, x1.y, x2.x, x2.y);
      if (ROT && q4 < 2 * rc) {
        const bf16_t* tp = p.table + (int64_t)min(kb * SR + row, p.table_rows - 1) * (16 * rc) + 4 * q4;
        const uint2 c = ldg8(tp), sn = ldg8(tp + 8 * rc);
        st.b = make_uint4(c.x, c.y, sn.x, sn.y);
      }
    } else {
      const int t = tid - 256, row = t >> 3, ch = t & 7;
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (int64_t)kb * SR * vrow_b, (rows - 1) * vrow_b + 2 * kHeadDim);
      st.a = ldb16(rv, (uint32_t)(row * vrow_b + 16 * ch));
      if (ROTM == 1 && qtab) st.b = ldg16(p.table + (int64_t)min(kb * SR + row, p.table_rows - 1) * kHeadDim + 8 * ch);
    }
  };
  auto store_block = [&](int kb, bool qtab, const St& st) __attribute__((always_inline)) {
    const int slot = kb % SLOTS;
    const int tid = fresh_tid();
    if (wave < 4) {
      const int row = tid >> 3, q4 = tid & 7;
      uint2 y1 = make_uint2(st.a.x, st.a.y), y2 = make_uint2(st.a.z, st.a.w);
      if (ROT && q4 < 2 * rc)
        rope4(make_uint2(st.a.x, st.a.y), make_uint2(st.a.z, st.a.w), make_uint2(st.b.x, st.b.y),
              make_uint2(st.b.z, st.b.w), y1, y2);
      bf16_t* d = ring_k + (slot * SR + row) * RS;
      *reinterpret_cast<uint2*>(d + kd1(q4)) = y1;
      *reinterpret_cast<uint2*>(d + kd2(q4)) = y2;
    } else {
      const int t = tid - 256, row = t >> 3, ch = t & 7;
      *reinterpret_cast<uint4*>(ring_v + (slot * SR + row) * RS + 8 * ch) = st.a;
      if (ROTM == 1 && qtab) *reinterpret_cast<uint4*>(tab_s[kb & 1] + row * TS + 8 * ch) = st.b;
    }
  };

  // ---- q of a block: the wave's 32 rows as two 16-column B operands ----
  struct Stage { St st; uint4 q[2][2]; };   // one block's loads in flight: its new key block and q rows
  bf16x8_t qf[2][2];
  auto load_q = [&](int jq, Stage& sg) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int pos = min(jq * SR + 16 * c + col, L - 1);   // rows past the end are never stored
      const bf16_t* qp = qbase + (int64_t)pos * p.q_st + 8 * grp;
      sg.q[c][0] = ldg16(qp);
      sg.q[c][1] = ldg16(qp + 32);
    }
  };
  auto rotate_q = [&](int jq, const Stage& sg) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint4 y1 = sg.q[c][0], y2 = sg.q[c][1];
      if (ROTM == 1) {
        const bf16_t* tp = tab_s[jq & 1] + (16 * c + col) * TS + 8 * grp;
        rope8(sg.q[c][0], sg.q[c][1], lds16(tp), lds16(tp + 32), y1, y2);
      } else if (ROTM == 2) {   // partial rotary: partners and table rows from global memory
        const int pos = min(jq * SR + 16 * c + col, L - 1);
        const bf16_t* qp = qbase + (int64_t)pos * p.q_st;
        const bf16_t* tp = p.table + (int64_t)min(pos, p.table_rows - 1) * (16 * rc);
        y1 = rope_chunk_partial(qp, tp, grp, rc, sg.q[c][0]);
        y2 = rope_chunk_partial(qp, tp, grp + 4, rc, sg.q[c][1]);
      }
      qf[c][0] = as_bf16x8(y1);
      qf[c][1] = as_bf16x8(y2);
    }
  };

  // key minus query within a step, less the constant parts: score element r of key
  // half kb2 and column block c is key kb2 * 16 + 4 grp + r against query col + 16 c
  const int kd = 4 * grp - col;

  const float sink = p.no_sink ? -INFINITY : __ldg(p.sinks + head) * kLog2e;
  const bool has_sink = sink > -INFINITY;

  // ---- prologue: the run's first block's key blocks, table rows and q ----
  Stage nx;
  {
    St st[5];
    const int kb0 = max(j0 - WS, 0);
#pragma unroll
    for (int u = 0; u < 5; ++u)
      if (kb0 + u <= j0) load_block(kb0 + u, kb0 + u == j0, st[u]);
    load_q(j0, nx);
#pragma unroll
    for (int u = 0; u < 5; ++u)
      if (kb0 + u <= j0) store_block(kb0 + u, kb0 + u == j0, st[u]);
  }
  __syncthreads();
  rotate_q(j0, nx);

  for (int j = j0; j < j1; ++j) {
    const bool more = j + 1 < j1;
    if (more) {   // the next block's new key block and q rows, in flight during this block
      load_block(j + 1, true, nx.st);
      load_q(j + 1, nx);
    }

    // ---- block j: softmax against a reference seeded with the sink logit (a row
    // without a sink takes the largest score of its first visible step), O^T in fp32 ----
    f32x4_t oacc[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int c = 0; c < 2; ++c) oacc[db][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float ref[2], lsum[2];
    bool unset[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      ref[c] = has_sink ? sink : 0.0f;
      lsum[c] = (grp == 0 && has_sink) ? 1.0f : 0.0f;
      unset[c] = !has_sink;
    }
    bool seeding = !has_sink;   // wave-uniform

    for (int kb = max(j - WS, 0); kb <= j; ++kb) {
      // the slot's offset as an opaque scalar: per-lane LDS addresses stay one base
      // plus immediate offsets instead of one induction register per read
      const int soff = __builtin_amdgcn_readfirstlane((kb % SLOTS) * SR * RS);
      const bf16_t* kt = ring_k + soff;
      const bf16_t* vt = ring_v + soff;
      const int pat = (kb == j) ? 2 : (kb == j - WS ? 1 : 0);   // diagonal / window edge / fully visible

      // S^T = K Q^T: sacc[kb2][c] element r = key kb2*16 + 4 grp + r, query col + 16 c
      f32x4_t sacc[2][2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16_t* krow = kt + (kb2 * 16 + col) * RS + 8 * grp;
        const bf16x8_t a0 = as_bf16x8(lds16(krow));
        const bf16x8_t a1 = as_bf16x8(lds16(krow + 32));
#pragma unroll
        for (int c = 0; c < 2; ++c) sacc[kb2][c] = mfma16(a0, qf[c][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int c = 0; c < 2; ++c) sacc[kb2][c] = mfma16(a1, qf[c][1], sacc[kb2][c]);
      }
      if (pat != 0) {
        const bool edge = pat == 1;   // edge step: key k visible to row i iff k > i; diagonal: iff k <= i
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int c = 0; c < 2; ++c)
              sacc[kb2][c][rr] = ((kd + 16 * kb2 + rr - 16 * c > 0) == edge) ? sacc[kb2][c][rr] : -INFINITY;
      }
      if (seeding) {
        bool left = false;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float v = -INFINITY;
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) v = __builtin_fmaxf(v, sacc[kb2][c][rr] * sl);
          const float mt = col_xor_max(v);
          if (unset[c] && mt > -INFINITY) {
            ref[c] = mt;
            unset[c] = false;
          }
          left |= unset[c];
        }
        seeding = __any(left);
      }
      // p = exp2(s tau log2(e) - ref) rounded to bf16, row sums of the rounded values
      bf16x8_t pf[2];
      float tsum[2];
      auto exp_col = [&](int c) __attribute__((always_inline)) {
        uint32_t w[4];
        const float nr = -ref[c];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          w[2 * kb2] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][c][0], sl, nr)),
                                   __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][c][1], sl, nr)));
          w[2 * kb2 + 1] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][c][2], sl, nr)),
                                       __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][c][3], sl, nr)));
        }
        float ts = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) ts = add_bf16x2(w[i], ts);
        tsum[c] = ts;
        pf[c] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      };
      bool bad = false;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        exp_col(c);
        bad |= !(tsum[c] <= kSumLimitW);
      }
      if (__any(bad)) {   // rare: a score far above the reference, the reference moves up
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float v = -INFINITY;
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) v = __builtin_fmaxf(v, sacc[kb2][c][rr]);
          const float mt = col_xor_max(v) * sl;
          if (mt > ref[c] + kRaiseGapW) {
            const float f = __builtin_amdgcn_exp2f(ref[c] - mt);
            lsum[c] *= f;
#pragma unroll
            for (int db = 0; db < 4; ++db) oacc[db][c] *= f;
            ref[c] = mt;
          }
          exp_col(c);
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) lsum[c] += tsum[c];
      // O^T += V^T P^T: V^T from the row-major V rows by transpose reads
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16_t* vb = vt + (4 * grp + (col >> 2)) * RS + 8 * (col & 3) + 4 * (db & 1) + 32 * (db >> 1);
        const uint2 lo = lds_read_tr16(vb);
        const uint2 hi = lds_read_tr16(vb + 16 * RS);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int c = 0; c < 2; ++c) oacc[db][c] = mfma16(a, pf[c], oacc[db][c]);
      }
    }

    // ---- epilogue of block j: o = acc / l (bf16), and the natural-log LSE if asked.
    // Stores go through buffer resources clipped to the block's rows inside the
    // sequence, so rows past its end are dropped by the range check instead of a
    // branch; with no branch the waits for the next block's loads need not cover
    // these stores. ----
    const int vrows = min(L - j * SR, SR);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(obase + (int64_t)j * SR * p.o_st, (vrows - 1) * orow_b + 2 * kHeadDim);
    const __amdgpu_buffer_rsrc_t rl =
        p.lse ? make_rsrc(p.lse + (row0 + j * SR) * Hq + head, ((vrows - 1) * Hq + 1) * 4)
              : make_rsrc(obase, 0);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float l = col_xor_sum(lsum[c]);
      const int r = 16 * c + col;
      const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
      const float lse = (l > 0.0f) ? (ref[c] + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
      stb4(rl, grp == 0 ? (uint32_t)(r * Hq * 4) : 0x7FFFFFF0u, __float_as_uint(lse));
#pragma unroll
      for (int h = 0; h < 2; ++h) {   // dims 32 h + 8 grp .. + 7: accumulators 2 h and 2 h + 1
        uint4 v;
        v.x = pack_bf16x2(oacc[2 * h][c][0] * inv, oacc[2 * h][c][1] * inv);
        v.y = pack_bf16x2(oacc[2 * h][c][2] * inv, oacc[2 * h][c][3] * inv);
        v.z = pack_bf16x2(oacc[2 * h + 1][c][0] * inv, oacc[2 * h + 1][c][1] * inv);
        v.w = pack_bf16x2(oacc[2 * h + 1][c][2] * inv, oacc[2 * h + 1][c][3] * inv);
        stb16(ro, (uint32_t)(r * orow_b + 2 * (32 * h + 8 * grp)), v);
      }
    }

    if (more) store_block(j + 1, true, nx.st);   // into slot (j + 1) mod 6, which block j does not read
    __syncthreads();
    if (more) rotate_q(j + 1, nx);
  }
}

template <bool THD>
void launch_runs(const PrefillParams& p, uint32_t blocks, hipStream_t stream) {
  const dim3 grid(blocks), block(NWV * 64);
  if (!p.table)
    hipLaunchKernelGGL((window_run_kernel<0, THD>), grid, block, 0, stream, p);
  else if (p.rot_chunks == kHeadDim / 16)
    hipLaunchKernelGGL((window_run_kernel<1, THD>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((window_run_kernel<2, THD>), grid, block, 0, stream, p);
}

}  // namespace

// BSHD: batch * runs_per_seq runs; THD: q_blocks = the run list's capacity (entries past
// *work_count exit at once)
hipError_t launch_window_runs(const PrefillParams& p, bool thd, hipStream_t stream) {
  const int64_t runs = thd ? (int64_t)p.q_blocks : (int64_t)p.batch * p.runs_per_seq;
  const int64_t blocks = runs * p.num_kv_heads;
  if (blocks == 0) return hipSuccess;
  if (thd)
    launch_runs<true>(p, (uint32_t)blocks, stream);
  else
    launch_runs<false>(p, (uint32_t)blocks, stream);
  return hipGetLastError();
}

}  // namespace gptoss
