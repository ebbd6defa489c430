// Backward pass of the GPT-OSS prefill attention on gfx950: gradients of the
// sink + GQA + causal / sliding-window attention (page
// "nemo_automodel.components.models.gpt_oss.layers", GptOssAttention;
// Transformers v4.55.0 release notes, "Architecture") with respect to q, k, v
// and the per-head sinks. The pages print no backward; these are the
// derivatives of the forward written out. With tau = softmax_scale, natural-log
// lse per row (from the forward), p = exp(s - lse):
//   D_i = <dO_i, o_i>,  dP_ij = <dO_i, v_j>,  dS_ij = p_ij (dP_ij - D_i)
//   dq~_i = tau sum_j dS_ij k~_j,  dk~_j = tau sum_i dS_ij q~_i,  dv_j = sum_i p_ij dO_i
//   dsigma_h = - sum_i exp(sigma_h - lse_i) D_i
// and the rotation is undone with its transpose (the bf16 cast of the rotated
// q and k passes the gradient through): dq = R^T dq~, dk = R^T dk~.
//
// Kernels, in launch order (the caller's q and k are rotated into the
// workspace first by the standalone rotation kernel):
//   bwd_pre_kernel     D for every (token, query head): 8 lanes per row.
//   bwd_sink_kernel    dsigma per head: one work group per head sums its rows
//                      in a fixed order (no atomics, reproducible).
//   bwd_dq_kernel      work item (sequence, KV head, 32 query positions): like
//                      the forward, every K/V tile is staged in LDS once for
//                      the 8 query heads; per tile a wave runs S^T = K Q^T and
//                      dP^T = V dO^T (16 + 16 MFMAs), forms dS^T in registers and
//                      accumulates dQ^T += K^T dS^T (16 MFMAs, K^T read from
//                      the row-major K tile with ds_read_b64_tr_b16).
//   bwd_dkdv_kernel    work item (sequence, KV head, 64 keys): K and V of the
//                      tile stay in registers as MFMA fragments; each of 4 waves
//                      takes 2 of the 8 query heads and walks every 32-query
//                      block that can see the tile: S = Q K^T and dP = dO V^T
//                      (16 + 16 MFMAs), then dV^T += dO^T P and dK^T += Q^T dS
//                      (16 + 16 MFMAs; dO^T and Q^T through a per-wave LDS
//                      tile and transpose reads). The 4 waves' partial dK, dV
//                      are summed through LDS at the end.
// dq, dk, dv are written once each (no atomics), rounded to bf16 from fp32.
#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

constexpr int BQ = kPrefillBQ;   // query positions per block
constexpr int NK = kBackwardNK;  // keys per tile
constexpr int KSB = 80;          // LDS row stride of the K tile (dq kernel): conflict-free transpose reads
constexpr int VSB = 72;          // LDS row stride of the V tile (dq kernel): conflict-free 16 B row reads
constexpr int QS = 80;           // LDS row stride of a wave's q / dO tile (dk/dv kernel)

__device__ __forceinline__ uint2 ldg8(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }

// ---------------------------------------------------------------------------
// D = <dO, o> per (token, query head), and lse in log2 units, both written
// head-major [Hq, tokens] so the kernels below read a head's consecutive rows
// contiguously. Work group: 32 tokens of one head, 8 lanes per row.
// ---------------------------------------------------------------------------
template <bool THD>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BackwardParams p) {
  const int Hq = p.num_kv_heads * kGroup;
  const int h = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int c = threadIdx.x & 7;
  if (t >= p.tokens) return;   // whole 8-lane groups leave together
  bool valid = true;
  int64_t oo, od;
  if (THD) {
    valid = t < __ldg(p.cu_seqlens + p.batch);   // tokens after the last sequence belong to none
    oo = t * p.o_st + h * p.o_sh;
    od = t * p.do_st + h * p.do_sh;
  } else {
    const int64_t b = t / p.seqlen, s = t - b * p.seqlen;
    oo = b * p.o_sb + s * p.o_st + h * p.o_sh;
    od = b * p.do_sb + s * p.do_st + h * p.do_sh;
  }
  float acc = 0.0f;
  if (valid) {
    const uint4 a = ldg16(p.o + oo + 8 * c), d = ldg16(p.dout + od + 8 * c);
    const uint32_t* pa = reinterpret_cast<const uint32_t*>(&a);
    const uint32_t* pd = reinterpret_cast<const uint32_t*>(&d);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16_lo(pa[i]) * bf16_lo(pd[i]) + bf16_hi(pa[i]) * bf16_hi(pd[i]);
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (c == 0) {
    const float l = valid ? p.lse[t * Hq + h] : -INFINITY;
    p.dd[(int64_t)h * p.tokens + t] = acc;
    // a row without any term (lse = -inf) gets +inf: its probabilities exp2(x - lse2) are 0
    p.lse2[(int64_t)h * p.tokens + t] = (l > -INFINITY) ? l * kLog2e : INFINITY;
  }
}

// dsigma_h = - sum over the head's rows of exp(sigma_h - lse) * D, one work
// group per head, each thread summing a fixed stride of rows, then a tree.
__global__ __launch_bounds__(256) void bwd_sink_kernel(BackwardParams p) {
  __shared__ float part[256];
  const int h = blockIdx.x;
  const float sig2 = p.sinks[h] * kLog2e;
  const float* l2 = p.lse2 + (int64_t)h * p.tokens;
  const float* dd = p.dd + (int64_t)h * p.tokens;
  float acc = 0.0f;
  if (sig2 > -INFINITY) {
    for (int64_t t = threadIdx.x; t < p.tokens; t += 256) acc -= __builtin_amdgcn_exp2f(sig2 - l2[t]) * dd[t];
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.dsinks[h] = part[0];
}

// Rotate back a gradient pair held by one lane: y1 = dims i (< 32), y2 = dims
// i + 32 of the rotated-space gradient; dx1 = y1 C + y2 S, dx2 = y2 C - y1 S.
// c4 / s4: the table's bf16 cos / sin for the lane's four consecutive i.
__device__ __forceinline__ void rotate_back4(f32x4_t& y1, f32x4_t& y2, uint2 c4, uint2 s4) {
  const float c[4] = {bf16_lo(c4.x), bf16_hi(c4.x), bf16_lo(c4.y), bf16_hi(c4.y)};
  const float s[4] = {bf16_lo(s4.x), bf16_hi(s4.x), bf16_lo(s4.y), bf16_hi(s4.y)};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float a = y1[r], b = y2[r];
    y1[r] = a * c[r] + b * s[r];
    y2[r] = b * c[r] - a * s[r];
  }
}

__device__ __forceinline__ uint2 pack4(const f32x4_t& v) {
  return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// ---------------------------------------------------------------------------
// dq: one work group of 8 waves per (sequence, KV head g, 32 query positions);
// wave w owns query head 8 g + w (two 16-column blocks cb of positions).
// ---------------------------------------------------------------------------
template <bool THD, bool ROT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(BackwardParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t lds_k[2 * NK * KSB];
  __shared__ __attribute__((aligned(16))) bf16_t lds_v[2 * NK * VSB];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int Hkv = p.num_kv_heads, Hq = Hkv * kGroup;
  const int item = blockIdx.x / Hkv;
  const int g = blockIdx.x - item * Hkv;
  int j, L, ts;
  int64_t row0, bq_, bk_, bv_, bd_;
  if (THD) {
    if (item >= __ldg(p.count_q)) return;
    const int2 w = p.work_q[item];
    j = w.y;
    const int n = min(max(w.x, 0), p.batch - 1);
    ts = min(max(__ldg(p.cu_seqlens + n), 0), p.seqlen);
    L = min(max(__ldg(p.cu_seqlens + n + 1), ts), p.seqlen) - ts;
    row0 = 0; bq_ = bk_ = bv_ = bd_ = 0;
  } else {
    const int r = item / p.batch, b = item - r * p.batch;
    j = p.q_blocks - 1 - r;   // most keys first
    ts = 0;
    L = p.seqlen;
    row0 = (int64_t)b * p.seqlen;
    bq_ = b * p.q_sb; bk_ = b * p.k_sb; bv_ = b * p.v_sb; bd_ = b * p.do_sb;
  }
  const int q0 = j * BQ;
  if (j < 0 || q0 >= L) return;
  const int qlast = min(q0 + BQ, L) - 1;
  const int W = p.window;
  const uint32_t weff = (W > 0) ? (uint32_t)W : 0x7FFFFFFFu;
  const int kv_lo = (W > 0) ? max(0, q0 - W + 1) : 0;
  const int kv_hi = qlast + 1;
  const int ntiles = (kv_hi - kv_lo + NK - 1) / NK;
  const float sl = p.scale_log2;
  const int head = g * kGroup + wave;

  // staging: thread -> (row tid / 8, 16-byte chunk tid % 8) of the K and V tiles
  const int srow = tid >> 3, scc = tid & 7;
  const int32_t krow_b = (int32_t)p.k_st * 2, vrow_b = (int32_t)p.v_st * 2;
  const char* k_tile0 = reinterpret_cast<const char*>(p.k + bk_ + (int64_t)(ts + kv_lo) * p.k_st + (int64_t)g * p.k_sh);
  const char* v_tile0 = reinterpret_cast<const char*>(p.v + bv_ + (int64_t)(ts + kv_lo) * p.v_st + (int64_t)g * p.v_sh);
  const uint32_t koff = (uint32_t)(srow * krow_b + 16 * scc);
  const uint32_t voff = (uint32_t)(srow * vrow_b + 16 * scc);
  uint4 sk, sv;
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    const int rows = kv_hi - (kv_lo + t * NK);
    sk = ldb16(make_rsrc(k_tile0 + (int64_t)t * NK * krow_b, (rows - 1) * krow_b + 2 * kHeadDim), koff);
    sv = ldb16(make_rsrc(v_tile0 + (int64_t)t * NK * vrow_b, (rows - 1) * vrow_b + 2 * kHeadDim), voff);
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    *reinterpret_cast<uint4*>(lds_k + buf * NK * KSB + srow * KSB + 8 * scc) = sk;
    *reinterpret_cast<uint4*>(lds_v + buf * NK * VSB + srow * VSB + 8 * scc) = sv;
  };

  if (ntiles > 0) load_tile(0);
  // q~ and dO of the wave's 32 rows as B-operand fragments (lane = query column,
  // 8 consecutive dims), and each column's lse (log2 units) and D.
  int qpos[2];
  bf16x8_t qf[2][2], df[2][2];
  float lse2[2], dd[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    qpos[cb] = q0 + 16 * cb + col;
    const int pos = min(qpos[cb], qlast);
    const bf16_t* qp = p.q + bq_ + (int64_t)(ts + pos) * p.q_st + (int64_t)head * p.q_sh + 8 * grp;
    const bf16_t* dp = p.dout + bd_ + (int64_t)(ts + pos) * p.do_st + (int64_t)head * p.do_sh + 8 * grp;
    qf[cb][0] = as_bf16x8(ldg16(qp));
    qf[cb][1] = as_bf16x8(ldg16(qp + 32));
    df[cb][0] = as_bf16x8(ldg16(dp));
    df[cb][1] = as_bf16x8(ldg16(dp + 32));
    const int64_t rr = (int64_t)head * p.tokens + row0 + ts + pos;
    lse2[cb] = p.lse2[rr];
    dd[cb] = p.dd[rr];
  }

  f32x4_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const bf16_t* kt = lds_k + buf * NK * KSB;
    const bf16_t* vt = lds_v + buf * NK * VSB;
    const int tile0 = kv_lo + t * NK;

    // S^T = K Q^T and dP^T = V dO^T: [kb][cb] element r = key kb*16 + 4*grp + r, query col
    f32x4_t s[4][2], dpt[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16_t* kr = kt + (kb * 16 + col) * KSB + 8 * grp;
      const bf16_t* vr = vt + (kb * 16 + col) * VSB + 8 * grp;
      const bf16x8_t a0 = as_bf16x8(*reinterpret_cast<const uint4*>(kr));
      const bf16x8_t a1 = as_bf16x8(*reinterpret_cast<const uint4*>(kr + 32));
      const bf16x8_t c0 = as_bf16x8(*reinterpret_cast<const uint4*>(vr));
      const bf16x8_t c1 = as_bf16x8(*reinterpret_cast<const uint4*>(vr + 32));
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        s[kb][cb] = mfma16(a1, qf[cb][1], mfma16(a0, qf[cb][0], z));
        dpt[kb][cb] = mfma16(c1, df[cb][1], mfma16(c0, df[cb][0], z));
      }
    }
    const bool full = (tile0 + NK - 1 <= q0) && (W == 0 || qlast - tile0 < W);
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kpos = tile0 + kb * 16 + 4 * grp + r;
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            s[kb][cb][r] = ((uint32_t)(qpos[cb] - kpos) < weff) ? s[kb][cb][r] : -INFINITY;
        }
    }
    // dS^T = P^T (dP^T - D), packed bf16 as the B operand of dQ^T = K^T dS^T
    // (keys of slice ks: e < 4 -> 4*grp + e of key block 2ks, e >= 4 -> of block 2ks+1)
    bf16x8_t dsf[2][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      uint32_t w[8];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][cb][r], sl, -lse2[cb]));
          x[r] = pr * (dpt[kb][cb][r] - dd[cb]);
        }
        w[2 * kb] = pack_bf16x2(x[0], x[1]);
        w[2 * kb + 1] = pack_bf16x2(x[2], x[3]);
      }
      dsf[cb][0] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      dsf[cb][1] = __builtin_bit_cast(bf16x8_t, make_uint4(w[4], w[5], w[6], w[7]));
    }
    // dQ^T += K^T dS^T (K^T read transposed from the row-major K tile)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16_t* kb_ = kt + (32 * ks + 4 * grp + (col >> 2)) * KSB + 16 * db + 4 * (col & 3);
        const uint2 lo = lds_read_tr16(kb_);
        const uint2 hi = lds_read_tr16(kb_ + 16 * KSB);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[db][cb] = mfma16(a, dsf[cb][ks], acc[db][cb]);
      }
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: dq~ = tau acc; dq = R^T dq~ at the query's position; lane holds d = 16*db + 4*grp + r
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int pos = qpos[cb];
    if (pos > qlast) continue;
    f32x4_t y[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) y[db] = acc[db][cb] * p.scale;
    if (ROT) {
      const bf16_t* tp = p.table + (int64_t)min(pos, p.table_rows - 1) * kHeadDim + 4 * grp;
#pragma unroll
      for (int dh = 0; dh < 2; ++dh) rotate_back4(y[dh], y[dh + 2], ldg8(tp + 16 * dh), ldg8(tp + 32 + 16 * dh));
    }
    bf16_t* op = p.dq + ((row0 + ts + pos) * Hq + head) * kHeadDim + 4 * grp;
#pragma unroll
    for (int db = 0; db < 4; ++db) *reinterpret_cast<uint2*>(op + 16 * db) = pack4(y[db]);
  }
}

// ---------------------------------------------------------------------------
// dv (PART 0) or dk (PART 1): one work group of 4 waves per (sequence, KV head
// g, 64 keys); wave w owns query heads 8 g + 2 w and 8 g + 2 w + 1. The two
// gradients are separate launches so each wave holds one 64-key x 64-dim fp32
// accumulator (64 VGPRs) and two waves fit on a SIMD; S = Q K^T is formed in
// both (its 16 MFMAs per step are the price).
// ---------------------------------------------------------------------------
constexpr int kKvLds = 4 * 16 * 64 * 16;   // cross-wave sum: 4 waves x 16 fragments x 64 lanes x 16 B
static_assert(4 * BQ * QS * 2 <= kKvLds, "per-wave transpose tiles fit in the reduction space");

template <bool THD, bool ROT, int PART>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kv_kernel(BackwardParams p) {
  __shared__ __attribute__((aligned(16))) char lds_raw[kKvLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int Hkv = p.num_kv_heads;
  const int item = blockIdx.x / Hkv;
  const int g = blockIdx.x - item * Hkv;
  int jt, L, ts;
  int64_t row0, bq_, bk_, bv_, bd_;
  if (THD) {
    if (item >= __ldg(p.count_k)) return;
    const int2 w = p.work_k[item];
    const int n = min(max(w.x, 0), p.batch - 1);
    ts = min(max(__ldg(p.cu_seqlens + n), 0), p.seqlen);
    L = min(max(__ldg(p.cu_seqlens + n + 1), ts), p.seqlen) - ts;
    jt = (L + NK - 1) / NK - 1 - w.y;   // the list counts tiles from the end: most queries first
    row0 = 0; bq_ = bk_ = bv_ = bd_ = 0;
  } else {
    const int r = item / p.batch, b = item - r * p.batch;
    jt = r;                   // tile 0 is seen by every query: most work first
    ts = 0;
    L = p.seqlen;
    row0 = (int64_t)b * p.seqlen;
    bq_ = b * p.q_sb; bk_ = b * p.k_sb; bv_ = b * p.v_sb; bd_ = b * p.do_sb;
  }
  const int t0 = jt * NK;
  if (jt < 0 || t0 >= L) return;
  const int tlast = min(t0 + NK, L) - 1;
  const int W = p.window;
  const uint32_t weff = (W > 0) ? (uint32_t)W : 0x7FFFFFFFu;
  const int qhi = (W > 0) ? min(L - 1, tlast + W - 1) : L - 1;   // last query that sees a key of the tile
  const float sl = p.scale_log2;

  // K (and, for dk, V) of the tile as B-operand fragments: lane = key column, 8 consecutive dims
  bf16x8_t kf[4][2], vf[4][2];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int key = min(t0 + kb * 16 + col, tlast);
    const bf16_t* kp = p.k + bk_ + (int64_t)(ts + key) * p.k_st + (int64_t)g * p.k_sh + 8 * grp;
    kf[kb][0] = as_bf16x8(ldg16(kp));
    kf[kb][1] = as_bf16x8(ldg16(kp + 32));
    if (PART == 1) {
      const bf16_t* vp = p.v + bv_ + (int64_t)(ts + key) * p.v_st + (int64_t)g * p.v_sh + 8 * grp;
      vf[kb][0] = as_bf16x8(ldg16(vp));
      vf[kb][1] = as_bf16x8(ldg16(vp + 32));
    }
  }
  f32x4_t acc[4][4];   // [d block][key block]: element r = dim 16*db + 4*grp + r, key col (dV^T or dK^T)
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // this wave's tile [32 queries][QS] for the transpose reads: dO (dv) or q (dk)
  bf16_t* lt = reinterpret_cast<bf16_t*>(lds_raw) + wave * (BQ * QS);

  // Steps: every block of 32 queries that can see the tile, once per head of the
  // wave (head 8 g + 2 wave + hh). In dv the global loads of the next step are in
  // flight while a step computes.
  const int qb_lo = t0 / BQ;
  // Rows are read through buffer ranges that end with the sequence: rows past it
  // read as zeros (their dO is 0, so they add nothing to dV or dK) and need no
  // clamps; one 32-bit offset per load. The ranges of the wave's two heads are
  // wave-uniform.
  const int32_t qrow_b = (int32_t)p.q_st * 2, drow_b = (int32_t)p.do_st * 2;   // < 2^31 / (L + 32): host check
  __amdgpu_buffer_rsrc_t rq[2], rd[2], rl[2], rdd[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int head = g * kGroup + 2 * wave + hh;
    rq[hh] = make_rsrc(p.q + bq_ + (int64_t)ts * p.q_st + (int64_t)head * p.q_sh, (L - 1) * qrow_b + 2 * kHeadDim);
    rd[hh] = make_rsrc(p.dout + bd_ + (int64_t)ts * p.do_st + (int64_t)head * p.do_sh, (L - 1) * drow_b + 2 * kHeadDim);
    rl[hh] = make_rsrc(p.lse2 + (int64_t)head * p.tokens + row0 + ts, L * 4);
    rdd[hh] = make_rsrc(p.dd + (int64_t)head * p.tokens + row0 + ts, L * 4);
  }
  struct Fetch { uint4 qa[2][2], da[2][2]; float l2[2][4], dd[2][4]; };
  // hh is a constant at every call (the calls are unrolled), so the ranges stay scalar
  auto fetch = [&](int qb, int hh, Fetch& f) __attribute__((always_inline)) {
    const int q0 = qb * BQ;
    const __amdgpu_buffer_rsrc_t bq = rq[hh], bd = rd[hh], bl = rl[hh], bdd = rdd[hh];
#pragma unroll
    for (int qm = 0; qm < 2; ++qm) {
      // q~ and dO rows as A-operand fragments (lane = query row, 8 consecutive dims)
      const uint32_t qo = (uint32_t)((q0 + qm * 16 + col) * qrow_b + 16 * grp);
      const uint32_t dof = (uint32_t)((q0 + qm * 16 + col) * drow_b + 16 * grp);
      f.qa[qm][0] = ldb16(bq, qo); f.qa[qm][1] = ldb16(bq, qo + 64);
      f.da[qm][0] = ldb16(bd, dof); f.da[qm][1] = ldb16(bd, dof + 64);
      // lse (log2 units) and D of the lane's queries q0 + 16 qm + 4 grp + e
      const uint32_t lo = (uint32_t)((q0 + qm * 16 + 4 * grp) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f.l2[qm][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bl, lo + 4 * e, 0, 0));
        if (PART == 1) f.dd[qm][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bdd, lo + 4 * e, 0, 0));
      }
    }
  };
  auto step = [&](int qb, const Fetch& f) __attribute__((always_inline)) {
    const int q0 = qb * BQ;
    const bool full = (q0 >= t0 + NK - 1) && (W == 0 || q0 + BQ - 1 - t0 < W);
    {
      const uint4 (&qa)[2][2] = f.qa;
      const uint4 (&da)[2][2] = f.da;
      const float (&lse2)[2][4] = f.l2;
      const float (&dd)[2][4] = f.dd;
      // the previous step's transpose reads are complete before the tile is rewritten
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int qm = 0; qm < 2; ++qm)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          *reinterpret_cast<uint4*>(lt + (qm * 16 + col) * QS + 32 * ks + 8 * grp) = PART ? qa[qm][ks] : da[qm][ks];

      // Per 16-query half qm: S = Q K^T (and dP = dO V^T) with [kb] element e = query
      // q0 + 16 qm + 4 grp + e, key t0 + 16 kb + col; then P (dv) or dS = P (dP - D) (dk),
      // packed as the B operand over the 32 queries (elements 4 qm .. 4 qm + 3)
      uint32_t bw[4][4];   // [kb][word]
#pragma unroll
      for (int qm = 0; qm < 2; ++qm) {
        f32x4_t s_[4], dp_[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          s_[kb] = mfma16(as_bf16x8(qa[qm][1]), kf[kb][1], mfma16(as_bf16x8(qa[qm][0]), kf[kb][0], z));
          if (PART == 1)
            dp_[kb] = mfma16(as_bf16x8(da[qm][1]), vf[kb][1], mfma16(as_bf16x8(da[qm][0]), vf[kb][0], z));
        }
        if (!full) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int qq = q0 + qm * 16 + 4 * grp + e, key = t0 + kb * 16 + col;
              s_[kb][e] = ((uint32_t)(qq - key) < weff) ? s_[kb][e] : -INFINITY;
            }
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s_[kb][e], sl, -lse2[qm][e]));
            x[e] = (PART == 1) ? pr * (dp_[kb][e] - dd[qm][e]) : pr;
          }
          bw[kb][2 * qm] = pack_bf16x2(x[0], x[1]);
          bw[kb][2 * qm + 1] = pack_bf16x2(x[2], x[3]);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      // dV^T += dO^T P (dv) or dK^T += Q^T dS (dk), the first operand read transposed from the tile
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int off = (4 * grp + (col >> 2)) * QS + 16 * db + 4 * (col & 3);
        const uint2 lo = lds_read_tr16(lt + off), hi = lds_read_tr16(lt + off + 16 * QS);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc[db][kb] = mfma16(a, __builtin_bit_cast(bf16x8_t, make_uint4(bw[kb][0], bw[kb][1], bw[kb][2], bw[kb][3])),
                               acc[db][kb]);
      }
    }
  };
  // Query blocks are walked from the last one down: the work groups of one
  // (sequence, KV head) run together on one XCD (consecutive work groups take
  // consecutive KV heads, dealt round-robin over the 8 XCDs) and then read the
  // same q / dO block at about the same time, so L2 serves the repeats.
  const int qb_hi = qhi / BQ;
  if (PART == 0) {
    // dv holds two fetch buffers in turn: each step computes from one while the
    // other receives the next step's rows, with no register copies between steps
    Fetch fa, fb;
    fetch(qb_hi, 0, fa);
    for (int qb = qb_hi; qb >= qb_lo; --qb) {
      fetch(qb, 1, fb);
      step(qb, fa);
      fetch(max(qb - 1, qb_lo), 0, fa);   // the last block fetches itself again: no branch
      step(qb, fb);
    }
  } else {
    // dk has no registers to spare for a second buffer: each step loads its own rows
    for (int qb = qb_hi; qb >= qb_lo; --qb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        Fetch f;
        fetch(qb, hh, f);
        step(qb, f);
      }
    }
  }

  // sum the 4 waves' partials through LDS; wave w finishes d blocks (w & 1, (w & 1) + 2)
  // -- the rotation pairs dims i and i + 32 -- of key blocks 2 (w >> 1) and 2 (w >> 1) + 1
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds_raw);
  const int pr = wave & 1, kh = wave >> 1;
  __syncthreads();
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) red[(wave * 16 + db * 4 + kb) * 64 + lane] = acc[db][kb];
  __syncthreads();
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int kb = 2 * kh + kk;
    const int key = t0 + kb * 16 + col;
    f32x4_t y1 = {0.f, 0.f, 0.f, 0.f}, y2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      y1 += red[(w * 16 + pr * 4 + kb) * 64 + lane];
      y2 += red[(w * 16 + (pr + 2) * 4 + kb) * 64 + lane];
    }
    if (key > tlast) continue;
    if (PART == 1) {
      y1 *= p.scale;
      y2 *= p.scale;
      if (ROT) {
        const bf16_t* tp = p.table + (int64_t)min(key, p.table_rows - 1) * kHeadDim + 16 * pr + 4 * grp;
        rotate_back4(y1, y2, ldg8(tp), ldg8(tp + 32));
      }
    }
    bf16_t* op = (PART == 1 ? p.dk : p.dv) + ((row0 + ts + key) * Hkv + g) * kHeadDim + 16 * pr + 4 * grp;
    *reinterpret_cast<uint2*>(op) = pack4(y1);
    *reinterpret_cast<uint2*>(op + 32) = pack4(y2);
  }
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* x, int32_t n, float value) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = value;
}

template <bool THD, bool ROT>
hipError_t launch_all(const BackwardParams& p, hipStream_t stream) {
  const int Hq = p.num_kv_heads * kGroup;
  const int64_t tokens = THD ? (int64_t)p.seqlen : (int64_t)p.batch * p.seqlen;
  hipLaunchKernelGGL(bwd_pre_kernel<THD>, dim3((uint32_t)((tokens + 31) / 32), Hq), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(bwd_sink_kernel, dim3(Hq), dim3(256), 0, stream, p);
  const int64_t rep = THD ? 1 : p.batch;
  hipLaunchKernelGGL((bwd_dq_kernel<THD, ROT>), dim3((uint32_t)(p.q_blocks * rep * p.num_kv_heads)), dim3(512), 0,
                     stream, p);
  const dim3 kv_grid((uint32_t)(p.k_tiles * rep * p.num_kv_heads));
  hipLaunchKernelGGL((bwd_kv_kernel<THD, ROT, 0>), kv_grid, dim3(256), 0, stream, p);
  hipLaunchKernelGGL((bwd_kv_kernel<THD, ROT, 1>), kv_grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_f32(float* x, int32_t n, float value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream, x, n, value);
  return hipGetLastError();
}

hipError_t launch_backward(const BackwardParams& p, bool thd, hipStream_t stream) {
  const bool rot = p.table != nullptr;
  if (thd) return rot ? launch_all<true, true>(p, stream) : launch_all<true, false>(p, stream);
  return rot ? launch_all<false, true>(p, stream) : launch_all<false, false>(p, stream);
}

}  // namespace gptoss
