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
// Kernels, in launch order (the caller's k, and with partial rotary also q,
// is rotated into the workspace first by the standalone rotation kernel):
//   bwd_dq_kernel      work item (sequence, KV head, 32 query positions): like
//                      the forward, it rotates its q rows on load (exactly, as
//                      the standalone rotation does) and also writes them, rotated,
//                      to the workspace for the dk / dv kernel; every K/V tile
//                      is staged in LDS once for the 8 query heads (full layers:
//                      one 8-wave work group; window layers: two 4-wave groups,
//                      4 heads each, two per CU); per tile a wave runs S^T = K Q^T and
//                      dP^T = V dO^T (16 + 16 MFMAs), forms dS^T in registers and
//                      accumulates dQ^T += K^T dS^T (16 MFMAs, K^T read from
//                      the row-major K tile with ds_read_b64_tr_b16). It also
//                      forms D = <dO, o> per row and writes (lse in log2
//                      units, -D) head-major for the kernels after it; the
//                      dP sums start from -D, so dP - D needs no subtraction.
//                      Each work item also sums its rows' share of dsigma per
//                      head (in a fixed order) into a per-item partial.
//   bwd_sink_kernel    dsigma per head: one work group per head sums the
//                      partials of the dq work items in a fixed order (no
//                      atomics, reproducible).
//   bwd_kv_kernel      work item (sequence, KV head, 128 keys), 4 waves: wave w
//                      holds K and V of its own 32 keys as MFMA fragments and
//                      fp32 dK^T, dV^T for them over all 8 query heads of the
//                      group, so no sum across waves is needed. The waves walk
//                      every 32-query block that can see the keys, from the last
//                      one down, one query head at a time: S = Q K^T and
//                      dP = dO V^T - D (8 + 8 MFMAs, q and dO rows as A operands
//                      from LDS), P and dS in registers, then dV^T += dO^T P and
//                      dK^T += Q^T dS (8 + 8 MFMAs, dO^T and Q^T by transpose
//                      reads). Each step's 32 q and dO rows and their (lse, -D)
//                      words are fetched by the 4 waves together, a quarter each,
//                      two steps ahead, into a ring of four LDS tiles: one barrier
//                      per two steps.
// dq, dk, dv are written once each (no atomics), rounded to bf16 from fp32.
#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

constexpr int BQ = kPrefillBQ;   // query positions per block
constexpr int NK = kBackwardNK;  // keys per tile
constexpr int KSB = 80;          // LDS row stride of the K tile (dq kernel): conflict-free transpose reads
constexpr int VSB = 80;          // LDS row stride of the V tile (dq kernel): 16 B row reads (72 measured 0.5 % slower)
constexpr int QS = 80;           // LDS row stride of a wave's q / dO tile (dk/dv kernel)

__device__ __forceinline__ uint2 ldg8(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }

// dsigma_h = - sum over the head's rows of exp(sigma_h - lse) * D. The dq
// kernel leaves one partial per (head, work item): the sum over the item's 32
// rows. One work group per head adds the partials, each thread a fixed stride
// of items, then a tree (a fixed order: repeated calls give the same bits).
// THD items past the schedule's count hold no partial and are left out.
template <bool THD>
__global__ __launch_bounds__(256) void bwd_sink_kernel(BackwardParams p) {
  __shared__ float part[256];
  const int h = blockIdx.x;
  const float* src = p.dsink_part + (int64_t)h * p.dsink_items;
  const int n = THD ? min(max(__ldg(p.count_q), 0), p.dsink_items) : p.dsink_items;
  float acc = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) acc += src[i];
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
// dq: WAVES waves per (sequence, KV head g, 32 query positions) and work group:
// 8 (one work group per CU, each K/V tile staged once for the whole group) or 4
// (two work groups per (sequence, g, block), 8 / WAVES = 2 head halves, two per
// CU, so that one group's prologue overlaps the other's tiles: short items).
// Wave w owns query head 8 g + WAVES * half + w (two 16-column blocks cb of
// positions).
// ---------------------------------------------------------------------------
template <bool THD, bool ROT, bool ROTIN, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(BackwardParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t lds_k[2 * NK * KSB];
  __shared__ __attribute__((aligned(16))) bf16_t lds_v[2 * NK * VSB];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  static_assert(WAVES == 4 || WAVES == 8, "one wave per query head of the group or of its half");
  constexpr int NTH = 64 * WAVES;
  constexpr int HALVES = kGroup / WAVES;
  const int Hkv = p.num_kv_heads, Hq = Hkv * kGroup;
  // consecutive work groups take consecutive KV heads (one XCD per KV head with 8 of
  // them), then the head halves, then the items
  const int g = blockIdx.x % Hkv;
  const int hv = (int)(blockIdx.x / Hkv);
  const int item = hv / HALVES;
  const int half = hv - item * HALVES;
  int j, L, ts;
  int64_t row0, bq_, bk_, bv_, bd_, bo_, bqi_;
  if (THD) {
    if (item >= __ldg(p.count_q)) return;
    const int2 w = p.work_q[item];
    j = w.y;
    const int n = min(max(w.x, 0), p.batch - 1);
    ts = min(max(__ldg(p.cu_seqlens + n), 0), p.seqlen);
    L = min(max(__ldg(p.cu_seqlens + n + 1), ts), p.seqlen) - ts;
    row0 = 0; bq_ = bk_ = bv_ = bd_ = bo_ = bqi_ = 0;
  } else {
    const int r = item / p.batch, b = item - r * p.batch;
    j = p.q_blocks - 1 - r;   // most keys first
    ts = 0;
    L = p.seqlen;
    row0 = (int64_t)b * p.seqlen;
    bq_ = b * p.q_sb; bk_ = b * p.k_sb; bv_ = b * p.v_sb; bd_ = b * p.do_sb; bo_ = b * p.o_sb;
    bqi_ = b * p.qi_sb;
  }
  const int q0 = j * BQ;
  if (j < 0 || q0 >= L) {   // an empty item still leaves its (zero) dsigma partial
    if (lane == 0) p.dsink_part[(int64_t)(g * kGroup + WAVES * half + wave) * p.dsink_items + item] = 0.0f;
    return;
  }
  const int qlast = min(q0 + BQ, L) - 1;
  const int W = p.window;
  const uint32_t weff = (W > 0) ? (uint32_t)W : 0x7FFFFFFFu;
  const int kv_lo = (W > 0) ? max(0, q0 - W + 1) : 0;
  const int kv_hi = qlast + 1;
  const int ntiles = (kv_hi - kv_lo + NK - 1) / NK;
  const float sl = p.scale_log2;
  const int head = g * kGroup + WAVES * half + wave;

  // staging: thread -> (rows tid / 8 + NTH / 8 i, 16-byte chunk tid % 8) of the K and V tiles
  constexpr int SP = 64 * 8 / NTH;   // rows per thread
  const int srow = tid >> 3, scc = tid & 7;
  const int32_t krow_b = (int32_t)p.k_st * 2, vrow_b = (int32_t)p.v_st * 2;
  const char* k_tile0 = reinterpret_cast<const char*>(p.k + bk_ + (int64_t)(ts + kv_lo) * p.k_st + (int64_t)g * p.k_sh);
  const char* v_tile0 = reinterpret_cast<const char*>(p.v + bv_ + (int64_t)(ts + kv_lo) * p.v_st + (int64_t)g * p.v_sh);
  const uint32_t koff = (uint32_t)(srow * krow_b + 16 * scc);
  const uint32_t voff = (uint32_t)(srow * vrow_b + 16 * scc);
  uint4 sk[SP], sv[SP];
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    const int rows = min(kv_hi - (kv_lo + t * NK), NK);   // the tile's own rows: the range stays < 2^31 bytes
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_tile0 + (int64_t)t * NK * krow_b, (rows - 1) * krow_b + 2 * kHeadDim);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_tile0 + (int64_t)t * NK * vrow_b, (rows - 1) * vrow_b + 2 * kHeadDim);
#pragma unroll
    for (int i = 0; i < SP; ++i) {
      sk[i] = ldb16(rk, koff + (uint32_t)(i * (NTH / 8) * krow_b));
      sv[i] = ldb16(rv, voff + (uint32_t)(i * (NTH / 8) * vrow_b));
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SP; ++i) {
      *reinterpret_cast<uint4*>(lds_k + buf * NK * KSB + (srow + i * (NTH / 8)) * KSB + 8 * scc) = sk[i];
      *reinterpret_cast<uint4*>(lds_v + buf * NK * VSB + (srow + i * (NTH / 8)) * VSB + 8 * scc) = sv[i];
    }
  };

  if (ntiles > 0) load_tile(0);
  // q~ and dO of the wave's 32 rows as B-operand fragments (lane = query column,
  // 8 consecutive dims); each column's D = <dO, o> (the 16 dims of a lane, then
  // summed over the column's 4 lanes) and lse in log2 units (+inf for a row
  // without any term: its probabilities are 0). Both are also written head-major
  // to the workspace for the dk / dv kernels and the sink gradient, which run
  // after this kernel.
  int qpos[2];
  bf16x8_t qf[2][2], df[2][2];
  float lse2[2];
  f32x4_t negd[2];   // -D of the lane's query, the starting value of the dP^T sums
  const float sig2 = __ldg(p.sinks + head) * kLog2e;
  float dsig = 0.0f;  // this item's share of dsigma for the wave's head: sum of exp2(sig2 - lse2) (-D)
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    qpos[cb] = q0 + 16 * cb + col;
    const int pos = min(qpos[cb], qlast);
    const bf16_t* dp = p.dout + bd_ + (int64_t)(ts + pos) * p.do_st + (int64_t)head * p.do_sh + 8 * grp;
    const bf16_t* op = p.o + bo_ + (int64_t)(ts + pos) * p.o_st + (int64_t)head * p.o_sh + 8 * grp;
    if (ROTIN) {
      // the caller's q, rotated here with the row's table entries (the two chunks of a
      // lane are the rotation pairs i, i + 32), then kept for the dk / dv kernel
      const bf16_t* qp = p.q_in + bqi_ + (int64_t)(ts + pos) * p.qi_st + (int64_t)head * p.qi_sh + 8 * grp;
      const bf16_t* tp = p.table + (int64_t)min(pos, p.table_rows - 1) * kHeadDim + 8 * grp;
      const uint4 x1 = ldg16(qp), x2 = ldg16(qp + 32), c = ldg16(tp), sn = ldg16(tp + 32);
      uint4 y1, y2;
      rope8(x1, x2, c, sn, y1, y2);
      qf[cb][0] = as_bf16x8(y1);
      qf[cb][1] = as_bf16x8(y2);
      if (qpos[cb] <= qlast) {
        bf16_t* qr = p.q_rot + ((row0 + ts + pos) * Hq + head) * kHeadDim + 8 * grp;
        stg16(qr, y1);
        stg16(qr + 32, y2);
      }
    } else {
      const bf16_t* qp = p.q + bq_ + (int64_t)(ts + pos) * p.q_st + (int64_t)head * p.q_sh + 8 * grp;
      qf[cb][0] = as_bf16x8(ldg16(qp));
      qf[cb][1] = as_bf16x8(ldg16(qp + 32));
    }
    const uint4 d0 = ldg16(dp), d1 = ldg16(dp + 32), o0 = ldg16(op), o1 = ldg16(op + 32);
    df[cb][0] = as_bf16x8(d0);
    df[cb][1] = as_bf16x8(d1);
    const float l = p.lse[(row0 + ts + pos) * Hq + head];
    lse2[cb] = (l > -INFINITY) ? l * kLog2e : INFINITY;
    float dot = 0.0f;
    const uint32_t* pd0 = reinterpret_cast<const uint32_t*>(&d0);
    const uint32_t* pd1 = reinterpret_cast<const uint32_t*>(&d1);
    const uint32_t* po0 = reinterpret_cast<const uint32_t*>(&o0);
    const uint32_t* po1 = reinterpret_cast<const uint32_t*>(&o1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dot += bf16_lo(pd0[i]) * bf16_lo(po0[i]) + bf16_hi(pd0[i]) * bf16_hi(po0[i]) +
             bf16_lo(pd1[i]) * bf16_lo(po1[i]) + bf16_hi(pd1[i]) * bf16_hi(po1[i]);
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    negd[cb] = f32x4_t{-dot, -dot, -dot, -dot};
    if (grp == 0 && qpos[cb] <= qlast) {
      const int64_t rr = (int64_t)head * p.tokens + row0 + ts + pos;
      reinterpret_cast<float2*>(p.ld)[rr] = make_float2(lse2[cb], -dot);
      if (sig2 > -INFINITY) dsig += __builtin_amdgcn_exp2f(sig2 - lse2[cb]) * -dot;
    }
  }
  // the 32 rows' terms sit in lanes 0..15 (2 each); a fixed xor tree over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) dsig += __shfl_xor(dsig, off);
  if (lane == 0) p.dsink_part[(int64_t)head * p.dsink_items + item] = dsig;

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

    // S^T = K Q^T and dP^T - D = V dO^T - D: [kb][cb] element r = key kb*16 + 4*grp + r, query col
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
        dpt[kb][cb] = mfma16(c1, df[cb][1], mfma16(c0, df[cb][0], negd[cb]));   // dP^T - D
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
          x[r] = pr * dpt[kb][cb][r];
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
// dk and dv: one work group of 4 waves per (sequence, KV head g, 128 keys).
// Wave w holds K and V of the 32 keys t0 + 32 w .. + 31 as MFMA fragments and
// fp32 dK^T, dV^T for them (64 VGPRs) over all 8 query heads of the group, so no
// sum across waves is needed. The 4 waves walk the same steps (32 queries of
// one head each) and share each step's q / dO rows through LDS tiles that each
// wave fills a quarter of: a row is fetched once per work group, not once per
// wave.
// ---------------------------------------------------------------------------
constexpr int KT = kBackwardKT;   // keys per work group
static_assert(KT == 4 * 32, "one wave per 32 keys");

template <bool THD, bool ROT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kv_kernel(BackwardParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t lds_t[4][2 * BQ * QS];   // [buffer][q tile, dO tile]
  __shared__ __attribute__((aligned(16))) float lds_ld[4][2 * BQ];        // [buffer][lse of 32 queries, -D of 32]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int Hkv = p.num_kv_heads;
  const int item = blockIdx.x / Hkv;
  const int g = blockIdx.x - item * Hkv;
  int jt0, jt1 = -1, L, ts;
  int64_t row0, bq_, bk_, bv_, bd_;
  if (THD) {
    if (item >= __ldg(p.count_k)) return;
    const int2 w = p.work_k[item];
    const int n = min(max(w.x, 0), p.batch - 1);
    ts = min(max(__ldg(p.cu_seqlens + n), 0), p.seqlen);
    L = min(max(__ldg(p.cu_seqlens + n + 1), ts), p.seqlen) - ts;
    jt0 = (L + KT - 1) / KT - 1 - w.y;   // the list counts tiles from the end: most queries first
    row0 = 0; bq_ = bk_ = bv_ = bd_ = 0;
  } else {
    int r, b;
    if (p.kv_pairs) {
      // Full causal: key tile t is seen by the queries from 128 t on, so its work falls
      // linearly with t. Each work group takes two tiles. The first half of the grid
      // (dispatched first, one per CU, and faster: the older waves win the issue
      // arbitration) takes {i, 3T/4 - 1 - i}, the second half {T/4 + i, T - 1 - i},
      // i < T/4: 5T/4 + 1 against 3T/4 + 1 tiles of work, so that both end together.
      const int T = p.k_tiles, q4 = T / 4, half = p.batch * q4;
      const bool second = item >= half;
      const int it2 = second ? item - half : item;
      r = it2 / p.batch;
      b = it2 - r * p.batch;
      jt0 = second ? q4 + r : r;
      jt1 = second ? T - 1 - r : 3 * q4 - 1 - r;
    } else {
      r = item / p.batch;
      b = item - r * p.batch;
      jt0 = r;                  // tile 0 is seen by every query: most work first
    }
    ts = 0;
    L = p.seqlen;
    row0 = (int64_t)b * p.seqlen;
    bq_ = b * p.q_sb; bk_ = b * p.k_sb; bv_ = b * p.v_sb; bd_ = b * p.do_sb;
  }
  for (int pi = 0; pi < 2; ++pi) {
  const int jt = pi ? jt1 : jt0;
  const int t0 = jt * KT;
  if (jt < 0 || t0 >= L) continue;   // uniform over the work group
  const int tlast = min(t0 + KT, L) - 1;
  const int k0 = t0 + 32 * wave;   // the wave's first key (past tlast: the wave only helps fetch)
  const int W = p.window;
  const uint32_t weff = (W > 0) ? (uint32_t)W : 0x7FFFFFFFu;
  const int qhi = (W > 0) ? min(L - 1, tlast + W - 1) : L - 1;   // last query that sees a key of the tile
  const float sl = p.scale_log2;

  // K and V of the wave's 32 keys as B-operand fragments: lane = key column, 8 consecutive dims
  bf16x8_t kf[2][2], vf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = min(k0 + kb * 16 + col, tlast);
    const bf16_t* kp = p.k + bk_ + (int64_t)(ts + key) * p.k_st + (int64_t)g * p.k_sh + 8 * grp;
    const bf16_t* vp = p.v + bv_ + (int64_t)(ts + key) * p.v_st + (int64_t)g * p.v_sh + 8 * grp;
    kf[kb][0] = as_bf16x8(ldg16(kp));
    kf[kb][1] = as_bf16x8(ldg16(kp + 32));
    vf[kb][0] = as_bf16x8(ldg16(vp));
    vf[kb][1] = as_bf16x8(ldg16(vp + 32));
  }
  f32x4_t dkt[4][2], dvt[4][2];   // [d block][key block]: element r = dim 16*db + 4*grp + r, key col
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) dkt[a][b] = dvt[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fetch of a step's rows: wave w takes rows 8 w .. 8 w + 7 of the 32, lane =
  // (row, 16-byte chunk). Rows are read through buffer ranges that end with the
  // sequence: rows past it read as zeros (their dO is 0, so they add nothing to
  // dV or dK) and need no clamps; one 32-bit offset per load (the host checks
  // that a sequence's rows span less than 2 GiB). The (lse, -D) words of the 32
  // queries come with them, one per lane.
  const int srow = 8 * wave + (lane >> 3), sch = lane & 7;
  const int32_t qrow_b = (int32_t)p.q_st * 2, drow_b = (int32_t)p.do_st * 2;
  struct Fetch { uint4 q, d; uint32_t w; };
  auto fetch = [&](int qb, int hh, Fetch& f) __attribute__((always_inline)) {
    const int q0 = qb * BQ;
    const int head = g * kGroup + hh;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(p.q + bq_ + (int64_t)ts * p.q_st + (int64_t)head * p.q_sh, (L - 1) * qrow_b + 2 * kHeadDim);
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(p.dout + bd_ + (int64_t)ts * p.do_st + (int64_t)head * p.do_sh, (L - 1) * drow_b + 2 * kHeadDim);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.ld + 2 * ((int64_t)head * p.tokens + row0 + ts), L * 8);
    f.q = ldb16(rq, (uint32_t)((q0 + srow) * qrow_b + 16 * sch));
    f.d = ldb16(rd, (uint32_t)((q0 + srow) * drow_b + 16 * sch));
    f.w = __builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)((2 * q0 + lane) * 4), 0, 0);
  };
  auto write_tile = [&](int buf, const Fetch& f) __attribute__((always_inline)) {
    bf16_t* lq = lds_t[buf];
    *reinterpret_cast<uint4*>(lq + srow * QS + 8 * sch) = f.q;
    *reinterpret_cast<uint4*>(lq + BQ * QS + srow * QS + 8 * sch) = f.d;
    // words 16 w .. 16 w + 15 of the 64, split into the lse and -D vectors
    if ((lane >> 4) == wave) lds_ld[buf][(lane & 1) * BQ + (lane >> 1)] = __uint_as_float(f.w);
  };

  // One step: 32 queries (block qb) of head hh against the wave's 32 keys, from
  // LDS buffer buf. A wave whose keys the block cannot see skips it.
  auto step = [&](int buf, int qb) __attribute__((always_inline)) {
    const int q0 = qb * BQ;
    const bool none = (k0 > tlast) || (q0 + BQ - 1 < k0) || (W > 0 && q0 - (k0 + 31) >= W);
    if (none) return;
    const bool full = (q0 >= k0 + 31) && (W == 0 || q0 + BQ - 1 - k0 < W);
    const bf16_t* lq = lds_t[buf];
    const bf16_t* ldo = lq + BQ * QS;
    const float* lld = lds_ld[buf];
    // lse (log2 units) and -D of the lane's queries q0 + 16 qm + 4 grp + e, e = 0..3
    f32x4_t l2[2], negd[2];
#pragma unroll
    for (int qm = 0; qm < 2; ++qm) {
      l2[qm] = *reinterpret_cast<const f32x4_t*>(lld + 16 * qm + 4 * grp);
      negd[qm] = *reinterpret_cast<const f32x4_t*>(lld + BQ + 16 * qm + 4 * grp);
    }
    // S = Q K^T and dP - D = dO V^T - D: [qm][kb] element e = query q0 + 16 qm + 4 grp + e,
    // key k0 + 16 kb + col (q and dO rows as A operands: lane = query row, 8 dims)
    f32x4_t s_[2][2], dp_[2][2];
#pragma unroll
    for (int qm = 0; qm < 2; ++qm) {
      const bf16_t* qr = lq + (qm * 16 + col) * QS + 8 * grp;
      const bf16_t* dr = ldo + (qm * 16 + col) * QS + 8 * grp;
      const bf16x8_t qa0 = as_bf16x8(*reinterpret_cast<const uint4*>(qr));
      const bf16x8_t qa1 = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 32));
      const bf16x8_t da0 = as_bf16x8(*reinterpret_cast<const uint4*>(dr));
      const bf16x8_t da1 = as_bf16x8(*reinterpret_cast<const uint4*>(dr + 32));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        s_[qm][kb] = mfma16(qa1, kf[kb][1], mfma16(qa0, kf[kb][0], z));
        dp_[qm][kb] = mfma16(da1, vf[kb][1], mfma16(da0, vf[kb][0], negd[qm]));
      }
    }
    // dO^T and Q^T as A operands (transpose reads of the row-major tiles)
    bf16x8_t a_do[4], a_q[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int off = (4 * grp + (col >> 2)) * QS + 16 * db + 4 * (col & 3);
      const uint2 dlo = lds_read_tr16(ldo + off), dhi = lds_read_tr16(ldo + off + 16 * QS);
      const uint2 qlo = lds_read_tr16(lq + off), qhi2 = lds_read_tr16(lq + off + 16 * QS);
      a_do[db] = __builtin_bit_cast(bf16x8_t, make_uint4(dlo.x, dlo.y, dhi.x, dhi.y));
      a_q[db] = __builtin_bit_cast(bf16x8_t, make_uint4(qlo.x, qlo.y, qhi2.x, qhi2.y));
    }
    // P = exp(S - lse) and dS = P (dP - D), packed as B operands over the 32
    // queries (elements 4 qm .. 4 qm + 3 of a lane's 8)
    uint32_t pw[2][4], dw[2][4];   // [kb][word]
#pragma unroll
    for (int qm = 0; qm < 2; ++qm) {
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int qq = q0 + qm * 16 + 4 * grp + e, key = k0 + kb * 16 + col;
            s_[qm][kb][e] = ((uint32_t)(qq - key) < weff) ? s_[qm][kb][e] : -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[4], dv_[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_[qm][kb][e], sl, -l2[qm][e]));
          dv_[e] = pv[e] * dp_[qm][kb][e];
        }
        pw[kb][2 * qm] = pack_bf16x2(pv[0], pv[1]);
        pw[kb][2 * qm + 1] = pack_bf16x2(pv[2], pv[3]);
        dw[kb][2 * qm] = pack_bf16x2(dv_[0], dv_[1]);
        dw[kb][2 * qm + 1] = pack_bf16x2(dv_[2], dv_[3]);
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dvt[db][kb] = mfma16(a_do[db], __builtin_bit_cast(bf16x8_t, make_uint4(pw[kb][0], pw[kb][1], pw[kb][2], pw[kb][3])),
                             dvt[db][kb]);
        dkt[db][kb] = mfma16(a_q[db], __builtin_bit_cast(bf16x8_t, make_uint4(dw[kb][0], dw[kb][1], dw[kb][2], dw[kb][3])),
                             dkt[db][kb]);
      }
  };

  // Steps: every block of 32 queries that can see the tile, walked from the last
  // one down, each for the 8 query heads. The work groups of one (sequence, KV
  // head) run together on one XCD (consecutive work groups take consecutive KV
  // heads, dealt round-robin over the 8 XCDs) and then read the same q / dO
  // block at about the same time, so L2 serves the repeats. Two steps per
  // barrier (nsteps is a multiple of kGroup, so even): the rows of steps s + 2
  // and s + 3 load while s and s + 1 compute and are written to the other two of
  // four LDS buffers at the end (with one step per barrier the layer took 1 %
  // longer). The last two steps fetch the last step's rows again (no branch
  // around the loads).
  const int qb_lo = t0 / BQ, qb_hi = qhi / BQ;
  const int nsteps = (qb_hi - qb_lo + 1) * kGroup;
  Fetch fa, fb;
  fetch(qb_hi, 0, fa);
  fetch(qb_hi, 1, fb);
  write_tile(0, fa);
  write_tile(1, fb);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    const int na = min(s + 2, nsteps - 1), nb = min(s + 3, nsteps - 1);
    fetch(qb_hi - na / kGroup, na % kGroup, fa);
    fetch(qb_hi - nb / kGroup, nb % kGroup, fb);
    step(s & 3, qb_hi - s / kGroup);
    step((s + 1) & 3, qb_hi - (s + 1) / kGroup);
    write_tile((s + 2) & 3, fa);
    write_tile((s + 3) & 3, fb);
    __syncthreads();
  }

  // epilogue: dk~ = tau dK^T, dk = R^T dk~ (the rotation pairs dims i and i + 32:
  // d blocks pr and pr + 2 of the same lane); dv as accumulated
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = k0 + kb * 16 + col;
    if (key > tlast) continue;
    const int64_t orow = ((row0 + ts + key) * Hkv + g) * kHeadDim + 4 * grp;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      f32x4_t y1 = dkt[pr][kb] * p.scale, y2 = dkt[pr + 2][kb] * p.scale;
      if (ROT) {
        const bf16_t* tp = p.table + (int64_t)min(key, p.table_rows - 1) * kHeadDim + 16 * pr + 4 * grp;
        rotate_back4(y1, y2, ldg8(tp), ldg8(tp + 32));
      }
      *reinterpret_cast<uint2*>(p.dk + orow + 16 * pr) = pack4(y1);
      *reinterpret_cast<uint2*>(p.dk + orow + 16 * pr + 32) = pack4(y2);
      *reinterpret_cast<uint2*>(p.dv + orow + 16 * pr) = pack4(dvt[pr][kb]);
      *reinterpret_cast<uint2*>(p.dv + orow + 16 * pr + 32) = pack4(dvt[pr + 2][kb]);
    }
  }
  }   // key tiles of the work group
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* x, int32_t n, float value) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = value;
}

template <bool THD, bool ROT>
hipError_t launch_all(const BackwardParams& p, hipStream_t stream) {
  const int Hq = p.num_kv_heads * kGroup;
  const int64_t rep = THD ? 1 : p.batch;
  // dq first: it also writes D and lse (log2 units) for the kernels after it
  // window layers (a few key tiles per item): 4-wave work groups, two per CU
  const uint32_t nq = (uint32_t)(p.q_blocks * rep * p.num_kv_heads);
  if (p.window > 0) {
    if (ROT && p.q_in)
      hipLaunchKernelGGL((bwd_dq_kernel<THD, ROT, true, 4>), dim3(2 * nq), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<THD, ROT, false, 4>), dim3(2 * nq), dim3(256), 0, stream, p);
  } else {
    if (ROT && p.q_in)
      hipLaunchKernelGGL((bwd_dq_kernel<THD, ROT, true, 8>), dim3(nq), dim3(512), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<THD, ROT, false, 8>), dim3(nq), dim3(512), 0, stream, p);
  }
  hipLaunchKernelGGL(bwd_sink_kernel<THD>, dim3(Hq), dim3(256), 0, stream, p);
  const int64_t kv_items = p.kv_pairs ? (int64_t)p.k_tiles / 2 * rep : (int64_t)p.k_tiles * rep;
  hipLaunchKernelGGL((bwd_kv_kernel<THD, ROT>), dim3((uint32_t)(kv_items * p.num_kv_heads)), dim3(256), 0, stream,
                     p);
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
