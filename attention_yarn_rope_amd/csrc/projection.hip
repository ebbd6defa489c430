// q/k/v projections of GPT-OSS attention with the RoPE applied in the GEMM's
// epilogue, on gfx950.
//
// The gpt-oss-20b module print-out lists q_proj 2880 -> 4096 and k_proj /
// v_proj 2880 -> 512, each a Linear with bias; the rope_utils page
// (_apply_rotary_emb_qk) rotates q and k in their dtype with one table. Each
// output here is z = x W^T + b, accumulated in fp32 and rounded once to bf16;
// q and k are then rotated exactly (rope1: one more rounding), so the fused
// result equals the projection followed by the standalone rotation, bit for
// bit.
//
// One work group of 8 waves per 256 x 256 output tile (tokens x features over
// the concatenated q, k, v outputs); wave (wm, wn) owns 128 tokens x 64
// features (one head): 8 x 4 MFMA tiles of v_mfma_f32_16x16x32_bf16 and 128
// fp32 accumulators per lane, two waves per SIMD. Both operands are
// K-contiguous rows (x rows; W rows, Linear's layout), so every MFMA fragment
// is one 16-byte LDS read of a staged row. K advances 64 at a time through two
// LDS stages (2 x 80 KB): the next step's 32 KB of x and 32 KB of W are loaded
// into registers while the current stage feeds 64 MFMAs per wave, then
// written to the other stage; one barrier per step.
// Work groups are dealt round-robin over the 8 XCDs; each XCD takes a band of
// token tiles and walks them 4 at a time across the feature tiles, so the
// concurrent work groups of an XCD share x rows and W rows in its L2.
//
// Epilogue: the output layout of the MFMA puts feature n and its rotation
// partner n + 32 (same head) in the same lane (column blocks nb and nb + 2),
// for 4 consecutive tokens per register quad, so the rotation needs no data
// exchange. With rotary_dim 32 the partners are blocks 0 and 1 and blocks 2,
// 3 of the head pass through.
#include "common.h"
#include "internal.h"

namespace gptoss {
namespace {

constexpr int TT = kProjTile;   // tokens per tile
constexpr int TF = kProjTile;   // features per tile
constexpr int TK = 64;          // K per step
constexpr int LS = 80;          // LDS row stride (elements): 16-byte row reads without bank conflicts (measured)
constexpr int kStage = (TT + TF) * LS;

__device__ __forceinline__ float round_bf16f(float z) { return bf16_lo(pack_bf16x2(z, 0.0f)); }

template <bool ROT, bool THD>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void qkv_proj_kernel(ProjParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;   // 128-token half, 64-feature quarter

  // tile of this work group: XCD band of token tiles, 4 token tiles x all feature tiles at a time
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int band = (p.m_tiles + 7) / 8;
  constexpr int GM = 4;
  const int g = local / (GM * p.n_tiles);
  const int gm = min(GM, band - g * GM);
  if (gm <= 0) return;
  const int in = local - g * GM * p.n_tiles;
  const int nt = in / gm;
  const int mt = xcd * band + g * GM + in % gm;
  if (mt >= p.m_tiles || nt >= p.n_tiles) return;
  // (the divisions above run on the vector unit: mark the results wave-uniform)
  const int m0 = __builtin_amdgcn_readfirstlane(mt * TT), n0 = __builtin_amdgcn_readfirstlane(nt * TF);

  // staging: thread -> rows (tid >> 3) + 64 i (i = 0..3) of the x tile and of the W tile, 16-byte chunk tid & 7
  const int srow = tid >> 3, sch = tid & 7;
  const int32_t xrow_b = (int32_t)p.x_st * 2;   // a tile's rows span < 2 GiB (host check)
  const int rows_valid = __builtin_amdgcn_readfirstlane(min(TT, p.tokens - m0));
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(p.x + (int64_t)m0 * p.x_st, (rows_valid - 1) * xrow_b + 2 * p.hidden);
  // the feature tile lies inside one of the q, k, v weights (their widths are multiples of 256)
  const int wsel = (n0 < p.nq) ? 0 : (n0 < p.nq + p.nkv ? 1 : 2);
  const int nl0 = n0 - (wsel == 0 ? 0 : (wsel == 1 ? p.nq : p.nq + p.nkv));
  const int32_t wrow_b = 2 * p.hidden;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w[wsel] + (int64_t)nl0 * p.hidden, TF * wrow_b);
  uint4 ra[4], rb[4];
  auto load = [&](int ks, uint4 (&sa)[4], uint4 (&sb)[4]) __attribute__((always_inline)) {
    const uint32_t k_b = (uint32_t)(ks * TK * 2 + 16 * sch);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = ldb16(rx, (uint32_t)((srow + 64 * i) * xrow_b) + k_b);
      sb[i] = ldb16(rw, (uint32_t)((srow + 64 * i) * wrow_b) + k_b);
    }
  };
  auto store = [&](int st, const uint4 (&sa)[4], const uint4 (&sb)[4]) __attribute__((always_inline)) {
    bf16_t* a = lds + st * kStage;
    bf16_t* b = a + TT * LS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(a + (srow + 64 * i) * LS + 8 * sch) = sa[i];
      *reinterpret_cast<uint4*>(b + (srow + 64 * i) * LS + 8 * sch) = sb[i];
    }
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = p.hidden / TK;
  auto compute = [&](int st) __attribute__((always_inline)) {
    const bf16_t* As = lds + st * kStage + (wm * 128 + col) * LS + 8 * grp;
    const bf16_t* Bs = lds + st * kStage + TT * LS + (wn * 64 + col) * LS + 8 * grp;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      bf16x8_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = *reinterpret_cast<const bf16x8_t*>(Bs + i * 16 * LS + 32 * sub);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(As + mb * 16 * LS + 32 * sub);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma16(a, b[nb], acc[mb][nb]);
      }
    }
  };
  load(0, ra, rb);
  store(0, ra, rb);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    load(min(ks + 1, nk - 1), ra, rb);   // the last step loads its own rows again (no branch around the loads)
    compute(ks & 1);
    if (ks + 1 < nk) store((ks + 1) & 1, ra, rb);
    __syncthreads();
  }

  // epilogue: the wave's 64 features are one head of q, k or v
  const int hc = n0 + wn * 64;
  const int which = (hc < p.nq) ? 0 : (hc < p.nq + p.nkv ? 1 : 2);
  const int fbase = hc - (which == 0 ? 0 : (which == 1 ? p.nq : p.nq + p.nkv));
  const int width = (which == 0) ? p.nq : p.nkv;
  uint16_t* out = p.out[which];
  float bias[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
    bias[qb] = p.b[which] ? bf16_lo((uint32_t)__ldg(p.b[which] + fbase + 16 * qb + col)) : 0.0f;
  const bool rot = ROT && which < 2;
  // Two halves of 64 tokens. Per half the wave first copies its tokens' table
  // rows into its LDS block (one round trip of coalesced 16-byte loads instead
  // of a dependent 2-byte load per token), then rounds, rotates and writes its
  // 64 x 64 bf16 results to the same block, then stores whole 128-byte head
  // rows in 16-byte pieces. The LDS stages are free after the last barrier of
  // the K loop; each wave uses only its own block.
  constexpr int OS = 72;                   // LDS row stride of the output rows (elements)
  constexpr int kBlock = 64 * OS + 64 * 64;   // output rows, then 64 table rows of 64 entries
  static_assert(8 * kBlock <= 2 * kStage, "the per-wave blocks fit in the stages");
  uint16_t* ob = reinterpret_cast<uint16_t*>(lds) + wave * kBlock;
  uint16_t* tb = ob + 64 * OS;
  const int tw = 2 * p.rot_half;           // table row width (entries)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (rot) {
      // table rows of tokens wm * 128 + 64 half + i: lane -> row (lane >> 3) + 8 j, 16-byte piece lane & 7
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = (lane >> 3) + 8 * j;
        const int pc = lane & 7;
        if (8 * pc < tw) {
          const int t = min(m0 + wm * 128 + 64 * half + i, p.tokens - 1);
          int pos = THD ? t - __ldg(p.cu_seqlens + find_seq(p.cu_seqlens, p.batch, t)) : t % p.seqlen;
          pos = min(max(pos, 0), p.table_rows - 1);
          const uint4 v = ldg16(p.table + (int64_t)pos * tw + 8 * pc);
          *reinterpret_cast<uint4*>(tb + i * 64 + 8 * pc) = v;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int mh = 0; mh < 4; ++mh) {
      const int mb = 4 * half + mh;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int il = mh * 16 + 4 * grp + r;   // row within the half
        float y[4];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) y[qb] = round_bf16f(acc[mb][qb][r] + bias[qb]);
        if (rot) {
          const uint16_t* tp = tb + il * 64;
          if (p.rot_half == 32) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              const int d = 16 * qb + col;
              rope1(y[qb], y[qb + 2], bf16_lo(tp[d]), bf16_lo(tp[32 + d]), y[qb], y[qb + 2]);
            }
          } else {   // rotary_dim 32: dims 0..15 pair with 16..31, dims 32..63 pass through
            rope1(y[0], y[1], bf16_lo(tp[col]), bf16_lo(tp[16 + col]), y[0], y[1]);
          }
        }
        uint16_t* orow = ob + il * OS + col;
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) orow[16 * qb] = (uint16_t)(pack_bf16x2(y[qb], 0.0f) & 0xFFFFu);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rl = (lane >> 3) + 8 * j;
      const int t = m0 + wm * 128 + 64 * half + rl;
      const uint4 val = *reinterpret_cast<const uint4*>(ob + rl * OS + 8 * (lane & 7));
      if (t < p.tokens) *reinterpret_cast<uint4*>(out + (int64_t)t * width + fbase + 8 * (lane & 7)) = val;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // the block's reads are done before the next half rewrites it
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_qkv_proj(const ProjParams& p, hipStream_t stream) {
  if (p.tokens == 0) return hipSuccess;
  const int band = (p.m_tiles + 7) / 8;
  const dim3 grid((unsigned)(8 * band * p.n_tiles));
  const bool thd = p.cu_seqlens != nullptr;
  if (!p.table)
    hipLaunchKernelGGL((qkv_proj_kernel<false, false>), grid, dim3(512), 0, stream, p);
  else if (thd)
    hipLaunchKernelGGL((qkv_proj_kernel<true, true>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((qkv_proj_kernel<true, false>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gptoss
