// Device helpers shared by the gfx950 kernels: bf16 packing, the exactly
// rounded RoPE pair rotation, MFMA fragment types and LDS transpose reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptoss {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round two fp32 values to bf16 (nearest-even, hardware v_cvt_pk_bf16_f32) and pack.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// RoPE rotation of one half-split pair, rounded once to bf16.
//
// y1 = x1*C - x2*S and y2 = x2*C + x1*S with bf16 x1, x2, C, S. Each product of
// two bf16 values has at most 16 significant bits, so it is exact in fp32
// (barring fp32 underflow below 2^-126). One fma then yields y correctly
// rounded to fp32. Rounding that fp32 value to bf16 can only differ from
// rounding the exact value once when the fp32 result sits exactly on a bf16
// midpoint (low 16 bits == 0x8000) while the exact value does not; then the
// fp32 value is moved one fp32 ulp towards the exact value, which is below or
// above the midpoint by the sign of the fma's rounding error e (found with
// the TwoSum error-free transformation). The result equals the exact value
// rounded once to bf16 (nearest-even).
//
// The fix-up only runs where it can matter. Write y = p - t with p and t the
// two exact products. Each is an integer multiple of 2^(E - 15), E its binary
// exponent, so y is a multiple of 2^(min(Ep, Et) - 15) and fits in fp32's 24
// bits unless its exponent reaches min(Ep, Et) + 9. An inexact result s
// therefore has min(|p|, |t|) < 2^(Es - 8) <= |s| * 2^-8. Outputs on a bf16
// midpoint that fail this test are exact (the common case: exact results often
// end in zero bits) and need no fix; with random bf16 data the test leaves
// about one wave in a hundred on the slow path instead of nearly all of them.
// ---------------------------------------------------------------------------
#pragma clang fp contract(off)
__device__ __forceinline__ float two_sum_err(float a, float b, float s) {
  float bb = s - a;
  return (a - (s - bb)) + (b - bb);
}
#pragma clang fp contract(on)

// Exact-rounding fix-up of s = RN_fp32(a + b) where a and b are exact fp32
// values (branch free: a select, not a branch, per element).
__device__ __forceinline__ float fix_bf16_tie(float a, float b, float s) {
  const uint32_t u = __float_as_uint(s);
  const float e = two_sum_err(a, b, s);
  const uint32_t step = (e == 0.0f) ? 0u : (((e > 0.0f) == (s > 0.0f)) ? 1u : 0xFFFFFFFFu);
  return __uint_as_float(((u & 0xFFFFu) == 0x8000u) ? u + step : u);
}

// s = RN_fp32(p + t) with p, t exact products of bf16 values: true when s lies
// on a bf16 midpoint (low 16 bits 0x8000) and may be inexact (see above).
__device__ __forceinline__ bool maybe_inexact_tie(float s, float p, float t) {
  return ((__float_as_uint(s) & 0xFFFFu) == 0x8000u) &&
         (__builtin_fminf(__builtin_fabsf(p), __builtin_fabsf(t)) < __builtin_fabsf(s) * 0x1p-8f);
}

// Rotate one pair of bf16 values (held in floats) by a bf16 cos / sin: the
// results RN(x1*C - x2*S) and RN(x2*C + x1*S), each rounded once to bf16 (the
// products are exact in fp32; fix_bf16_tie repairs an inexact sum that lands on
// a bf16 midpoint, branch free). Returns the two results as floats ready for
// pack_bf16x2.
__device__ __forceinline__ void rope1(float a1, float a2, float cc, float ss, float& o1, float& o2) {
  const float p1 = a1 * cc, t1 = a2 * ss, p2 = a2 * cc, t2 = a1 * ss;
  o1 = p1 - t1;
  o2 = p2 + t2;
  // only a result on a bf16 midpoint can need the repair (rare: the lanes that do
  // take the branch)
  const uint32_t mid = ((__float_as_uint(o1) & 0xFFFFu) ^ 0x8000u) * ((__float_as_uint(o2) & 0xFFFFu) ^ 0x8000u);
  if (mid == 0u) {
    o1 = fix_bf16_tie(p1, -t1, o1);
    o2 = fix_bf16_tie(p2, t2, o2);
  }
}

// Rotate 2 NW pairs held as NW 32-bit words of two bf16 each: x1 holds dims
// i..i+2NW-1, x2 their partners i+h.. (h = rotary_dim / 2), c / s the table's
// cos / sin for the same i. Writes rounded bf16 outputs.
template <int NW>
__device__ __forceinline__ void rope_words(const uint32_t* px1, const uint32_t* px2, const uint32_t* pc,
                                           const uint32_t* ps, uint32_t* py1, uint32_t* py2) {
  float r1[2 * NW], r2[2 * NW];
  bool fix = false;   // some output may be an inexact result on a bf16 midpoint
#pragma unroll
  for (int w = 0; w < NW; ++w) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float a1 = h ? bf16_hi(px1[w]) : bf16_lo(px1[w]);
      float a2 = h ? bf16_hi(px2[w]) : bf16_lo(px2[w]);
      float cc = h ? bf16_hi(pc[w]) : bf16_lo(pc[w]);
      float ss = h ? bf16_hi(ps[w]) : bf16_lo(ps[w]);
      float p1 = a1 * cc, t1 = a2 * ss;        // exact
      float p2 = a2 * cc, t2 = a1 * ss;        // exact
      float o1 = p1 - t1;                      // RN(x1*C - x2*S)
      float o2 = p2 + t2;                      // RN(x2*C + x1*S)
      r1[2 * w + h] = o1;
      r2[2 * w + h] = o2;
      fix |= maybe_inexact_tie(o1, p1, t1);
      fix |= maybe_inexact_tie(o2, p2, t2);
    }
  }
  if (fix) {  // rare: redo every element with the exact fix-up (a no-op where not needed)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float a1 = h ? bf16_hi(px1[w]) : bf16_lo(px1[w]);
        float a2 = h ? bf16_hi(px2[w]) : bf16_lo(px2[w]);
        float cc = h ? bf16_hi(pc[w]) : bf16_lo(pc[w]);
        float ss = h ? bf16_hi(ps[w]) : bf16_lo(ps[w]);
        r1[2 * w + h] = fix_bf16_tie(a1 * cc, -(a2 * ss), r1[2 * w + h]);
        r2[2 * w + h] = fix_bf16_tie(a2 * cc, a1 * ss, r2[2 * w + h]);
      }
    }
  }
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    py1[w] = pack_bf16x2(r1[2 * w], r1[2 * w + 1]);
    py2[w] = pack_bf16x2(r2[2 * w], r2[2 * w + 1]);
  }
}

// Rotate 8 pairs (16-byte chunks: dims i..i+7 and i+h..i+h+7).
__device__ __forceinline__ void rope8(const uint4& x1, const uint4& x2, const uint4& c,
                                      const uint4& s, uint4& y1, uint4& y2) {
  rope_words<4>(reinterpret_cast<const uint32_t*>(&x1), reinterpret_cast<const uint32_t*>(&x2),
                reinterpret_cast<const uint32_t*>(&c), reinterpret_cast<const uint32_t*>(&s),
                reinterpret_cast<uint32_t*>(&y1), reinterpret_cast<uint32_t*>(&y2));
}
// Rotate 4 pairs (8-byte chunks).
__device__ __forceinline__ void rope4(const uint2& x1, const uint2& x2, const uint2& c,
                                      const uint2& s, uint2& y1, uint2& y2) {
  rope_words<2>(reinterpret_cast<const uint32_t*>(&x1), reinterpret_cast<const uint32_t*>(&x2),
                reinterpret_cast<const uint32_t*>(&c), reinterpret_cast<const uint32_t*>(&s),
                reinterpret_cast<uint32_t*>(&y1), reinterpret_cast<uint32_t*>(&y2));
}



// ---------------------------------------------------------------------------
// MFMA v_mfma_f32_16x16x32_bf16 (one wave of 64 lanes):
//   A[i][k]: lane i + 16*(k/8), element k%8     (16 rows x 32 k)
//   B[k][n]: lane n + 16*(k/8), element k%8     (32 k x 16 cols)
//   D[i][n]: lane n + 16*(i/4), element i%4     (16 x 16, fp32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives in slot j the
// (i % 4)-th 16-bit element of the 8-byte chunk addressed by lane 4*j + i/4 of
// the same group.
__device__ __forceinline__ uint2 lds_read_tr16(const bf16_t* lds_ptr) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  // A C-style cast from the generic pointer emits an addrspacecast to LDS.
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
  return __builtin_bit_cast(uint2, v);
}

// Sum of the two bf16 halves of w, added to acc (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, acc, false);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return __builtin_fmaxf(a, __builtin_fmaxf(b, c)); }

// Raw buffer resource over `bytes` bytes from `base` (stride 0, the gfx9 word 3).
// A buffer load whose offset lies past `bytes` returns zeros instead of reading.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes < 0 ? 0 : bytes, 0x00020000);
}
// 16-byte buffer loads: cached, and non-temporal (buffer_load_dwordx4 ... nt) for read-once data
__device__ __forceinline__ uint4 ldb16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ldb16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 ldg16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void stg16(bf16_t* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Sequence index of packed token t: the largest n with cu[n] <= t.
__device__ __forceinline__ int32_t find_seq(const int32_t* cu, int32_t num_seqs, int32_t t) {
  int32_t lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int32_t mid = (lo + hi + 1) >> 1;
    if (__ldg(cu + mid) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Chunk c (dims 8c .. 8c + 7, already loaded as xc) of a row rotated with
// rotary_dim = 16 hb (rope_utils page, apply_rotary_emb: the first rotary_dim
// dims rotate in half-split pairs (i, i + rotary_dim / 2), the rest pass
// through). A chunk below hb pairs with chunk c + hb (its y1 = x1 C - x2 S), a
// chunk in [hb, 2 hb) with chunk c - hb (its y2 = x2 C + x1 S), chunks at or
// past 2 hb are returned as they are. row points at the row, tab at its table
// row (the cos of the 8 hb pairs, then their sin). Rounded exactly like rope8.
__device__ __forceinline__ uint4 rope_chunk_partial(const bf16_t* row, const bf16_t* tab, int c, int hb,
                                                    const uint4& xc) {
  if (c >= 2 * hb) return xc;
  const bool first = c < hb;
  const int pair = first ? c : c - hb;
  const uint4 partner = ldg16(row + 8 * (first ? c + hb : c - hb));
  const uint4 cs = ldg16(tab + 8 * pair), sn = ldg16(tab + 8 * (hb + pair));
  uint4 y1, y2;
  if (first) {
    rope8(xc, partner, cs, sn, y1, y2);
    return y1;
  }
  rope8(partner, xc, cs, sn, y1, y2);
  return y2;
}

// Rotation of one 64-dim row by a table row (cos of the rotary_dim / 2 pairs,
// then their sin), for the 8-dim chunks c and c + 4 a thread owns. Chunk c <
// hb (hb = rotary_dim / 16) is rotated together with chunk c + hb, its pair
// partner, and both results are stored; chunks at or past 2 hb (the partial-
// rotary tail) are copied; chunks in [hb, 2 hb) are stored by their partner's
// owner. With rotary_dim = 64 (hb = 4) thread cc rotates chunks cc and cc + 4.
__device__ __forceinline__ void rotate_row_chunks(const uint16_t* x, uint16_t* y, const uint16_t* tab, int hb,
                                                  int cc) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = cc + 4 * j;
    if (c < hb) {
      const uint4 x1 = ldg16(x + 8 * c), x2 = ldg16(x + 8 * (c + hb));
      uint4 y1, y2;
      rope8(x1, x2, ldg16(tab + 8 * c), ldg16(tab + 8 * (c + hb)), y1, y2);
      stg16(y + 8 * c, y1);
      stg16(y + 8 * (c + hb), y2);
    } else if (c >= 2 * hb) {
      stg16(y + 8 * c, ldg16(x + 8 * c));
    }
  }
}

}  // namespace gptoss
