// Device-side helpers shared by the quantizer kernels: the MX cast of one
// value, Philox4x32-10, the exact fallback for the Hadamard sums, and small
// bit utilities.
// gfx950 (CDNA4) only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/mxfp4.h"

namespace mx {

// ---------------------------------------------------------------------------
// The MX cast of one value: E8M0 scale as a float, 4-bit code, scale byte.

__device__ __forceinline__ uint32_t e8m0_scale_bits(uint32_t byte) {
  // the float whose exponent the scaled conversions divide by: 2^(byte-127)
  return byte ? (byte << 23) : 0x00400000u;        // 2^-127 is a subnormal float
}

// 4-bit code of one value y of a block with scale byte `byte` (finite y):
// sign bit 3, magnitude code = |y| / 2^(byte-127) on the grid, rounded by
// RTNE, or (SR) up from the level below iff floor(frac * 2^22) + (u >> 10)
// >= 2^22; saturating at the top level.  The element's 16-bit draw r comes in
// the top half of u (u = r << 16), which makes the rule floor(frac * 2^16) + r
// >= 2^16 exactly: floor(frac 2^22) + 2^6 r >= 2^22 <=> floor(frac 2^16) + r
// >= 2^16, r being an integer.
template <int GRID, int ROUND>
__device__ __forceinline__ uint32_t cast_one(float yy, uint32_t byte, uint32_t u) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  const float sc = __uint_as_float(e8m0_scale_bits(byte));
  if constexpr (GRID == MX_GRID_E2M1 && ROUND == MX_ROUND_RTNE) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, yy, 0.0f, sc, 0) & 0xFu;
  } else if constexpr (GRID == MX_GRID_E2M1) {
    // gfx950's stochastic fp4 conversion applies exactly this rule (the
    // element's own draw; the pair's second value is a placeholder, and the
    // other result bytes are not kept)
    return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, (v2f){yy, 0.0f}, u, sc, 0) & 0xFu;
  } else {
    // uniform grid: magnitude code = t = |y| * 2^(2-e), rounded (t < 8 in a finite block)
    const int ebias = (int)byte - 127;
    uint32_t k;
    if constexpr (ROUND == MX_ROUND_RTNE) {
      // t + 2^23 rounds t (< 2^23) to the nearest integer, ties to even, into the mantissa's low bits; the
      // bit pattern's unsigned min with that of 2^23 + 7 then saturates as min(k, 7) does
      const float f = ldexpf(fabsf(yy), 2 - ebias) + 8388608.0f;
      return (min(__float_as_uint(f), 0x4B000007u) & 7u) | ((__float_as_uint(yy) >> 28) & 8u);
    } else {
      // u holds the 16-bit draw r in its top half.  T = floor(t * 2^16) (exact scaling, truncating
      // conversion) is floor(t) * 2^16 + floor(f * 2^16), so floor(t) rounds up iff floor(f * 2^16) + r >= 2^16,
      // that is k = (T + r) >> 16: the high word of T * 2^16 + u, one 32x32 -> 64 multiply-add.  NaN converts
      // to T = 0 and Inf to T = 2^32 - 1, as the codes of such blocks are never kept.
      const uint32_t T = (uint32_t)ldexpf(fabsf(yy), 18 - ebias);
      k = (uint32_t)(((uint64_t)T * 65536u + u) >> 32);
    }
    return min(k, 7u) | ((__float_as_uint(yy) >> 28) & 8u);
  }
}

// Scale byte of a block whose largest |y| has float exponent field expf.
template <int GRID>
__device__ __forceinline__ uint32_t scale_byte(uint32_t expf) {
  constexpr uint32_t kEmax = GRID == MX_GRID_E2M1 ? 2u : 0u;
  return expf > kEmax ? expf - kEmax : 0u;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies on a 128-bit counter, Weyl-bumped 64-bit key.  The key
// is wave-uniform (it lives in SGPRs); each lane runs its own counter.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct U4 { uint32_t x, y, z, w; };

// a ^ b ^ c in one gfx950 three-input bit operation (truth table 0x96)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ U4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                            uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c0 * kPhiloxM0;
    const uint64_t p1 = (uint64_t)c2 * kPhiloxM1;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return U4{c0, c1, c2, c3};
}

// Philox4x32-10 of the NC counters (ctr + q, stream, 0), q = 0..NC-1 (ctr is
// the 64-bit block index in the first two counter words), run in lockstep:
// the dependency chains of multiplies interleave instead of waiting on one
// another.
template <int NC>
__device__ __forceinline__ void philox4x32_10_xn(uint64_t ctr, uint32_t stream, uint32_t k0, uint32_t k1,
                                                 U4 (&out)[NC]) {
  uint32_t c0[NC], c1[NC], c2[NC], c3[NC];
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    const uint64_t b = ctr + (uint64_t)q;
    c0[q] = (uint32_t)b;
    c1[q] = (uint32_t)(b >> 32);
    c2[q] = stream;
    c3[q] = 0u;
  }
#pragma unroll
  for (int r = 0; r < 10; ++r) {
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const uint64_t p0 = (uint64_t)c0[q] * kPhiloxM0;
      const uint64_t p1 = (uint64_t)c2[q] * kPhiloxM1;
      const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1[q], k0);
      const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3[q], k1);
      c1[q] = (uint32_t)p1;
      c3[q] = (uint32_t)p0;
      c0[q] = n0;
      c2[q] = n2;
    }
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
#pragma unroll
  for (int q = 0; q < NC; ++q) out[q] = U4{c0[q], c1[q], c2[q], c3[q]};
}

// The stochastic-rounding operands of 8 * NC consecutive elements (element
// index 8 ctr8 + e, e = 0 .. 8 NC - 1): element e takes the 16-bit half e % 2
// (low half first) of word (e % 8) / 2 of the call with counter ctr8 + e / 8,
// placed in the top half of its operand (cast_one takes u = r << 16).
template <int NC>
__device__ __forceinline__ void sr_draws(uint64_t ctr8, uint32_t stream, uint32_t k0, uint32_t k1,
                                         uint32_t (&u)[8 * NC]) {
  U4 r[NC];
  philox4x32_10_xn<NC>(ctr8, stream, k0, k1, r);
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    const uint32_t w[4] = {r[q].x, r[q].y, r[q].z, r[q].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u[8 * q + 2 * j] = w[j] << 16;
      u[8 * q + 2 * j + 1] = w[j] & 0xFFFF0000u;
    }
  }
}

// Eight E2M1 codes of y[0..7] by stochastic rounding from one Philox block r
// (element 2j takes the low half of word j, element 2j + 1 the high half, as
// in sr_draws), packed element 2j in the low nibble.  gfx950's scaled
// stochastic conversion rounds the first value of its pair with bits 31..10
// of the random operand and the second value with bits 30..9 (checked bit for
// bit on the GPU over random values in every E2M1 interval, both signs,
// values on a level and the saturating band).  Each pair is converted twice,
// with element 2j's draw placed at bits 31..16 and element 2j + 1's at bits
// 30..15, zeros below, which is the rule of cast_one for each; the first
// conversion's low nibble and the second's high nibble are kept.
//
// The conversion writes only the byte its op_sel picks and keeps the other
// three bytes of its destination (checked on the GPU against the builtin for
// every byte position).  The compiler's builtin does not model that: it treats
// the whole destination as written, so a chain of builtins loses all but the
// last byte.  The conversions are therefore written as one asm block with
// tied destinations: the four even-element conversions fill the bytes of `a`,
// the four odd-element ones those of `b`, and one bit-field insert takes the
// low nibbles of `a` and the high nibbles of `b`.  A VALU result written
// through op_sel needs one wait state before another VALU instruction reads
// it: the two chains alternate, so consecutive conversions of one chain are
// one instruction apart, and an s_nop closes the block (another opens it, for
// any partial write just before).  sc is the block's scale as the float
// e8m0_scale_bits gives; y must be finite.
__device__ __forceinline__ uint32_t sr_e2m1_8(const float* y, const U4& r, float sc) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2f p0 = {y[0], y[1]}, p1 = {y[2], y[3]}, p2 = {y[4], y[5]}, p3 = {y[6], y[7]};
  // element 2j's draw at bits 31..16, element 2j + 1's at bits 30..15
  const uint32_t e0 = r.x << 16, e1 = r.y << 16, e2 = r.z << 16, e3 = r.w << 16;
  const uint32_t o0 = (r.x >> 1) & 0x7FFF8000u, o1 = (r.y >> 1) & 0x7FFF8000u;
  const uint32_t o2 = (r.z >> 1) & 0x7FFF8000u, o3 = (r.w >> 1) & 0x7FFF8000u;
  uint32_t a, b;
  asm("" : "=v"(a), "=v"(b));     // any start value: the four conversions of each write all four bytes
  asm("s_nop 0\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %2, %6, %14\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %2, %7, %14\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %3, %8, %14 op_sel:[0,0,1,0]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %3, %9, %14 op_sel:[0,0,1,0]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %4, %10, %14 op_sel:[0,0,0,1]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %4, %11, %14 op_sel:[0,0,0,1]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %5, %12, %14 op_sel:[0,0,1,1]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %5, %13, %14 op_sel:[0,0,1,1]\n\t"
      "s_nop 0"
      : "+v"(a), "+v"(b)
      : "v"(p0), "v"(p1), "v"(p2), "v"(p3), "v"(e0), "v"(o0), "v"(e1), "v"(o1), "v"(e2), "v"(o2), "v"(e3),
        "v"(o3), "v"(sc));
  return (a & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
}

// The operand of one element at index i (see sr_draws).
__device__ __forceinline__ uint32_t sr_draw_one(uint64_t i, uint32_t stream, uint32_t k0, uint32_t k1) {
  const uint64_t g = i >> 3;
  const U4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), stream, 0u, k0, k1);
  const uint32_t j = ((uint32_t)i & 7u) >> 1;
  const uint32_t w = (j & 2u) ? ((j & 1u) ? r.w : r.z) : ((j & 1u) ? r.y : r.x);
  return (i & 1u) ? (w & 0xFFFF0000u) : (w << 16);
}

// ---------------------------------------------------------------------------
// Exact Hadamard sums for the rare chunks where float64 butterflies could
// round (inputs spanning more than 40 binades) or hold non-finite values.
//
// S_i = sum_j sgn(i, j) x_j with x_j bf16.  Each finite x_j is an integer
// significand (<= 8 bits) times 2^(max(E,1) - 134); placed at bit
// max(E,1) - 1 of a fixed-point accumulator whose bit 0 weighs 2^-133, the
// whole bf16 range fits in 9 limbs of 32 bits (signed int64 per limb so that
// 32 terms never overflow before the carry pass).  The result is rounded to
// the nearest fp32, ties to even (values below 2^-126 are exact subnormals).

__device__ __forceinline__ float rn32_from_limbs(int64_t (&acc)[9]) {
  // carry-propagate into canonical 32-bit limbs with a signed top limb
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    const int64_t c = acc[l] >> 32;            // arithmetic shift: floor division
    acc[l] -= c * 4294967296LL;
    acc[l + 1] += c;
  }
  uint32_t u[9];
  const bool neg = acc[8] < 0;
  {
    // magnitude: two's complement negate over the limbs when negative
    uint32_t carry = 1;
#pragma unroll
    for (int l = 0; l < 9; ++l) {
      const uint32_t w = (uint32_t)(acc[l] & 0xFFFFFFFFLL);
      if (neg) {
        const uint64_t s = (uint64_t)(~w) + carry;
        u[l] = (uint32_t)s;
        carry = (uint32_t)(s >> 32);
      } else {
        u[l] = w;
      }
    }
  }
  // most significant set bit
  int msb = -1;
#pragma unroll
  for (int l = 0; l < 9; ++l)
    if (u[l] != 0u) msb = l * 32 + 31 - __clz((int)u[l]);
  const uint32_t sbit = neg ? 0x80000000u : 0u;
  if (msb < 0) return 0.0f;                    // exact zero: +0
  // read a 64-bit window of the magnitude ending at bit msb
  auto bit_window = [&](int lo) -> uint64_t {  // bits [lo, lo+64) (lo may be negative)
    uint64_t r = 0;
#pragma unroll
    for (int l = 0; l < 9; ++l) {
      const int pos = l * 32 - lo;             // where limb l lands in the window
      if (pos >= 64 || pos <= -32) continue;
      const uint64_t w = u[l];
      r |= pos >= 0 ? (w << pos) : (w >> (-pos));
    }
    return r;
  };
  if (msb < 7) {                               // below 2^-126: an exact subnormal
    return __uint_as_float(sbit | (u[0] << 16));
  }
  const int exp_unb = msb - 133;               // floor(log2 |S|)
  if (exp_unb > 127) return __uint_as_float(sbit | 0x7F800000u);
  // 24 kept bits [msb-23, msb], round bit msb-24, sticky below
  const uint64_t win = bit_window(msb - 40);   // bit k of win = bit (msb-40+k)
  uint32_t mant = (uint32_t)(win >> 17) & 0xFFFFFFu;    // bits msb-23..msb
  const uint32_t rbit = (uint32_t)(win >> 16) & 1u;
  bool sticky = (win & 0xFFFFull) != 0;
  // bits below msb-40 also feed the sticky bit
  const int below = msb - 40;
  if (below > 0) {
#pragma unroll
    for (int l = 0; l < 9; ++l) {
      const int lo = l * 32;
      if (lo >= below) continue;
      const int nb = below - lo;               // bits of limb l below the window
      const uint32_t m = nb >= 32 ? 0xFFFFFFFFu : ((1u << nb) - 1u);
      sticky |= (u[l] & m) != 0u;
    }
  }
  int e = exp_unb;
  if (rbit && (sticky || (mant & 1u))) {
    mant += 1u;
    if (mant == 0x1000000u) { mant = 0x800000u; e += 1; }
  }
  if (e > 127) return __uint_as_float(sbit | 0x7F800000u);
  return __uint_as_float(sbit | ((uint32_t)(e + 127) << 23) | (mant & 0x7FFFFFu));
}

// Exact S_i for output i of a chunk of N bf16 values, input j's bit pattern
// given by get(j), with sign vector mask (bit j set: x_j negated).  Sets
// `nonfinite` when an input is Inf or NaN (the sum is then meaningless).
template <int N, typename Get>
__device__ __forceinline__ float exact_hadamard_rn32(Get get, int i, uint32_t mask, bool& nonfinite) {
  int64_t acc[9];
#pragma unroll
  for (int l = 0; l < 9; ++l) acc[l] = 0;
  nonfinite = false;
#pragma unroll 1
  for (int j = 0; j < N; ++j) {
    const uint32_t b = get(j);
    const uint32_t ef = (b >> 7) & 0xFFu;
    nonfinite |= ef == 0xFFu;
    const uint32_t sig = ef ? ((b & 0x7Fu) | 0x80u) : (b & 0x7Fu);
    if (sig == 0u || ef == 0xFFu) continue;
    const int p = (int)(ef ? ef : 1u) - 1;                 // 0 .. 253
    const int L = p >> 5, off = p & 31;
    const uint64_t v = (uint64_t)sig << off;
    const bool neg = (((b >> 15) & 1u) ^ ((mask >> j) & 1u) ^ (__popc((unsigned)(i & j)) & 1u)) != 0u;
    const int64_t lo = (int64_t)(v & 0xFFFFFFFFull), hi = (int64_t)(v >> 32);
#pragma unroll
    for (int l = 0; l < 9; ++l) {
      int64_t add = (l == L) ? lo : ((l == L + 1) ? hi : 0);
      acc[l] += neg ? -add : add;
    }
  }
  return rn32_from_limbs(acc);
}

}  // namespace mx
