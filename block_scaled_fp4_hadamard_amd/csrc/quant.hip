// Fused block-Hadamard + block-absmax + 4-bit cast for gfx950 (MI355X).
//
// A persistent workgroup (256 lanes, 4 waves) walks 32-row x 256-column bf16
// tiles.  Per tile:
//   1. the tile's 16-byte row pieces, loaded into registers while the
//      previous tile was being cast, give a tile-wide max and min-nonzero of
//      |x| (packed 16-bit integer ops); one barrier combines the waves;
//   2. the tile is staged in LDS as bf16 (XOR-swizzled 16-byte pieces: the
//      staging writes, the row-chunk reads and the column reads are all free
//      of bank conflicts), and the next tile's loads are issued;
//   3. row pass (blocks of 32 along a row: the Fprop/Dgrad operand) and
//      column pass (blocks of 32 down a column: the Wgrad operand, written
//      transposed).  When both run on a tile split into two magnitude parts
//      (below), the row pass hands its low parts to the column pass through a
//      third LDS tile, so each element is split once.
//
// The rotation of a 32-element block (deterministic H16/H32 or random-sign
// RHT, "Pre-addestramento ... con MXFP4", Metodologia) is defined as
// y = RN32(RN32(S) * c) with S the exact signed sum.  The hot path computes S
// as a matrix product on the matrix cores: D = A . B with A the 32x32
// sign-Hadamard matrix (rows permuted so that each lane's 16 results are 16
// consecutive outputs of one block) and B = 32 blocks of inputs, one
// v_mfma_f32_32x32x16_bf16 per 16 inputs.  Products of bf16 inputs with +-1
// are exact, and every partial sum of a block is an integer multiple of its
// smallest input's ulp; when the inputs span at most 11 binades every such
// sum fits fp32's 24-bit significand, so the fp32 accumulation is exact.
// Tiles spanning 12..23 binades are split by magnitude into a high part
// (within 11 binades of the tile maximum) and a low part, each product exact,
// and RN32(S_hi + S_lo) = RN32(S) takes one fp32 add.  Tiles spanning 24..35
// binades take a third part; the three exact fp32 sums then add exactly in
// float64 (at most 48 significant bits) before the one rounding to fp32.
// Wider tiles (and tiles with values below 2^-119, whose partial sums could be
// subnormal) take float64 butterflies, exact up to a 40-binade span.  Tiles
// that are wider still, or hold non-finite or near-overflow values, take the
// same butterflies for every block; then each block that on its own is that
// wide or holds such a value is redone exactly by the whole workgroup, one
// output per thread, in fixed point (a few such blocks cost a few
// microseconds, not the tile's whole fixed-point work on 256 lanes).
//
// The E2M1 casts use gfx950's scaled fp4 conversions, which divide by the
// power-of-two scale given as a float and saturate: ties to even for RTNE,
// and for stochastic rounding the add-and-truncate rule on each element's own
// 16-bit Philox draw (eight draws per Philox call).  The uniform grid runs in
// plain VALU code.
//
// Tile order is XCD-aware: workgroup w runs on XCD w % 8, and the 8 row tiles
// of a 256x256 region are all taken by workgroups of one XCD at about the
// same time, so the column-wise output's pieces of one 128-byte line meet in
// that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <algorithm>
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef short ss2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileRows = 32;
constexpr int kTileCols = 256;
constexpr int kThreads = 256;
constexpr int kRowBytes = 2 * kTileCols;           // one tile row of bf16 in LDS
constexpr int kPartBytes = kTileRows * kRowBytes;  // one staged copy of the tile (16 KB)
constexpr int kGroup = 8;                          // row tiles of one region (256 rows)

// fp32 RN32(1/sqrt(32)) = sqrt(2)/8 and 1/sqrt(16)
constexpr float kInvSqrt32 = 0x1.6a09e6p-3f;
constexpr float kInvSqrt16 = 0.25f;

// Resident workgroups per CU in the persistent grid (one wave of each per
// SIMD): four, or three for stochastic rounding, whose Philox draws need the
// larger register budget, and for rotated casts of both axes, which hold a
// third 16 KB LDS tile (the low parts the row pass hands to the column pass).
constexpr int wgs_per_cu(int round, bool share) { return round == MX_ROUND_SR || share ? 3 : 4; }

// tile classes (uniform per tile)
constexpr int kClsMfma1 = 0;     // matrix-core sums, one part (or no rotation)
constexpr int kClsMfma2 = 1;     // matrix-core sums, high + low parts
constexpr int kClsMfma3 = 2;     // matrix-core sums, high + middle + low parts
constexpr int kClsF64 = 3;       // float64 butterflies
constexpr int kClsSpecial = 4;   // float64 butterflies, then an exact redo of the blocks that need it

// LDS byte offset of tile element (r, c): 16-byte piece p = c / 8 of row r is
// stored at piece p ^ s(r, p); s flips piece bit 1 for the right half of a
// row, bit 0 for odd rows and bit 2 for rows 8..15 and 24..31.  Since s
// depends on r only through bits 0 and 3, lds_col(c, r & 9) + r * kRowBytes
// addresses any row r: the passes keep a few such per-lane bases and index
// rows with immediate offsets.
__device__ __forceinline__ uint32_t lds_col(int c, int rbits) {
  const int p = c >> 3;
  const int s = (((p >> 4) & 1) << 1) | (rbits & 1) | (((rbits >> 3) & 1) << 2);
  return (uint32_t)(((p ^ s) << 4) + ((c & 7) << 1));
}
__device__ __forceinline__ uint32_t lds_off(int r, int c) { return (uint32_t)(r * kRowBytes) + lds_col(c, r & 9); }

// Cast one 32-element block y[] of finite values into 4 code dwords; returns
// the scale byte.  For SR, ctr8 is the block's first element index / 8.
template <int GRID, int ROUND>
__device__ __forceinline__ uint32_t cast_block(const float (&y)[32], uint64_t ctr8, uint32_t stream, uint32_t k0,
                                               uint32_t k1, uint32_t (&w)[4]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(y[i]));
  const uint32_t byte = scale_byte<GRID>(__float_as_uint(m) >> 23);
  if constexpr (GRID == MX_GRID_E2M1 && ROUND == MX_ROUND_RTNE) {
    // ties-to-even, saturating: gfx950's scaled conversion, two values a time
    const float sc = __uint_as_float(e8m0_scale_bits(byte));
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t r = __float_as_uint(y[8 * d]);        // any value: the four conversions write all four bytes
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 0], y[8 * d + 1], sc, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 2], y[8 * d + 3], sc, 1);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 4], y[8 * d + 5], sc, 2);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 6], y[8 * d + 7], sc, 3);
      w[d] = r;
    }
  } else if constexpr (GRID == MX_GRID_E2M1) {
    // stochastic rounding on gfx950's conversion, a pair per instruction twice over (sr_e2m1_8)
    const float sc = __uint_as_float(e8m0_scale_bits(byte));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      U4 ph[2];
      philox4x32_10_xn<2>(ctr8 + 2 * hh, stream, k0, k1, ph);
#pragma unroll
      for (int d = 0; d < 2; ++d) w[2 * hh + d] = sr_e2m1_8(&y[16 * hh + 8 * d], ph[d], sc);
    }
  } else {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {                 // 16 outputs (two Philox calls) at a time
      uint32_t u[16] = {};
      if constexpr (ROUND == MX_ROUND_SR) sr_draws<2>(ctr8 + 2 * hh, stream, k0, k1, u);
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        uint32_t r = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) r |= cast_one<GRID, ROUND>(y[16 * hh + 8 * d + q], byte, u[8 * d + q]) << (4 * q);
        w[2 * hh + d] = r;
      }
    }
  }
  return byte;
}

// 16-point Walsh-Hadamard butterflies (natural order) in float64.
__device__ __forceinline__ void fwht16(double (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const double a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Inputs x[0 .. 16) (chunk positions base .. base+16) as float64, with the
// random signs applied: input j of a Hadamard chunk is negated when bit j of
// the mask is set.
template <int HAD>
__device__ __forceinline__ void widen16(const float (&x)[16], int base, uint32_t mask, double (&v)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
    v[j] = (double)__uint_as_float(__float_as_uint(x[j]) ^ (((mask >> ((base + j) % HAD)) & 1u) << 31));
}

// 32 inputs of one block, fetched 16 at a time by load16(h, x) (h = 0, 1),
// rotated in float64 butterflies (one 32-point or two 16-point transforms):
// y = RN32(RN32(S) * c), exact while the inputs span at most 40 binades.
// The second half is fetched only after the first is transformed, so that
// at most 32 float64 values are live besides the first half's results.
// Without rotation (HAD == 0) y = x.
template <int HAD, typename Load>
__device__ __forceinline__ void load_rotate(Load load16, uint32_t mask, float (&y)[32]) {
  if constexpr (HAD == 0) {
    float x0[16], x1[16];
    load16(0, x0);
    load16(1, x1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      y[i] = x0[i];
      y[16 + i] = x1[i];
    }
  } else {
    const float c = HAD == 32 ? kInvSqrt32 : kInvSqrt16;
    double lo[16], hi[16];
    float x[16];
    load16(0, x);
    widen16<HAD>(x, 0, mask, lo);
    fwht16(lo);
    // pin the first half's results here (an empty asm that reads and writes
    // them), so that the compiler cannot sink its work below the second
    // half's loads
    if constexpr (HAD == 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        y[i] = __builtin_fmaf((float)lo[i], c, 0.0f);   // +0 addend: a zero sum gives +0
        asm volatile("" : "+v"(y[i]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(lo[i]));
    }
    asm volatile("" ::: "memory");
    load16(1, x);
    widen16<HAD>(x, 16, mask, hi);
    fwht16(hi);
    if constexpr (HAD == 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[16 + i] = __builtin_fmaf((float)hi[i], c, 0.0f);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const double a = lo[i], b = hi[i];
        y[i] = __builtin_fmaf((float)(a + b), c, 0.0f);
        y[16 + i] = __builtin_fmaf((float)(a - b), c, 0.0f);
      }
    }
  }
}

// Sign-Hadamard MFMA operand A (32 x 32, two K-halves): lane l holds row
// m = l % 32, inputs j = 16h + 8(l / 32) + e.  Row m produces output
// o = 16((m >> 2) & 1) + 4(m >> 3) + (m & 3), which places outputs
// 16(l / 32) .. 16(l / 32) + 15 of every block in lane l's 16 accumulators.
// Entry: (-1)^(popcount(o & j) + sign bit j) within a Hadamard chunk, 0
// across the two chunks of an H16 block.
template <int HAD>
__device__ __forceinline__ void hadamard_operand(uint32_t mask, int lane, bf16x8 (&ha)[2]) {
  const int m = lane & 31;
  const int o = ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 16 * h + 8 * (lane >> 5) + e;
      const uint32_t neg = (__popc((unsigned)(o & j & (HAD - 1))) ^ (mask >> (j & (HAD - 1)))) & 1u;
      const bool zero = HAD == 16 && ((o ^ j) & 16) != 0;
      v[e] = zero ? (unsigned short)0 : (unsigned short)(neg ? 0xBF80u : 0x3F80u);
    }
    ha[h] = __builtin_bit_cast(bf16x8, v);
  }
}

// Low part of two packed bf16 values: those with |x| below the threshold t
// (bf16 magnitude bits, both halves of t2); the high part is w ^ low.
__device__ __forceinline__ uint32_t split_low(uint32_t w, uint32_t t2) {
  const us2 m = __builtin_bit_cast(us2, w & 0x7FFF7FFFu);
  const ss2 d = __builtin_bit_cast(ss2, m - __builtin_bit_cast(us2, t2));
  const ss2 below = d >> (ss2){15, 15};            // 0xFFFF where m < t
  return w & __builtin_bit_cast(uint32_t, below);
}

// Cast one lane's half of a block: y[0..16) are outputs 16(l / 32) .. +15,
// the other half is in lane l ^ 32.  Writes 2 code dwords; returns the scale
// byte.  For SR, ctr8 is the element index of y[0] / 8.
template <int GRID, int ROUND>
__device__ __forceinline__ uint32_t cast_half_block(const float (&y)[16], uint64_t ctr8, uint32_t stream,
                                                    uint32_t k0, uint32_t k1, uint32_t (&w)[2]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(y[i]));
  const uint32_t mb = __float_as_uint(m);
  // one of the swap's two results is the lane's own value and the other its partner's (lane l ^ 32)
  const auto sw = __builtin_amdgcn_permlane32_swap(mb, mb, false, false);
  const uint32_t byte = scale_byte<GRID>(max(sw[0], sw[1]) >> 23);
  if constexpr (GRID == MX_GRID_E2M1 && ROUND == MX_ROUND_RTNE) {
    const float sc = __uint_as_float(e8m0_scale_bits(byte));
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      uint32_t r = __float_as_uint(y[8 * d]);        // any value: the four conversions write all four bytes
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 0], y[8 * d + 1], sc, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 2], y[8 * d + 3], sc, 1);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 4], y[8 * d + 5], sc, 2);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 6], y[8 * d + 7], sc, 3);
      w[d] = r;
    }
  } else if constexpr (GRID == MX_GRID_E2M1) {
    // stochastic rounding on gfx950's conversion, a pair per instruction twice over (sr_e2m1_8)
    const float sc = __uint_as_float(e8m0_scale_bits(byte));
    U4 ph[2];
    philox4x32_10_xn<2>(ctr8, stream, k0, k1, ph);
#pragma unroll
    for (int d = 0; d < 2; ++d) w[d] = sr_e2m1_8(&y[8 * d], ph[d], sc);
  } else {
    uint32_t u[16] = {};
    if constexpr (ROUND == MX_ROUND_SR) sr_draws<2>(ctr8, stream, k0, k1, u);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      uint32_t r = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) r |= cast_one<GRID, ROUND>(y[8 * d + q], byte, u[8 * d + q]) << (4 * q);
      w[d] = r;
    }
  }
  return byte;
}

// Row sums of 32 blocks on the matrix cores: part[p][h] holds the lane's
// inputs 16h + 8(l / 32) .. +7 of block l % 32, split into PARTS magnitude
// parts (high first).  Each part's sum is exact in fp32; two exact parts add
// with one fp32 rounding, three add exactly in float64 first.
template <int PARTS>
__device__ __forceinline__ void mfma_block_sums(const bf16x8 (&ha)[2], const uint4 (&part)[3][2], float c,
                                                float (&y)[16]) {
  f32x16 acc[PARTS];
#pragma unroll
  for (int q = 0; q < PARTS; ++q) acc[q] = f32x16{};
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int q = 0; q < PARTS; ++q)
      acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha[h], __builtin_bit_cast(bf16x8, part[q][h]), acc[q], 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float s;
    if constexpr (PARTS == 1) s = acc[0][r];
    else if constexpr (PARTS == 2) s = acc[0][r] + acc[1][r];                 // RN32(S)
    else s = (float)((double)acc[0][r] + (double)acc[1][r] + (double)acc[2][r]);   // exact sum, then RN32
    y[r] = __builtin_fmaf(s, c, 0.0f);               // +0 addend: a zero sum gives +0
  }
}

// Split packed bf16 pairs into up to three magnitude parts: below t2 goes
// down a part, and of that, below t3 down another (both halves of each
// threshold hold the same bf16 magnitude bits).
template <int PARTS>
__device__ __forceinline__ void split_parts(const uint4& v, uint32_t t2, uint32_t t3, uint4 (&part)[3]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[3][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (PARTS == 1) {
      o[0][i] = w[i];
    } else {
      const uint32_t low = split_low(w[i], t2);
      o[0][i] = w[i] ^ low;
      if constexpr (PARTS == 2) {
        o[1][i] = low;
      } else {
        const uint32_t lowest = split_low(low, t3);
        o[1][i] = low ^ lowest;
        o[2][i] = lowest;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < PARTS; ++q) part[q] = uint4{o[q][0], o[q][1], o[q][2], o[q][3]};
}

// Element i of a block after the rotation, computed exactly from the bf16
// inputs get(j): y = RN32(RN32(S) * c), NaN when its Hadamard chunk holds a
// non-finite input.  Without rotation, y = x.
template <int HAD, typename Get>
__device__ __forceinline__ float special_value(Get get, int i, uint32_t mask) {
  if constexpr (HAD == 0) {
    return __uint_as_float(get(i) << 16);
  } else {
    const int base = i & ~(HAD - 1);
    bool nonfinite;
    const float s = exact_hadamard_rn32<HAD>([&](int j) { return get(base + j); }, i & (HAD - 1), mask, nonfinite);
    const float c = HAD == 32 ? kInvSqrt32 : kInvSqrt16;
    return nonfinite ? __uint_as_float(0x7FC00000u) : __builtin_fmaf(s, c, 0.0f);
  }
}

// Whether the block of 32 bf16 inputs get(j) must be redone exactly after the
// float64 butterflies: with rotation, when an input is Inf or NaN or has
// |x| >= 2^123 (the fp32 sum could overflow), or when the largest and the
// smallest nonzero |x| lie more than 40 binades apart (subnormals counted as
// exponent field 1); without rotation, when an input is Inf or NaN.
template <int HAD, typename Get>
__device__ __forceinline__ bool block_needs_exact(Get get) {
  uint32_t mx = 0, mn = 0xFFFFu;
#pragma unroll 8
  for (int j = 0; j < 32; ++j) {
    const uint32_t m = get(j) & 0x7FFFu;
    mx = max(mx, m);
    if (m != 0u) mn = min(mn, m);
  }
  if constexpr (HAD == 0) {
    return mx >= 0x7F80u;
  } else {
    if (mx >= (250u << 7)) return true;
    if (mn == 0xFFFFu) return false;
    return max((int)(mx >> 7), 1) - max((int)(mn >> 7), 1) > 40;
  }
}

// Exact redo of the n blocks listed in fix[]: entry = axis << 15 | owner,
// owner being the lane that holds the block in the float64 passes (row pass:
// 8 r + k for chunk k of tile row r; column pass: the tile column).  In round
// c, thread t computes output t % 32 of entry c + t / 32 in fixed point, so a
// block's 32 outputs meet in one half wave: the block maximum and the code
// words are gathered there.  A block with a non-finite output gets scale 0xFF
// and zero codes.  n is the same in every thread.
template <int HAD, int GRID, int ROUND>
__device__ __forceinline__ void exact_fixup(const QuantParams& p, const uint8_t* buf, int t, int64_t row0,
                                            int64_t col0, uint32_t mask, const uint16_t* fix, int n) {
  const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
  const int i = t & 31;
#pragma unroll 1
  for (int c = 0; c < n; c += kThreads / 32) {
    const int e = c + (t >> 5);
    const bool active = e < n;
    const uint32_t ent = active ? (uint32_t)fix[e] : 0u;
    const bool col_axis = (ent >> 15) != 0u;
    const int owner = (int)(ent & 0x7FFFu);
    float y;
    uint64_t first;                                  // element index of the block's output 0
    uint8_t* codes;
    uint8_t* scale;
    if (col_axis) {
      y = special_value<HAD>([&](int j) { return (uint32_t)*(const uint16_t*)(buf + lds_off(j, owner)); }, i, mask);
      const int64_t col = col0 + owner;
      first = (uint64_t)col * (uint64_t)p.rows + (uint64_t)row0;
      codes = p.col_codes + col * p.ld_col_codes + row0 / 2;
      scale = p.col_scales + col * p.ld_col_scales + row0 / 32;
    } else {
      const int r = owner >> 3, k = owner & 7;
      y = special_value<HAD>([&](int j) { return (uint32_t)*(const uint16_t*)(buf + lds_off(r, 32 * k + j)); }, i,
                             mask);
      const int64_t row = row0 + r, c0 = col0 + 32 * k;
      first = (uint64_t)row * (uint64_t)p.cols + (uint64_t)c0;
      codes = p.row_codes + row * p.ld_row_codes + c0 / 2;
      scale = p.row_scales + row * p.ld_row_scales + c0 / 32;
    }
    uint32_t mb = __float_as_uint(y) & 0x7FFFFFFFu;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, o));
    const bool nonfinite = mb >= 0x7F800000u;
    const uint32_t byte = nonfinite ? 0xFFu : scale_byte<GRID>(mb >> 23);
    uint32_t u = 0;
    if constexpr (ROUND == MX_ROUND_SR) u = sr_draw_one(first + (uint64_t)i, col_axis ? 1u : 0u, k0, k1);
    uint32_t word = nonfinite ? 0u : cast_one<GRID, ROUND>(y, byte, u) << (4 * (i & 7));
    word |= (uint32_t)__shfl_xor((int)word, 1);
    word |= (uint32_t)__shfl_xor((int)word, 2);
    word |= (uint32_t)__shfl_xor((int)word, 4);
    if (active) {
      if ((i & 7) == 0) *(uint32_t*)(codes + 4 * (i >> 3)) = word;
      if (i == 0) *scale = (uint8_t)byte;
    }
  }
}

// Tile walk: workgroup (xcd, j) of J per XCD takes the XCD's tile sequence
// tau = j, j + J, ...; tau / 8 is the XCD's region count, tau % 8 the row tile
// inside the region.  Moves tau to the next tile that exists; false at the end.
__device__ __forceinline__ bool next_tile(const QuantParams& p, uint32_t xcd, uint32_t J, uint32_t& tau,
                                          int64_t& row0, int64_t& col0) {
  const uint32_t n_regions = (uint32_t)p.n_col_tiles * (uint32_t)p.n_row_groups;
  for (;; tau += J) {
    const uint32_t region = (tau >> 3) * 8u + xcd;
    if (region >= n_regions) return false;
    const uint32_t col_tile = region / (uint32_t)p.n_row_groups;
    const uint32_t row_tile = (region % (uint32_t)p.n_row_groups) * kGroup + (tau & 7u);
    if (row_tile < (uint32_t)p.n_row_tiles) {
      row0 = (int64_t)row_tile * kTileRows;
      col0 = (int64_t)col_tile * kTileCols;
      return true;
    }
  }
}

// s_waitcnt immediate for vmcnt(0) (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] << 14); the other counters left unconstrained
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// global -> LDS copy of 16 bytes per lane (gfx950 LDS DMA): lane l's bytes
// land at LDS address m0 + 16 l.  The s_nop covers the M0 write hazard.  The
// input is read once, so the copy is non-temporal.  The outputs are plain
// stores: the GEMMs that consume them often run next and then find them in
// the last-level cache (streaming the row-wise outputs past it saved a few
// percent here but cost the step more), and the column-wise outputs' 16-byte
// pieces of a line must meet in L2 (streaming them made the kernel 1.6x
// slower).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// an output pointer that is the same in every lane, moved to SGPRs
__device__ __forceinline__ uint8_t* uniform_ptr(uint8_t* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (uint8_t*)(((uint64_t)hi << 32) | lo);
}

// a pointer that is the same in every lane, moved to SGPRs
__device__ __forceinline__ const uint16_t* wave_uniform(const uint16_t* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint16_t*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Start copying a tile into an LDS buffer.  Wave w fills rows 8w .. 8w+7, two
// rows (1 KB) per instruction: lane l writes stored piece l % 32 of row
// 8w + 2i + l / 32, so it loads the global piece that the swizzle puts there.
// That piece depends on the row only through r & 1 = l / 32 and (r >> 3) & 1
// = w & 1, so it is the same for the four copies, whose offsets then step by
// two rows.  Pieces outside the tensor are written as zeros instead; a tile
// wholly inside takes no per-lane test.
__device__ __forceinline__ void issue_tile(const QuantParams& p, int64_t row0, int64_t col0, int wave, int lane,
                                           uint8_t* buf) {
  const uint16_t* base = wave_uniform(p.x + row0 * p.ld_x + col0);
  const int ps = lane & 31, hr = lane >> 5;
  const int pg = ps ^ ((((ps >> 4) & 1) << 1) | hr | ((wave & 1) << 2));
  const uint32_t off0 = (uint32_t)(((8 * wave + hr) * p.ld_x + 8 * pg) * 2);
  const uint32_t step = (uint32_t)(4 * p.ld_x);                 // two rows of bf16, in bytes
  const bool interior = row0 + kTileRows <= p.rows && col0 + kTileCols <= p.cols;
  if (interior) {
    // straight-line: the wave's LDS rows from one scalar base, no per-copy tests
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(buf + 8 * wave * kRowBytes));
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(base, off0 + (uint32_t)i * step, lbase + (uint32_t)(2 * i * kRowBytes));
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * wave + 2 * i + hr;
    if (row0 + r < p.rows && col0 + 8 * pg < p.cols)
      dma16(base, off0 + (uint32_t)i * step, lds_addr(buf + (8 * wave + 2 * i) * kRowBytes));
    else
      *(uint4*)(buf + r * kRowBytes + ps * 16) = uint4{0u, 0u, 0u, 0u};
  }
}


// DPP lane exchanges within rows of 16 lanes: l ^ 1, l ^ 2 (quad permutes),
// and 7 - l within each group of 8 (half-row mirror)
__device__ __forceinline__ uint32_t dpp_x1(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_x2(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_hm(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_m(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false); }

// Packed 16-bit maxima over the whole wave (every lane active): each row of
// 16 lanes by quad, half-row and row mirror exchanges; then rows 1 and 3 take
// the last lane of rows 0 and 2 (row_bcast:15), and rows 2 and 3 take lane 31
// (row_bcast:31), so that lane 63 holds the maxima of all 64 lanes.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b)));
}
__device__ __forceinline__ uint32_t wave_pk_max_u16(uint32_t v) {
  v = pk_max_u16(v, dpp_x1(v));
  v = pk_max_u16(v, dpp_x2(v));
  v = pk_max_u16(v, dpp_hm(v));
  v = pk_max_u16(v, dpp_m(v));
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Scale bytes of 8 consecutive blocks of a row, held by lanes 8a .. 8a+7
// (k = lane % 8): with 8-byte aligned scale rows and all 8 blocks inside the
// tensor, the lane with k == 0 writes all 8 at once.  All lanes of the wave
// must call this (the gather is a cross-lane exchange: after the two quad
// steps every lane holds its quad's four bytes, and the half-row mirror
// brings the other quad's).
__device__ __forceinline__ void store_row_scales(uint8_t* dst, int k, uint32_t byte, bool wide, bool active) {
  uint32_t v = byte << (8 * (k & 3));
  v |= dpp_x1(v);
  v |= dpp_x2(v);
  const uint32_t hi = dpp_hm(v);
  if (!active) return;
  if (wide) {
    typedef unsigned int u2v __attribute__((ext_vector_type(2)));
    if (k == 0) *(__attribute__((address_space(1))) u2v*)dst = u2v{v, hi};
  } else {
    ((__attribute__((address_space(1))) uint8_t*)dst)[k] = (uint8_t)byte;
  }
}

// Passes in which each lane reads a whole block: no rotation or float64
// butterflies.  Row pass: lane (r, k) owns chunk k of row r; column pass:
// lane c owns column c.  In a kClsSpecial tile the blocks that the
// butterflies may get wrong are then listed in fix[] (count *fix_n, zero on
// entry and on return) and redone exactly.
template <int HAD, int GRID, int ROUND, bool DO_ROW, bool DO_COL>
__device__ __forceinline__ void lane_block_passes(const QuantParams& p, const uint8_t* hi_part, int t, int64_t row0,
                                                  int64_t col0, int cls, uint32_t mask, bool wide_scales,
                                                  uint16_t* fix, uint32_t* fix_n) {
  const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
  const bool full_width = col0 + kTileCols <= p.cols;
  {
    if constexpr (DO_ROW) {
      const int r = t >> 3, k = t & 7;
      const int64_t row = row0 + r, c0 = col0 + 32 * k;
      float y[32];
      load_rotate<HAD>(
          [&](int h, float (&x)[16]) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const uint4 v = *(const uint4*)(hi_part + lds_off(r, 32 * k + 16 * h + 8 * q));
              const uint32_t dw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                x[8 * q + 2 * e] = __uint_as_float(dw[e] << 16);
                x[8 * q + 2 * e + 1] = __uint_as_float(dw[e] & 0xFFFF0000u);
              }
            }
          },
          mask, y);
      uint32_t w[4];
      const uint32_t byte =
          cast_block<GRID, ROUND>(y, ((uint64_t)row * (uint64_t)p.cols + (uint64_t)c0) >> 3, 0u, k0, k1, w);
      const bool valid = row < p.rows && c0 < p.cols;
      if (valid) *(uint4*)(p.row_codes + row * p.ld_row_codes + c0 / 2) = uint4{w[0], w[1], w[2], w[3]};
      store_row_scales(p.row_scales + row * p.ld_row_scales + col0 / 32, k, byte, wide_scales && full_width, valid);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DO_COL) {
      const int64_t col = col0 + t;
      float y[32];
      load_rotate<HAD>(
          [&](int h, float (&x)[16]) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int j = 16 * h + i;
              const uint32_t off = j * kRowBytes + lds_col(t, j & 9);
              x[i] = __uint_as_float((uint32_t)*(const uint16_t*)(hi_part + off) << 16);
            }
          },
          mask, y);
      uint32_t w[4];
      const uint32_t byte =
          cast_block<GRID, ROUND>(y, ((uint64_t)col * (uint64_t)p.rows + (uint64_t)row0) >> 3, 1u, k0, k1, w);
      if (col < p.cols) {
        *(uint4*)(p.col_codes + col * p.ld_col_codes + row0 / 2) = uint4{w[0], w[1], w[2], w[3]};
        p.col_scales[col * p.ld_col_scales + row0 / 32] = (uint8_t)byte;
      }
    }
  }
  if (cls != kClsSpecial) return;
  // ---- list the blocks to redo, then redo them (all threads: the count and
  // the barriers are workgroup-uniform)
  if constexpr (DO_ROW) {
    const int r = t >> 3, k = t & 7;
    if (row0 + r < p.rows && col0 + 32 * k < p.cols &&
        block_needs_exact<HAD>([&](int j) { return (uint32_t)*(const uint16_t*)(hi_part + lds_off(r, 32 * k + j)); }))
      fix[atomicAdd(fix_n, 1u)] = (uint16_t)t;
  }
  if constexpr (DO_COL) {
    if (col0 + t < p.cols &&
        block_needs_exact<HAD>([&](int j) { return (uint32_t)*(const uint16_t*)(hi_part + lds_off(j, t)); }))
      fix[atomicAdd(fix_n, 1u)] = (uint16_t)(0x8000 | t);
  }
  // the butterflies' stores of these blocks are complete before they are
  // overwritten, and the list is whole
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int n = (int)*(volatile uint32_t*)fix_n;
  __syncthreads();
  if (t == 0) *fix_n = 0u;
  if (n > 0) exact_fixup<HAD, GRID, ROUND>(p, hi_part, t, row0, col0, mask, fix, n);
}

// Row and column passes of a tile on the matrix cores, with the inputs split
// into PARTS magnitude parts (thresholds t2, t3).  Two-part tiles cast on both
// axes split each element once: the row pass reads every 16-byte piece of the
// tile exactly once, and it writes the piece's low parts to lowbuf at the same
// offset; after a barrier the column pass reads them with the same transposed
// reads as the inputs, and the high part is x ^ low.
//   row pass: wave w, group g = the 32 blocks of rows 8w + 4g .. +3;
//   column pass: wave w, group g = columns 64w + 32g .. +31.  A lane's
//   operand (8 consecutive rows of its column) comes from two transposed LDS
//   reads: in each 16-lane group, lane s reads 4 consecutive columns of row
//   s / 4, and lane j receives column j of the 4 rows (ds_read_b64_tr_b16).
// FAST: a tile wholly inside the tensor, 8-byte aligned row-scale rows, and
// output pitches small enough for 32-bit offsets from the tile's first line
// (QuantParams::fast_ok).  Its stores then take a wave-uniform tile base plus a
// per-lane 32-bit offset and need no bounds tests.
template <int HAD, int GRID, int ROUND, bool DO_ROW, bool DO_COL, int PARTS, bool FAST>
__device__ __forceinline__ void mfma_passes(const QuantParams& p, const uint8_t* buf, uint8_t* lowbuf, int t,
                                            int64_t row0, int64_t col0, const uint4* htab, uint32_t t2, uint32_t t3,
                                            bool wide_scales) {
  constexpr bool kShare = PARTS == 2 && DO_ROW && DO_COL;
  const int lane = t & 63, wave = t >> 6, hl = lane >> 5, n = lane & 31;
  const bf16x8 ha[2] = {__builtin_bit_cast(bf16x8, htab[2 * lane]), __builtin_bit_cast(bf16x8, htab[2 * lane + 1])};
  const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
  const float c = HAD == 32 ? kInvSqrt32 : kInvSqrt16;
  if constexpr (DO_ROW) {
    const bool full_width = col0 + kTileCols <= p.cols;
    const bool interior = full_width && row0 + kTileRows <= p.rows;
    // the lane's output addresses for group 0; group g is 4g rows further
    const int64_t rl = row0 + 8 * wave + (n >> 3);
    uint8_t* const cbase = p.row_codes + rl * p.ld_row_codes + col0 / 2 + 16 * (n & 7) + 8 * hl;
    uint8_t* const sbase = p.row_scales + rl * p.ld_row_scales + col0 / 32;
    // FAST: the same addresses as a uniform tile base and a 32-bit lane offset
    uint8_t* const cbase_u = uniform_ptr(p.row_codes + row0 * p.ld_row_codes + col0 / 2);
    uint8_t* const sbase_u = uniform_ptr(p.row_scales + row0 * p.ld_row_scales + col0 / 32);
    const uint32_t coff = (uint32_t)(8 * wave + (n >> 3)) * (uint32_t)p.ld_row_codes + 16 * (n & 7) + 8 * hl;
    const uint32_t soff = (uint32_t)(8 * wave + (n >> 3)) * (uint32_t)p.ld_row_scales;
    const uint64_t ctr0 = (((uint64_t)rl * (uint64_t)p.cols + (uint64_t)(col0 + 32 * (n & 7))) >> 3) + 2 * hl;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int r = 8 * wave + 4 * g + (n >> 3), k = n & 7;
      uint4 part[3][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t off = (uint32_t)(r * kRowBytes) +
                             lds_col(32 * k + 16 * h + 8 * hl, ((n >> 3) & 1) | ((wave & 1) << 3));
        const uint4 v = *(const uint4*)(buf + off);
        uint4 ph[3];
        split_parts<PARTS>(v, t2, t3, ph);
        if constexpr (kShare) *(uint4*)(lowbuf + off) = ph[1];
#pragma unroll
        for (int q = 0; q < PARTS; ++q) part[q][h] = ph[q];
      }
      float y[16];
      mfma_block_sums<PARTS>(ha, part, c, y);
      uint32_t w[2];
      // counter of the lane's first output: (row * cols + c0) / 8 + 2 hl; group g is 4 rows further, and
      // cols % 8 == 0
      const uint32_t byte =
          cast_half_block<GRID, ROUND>(y, ctr0 + (uint64_t)g * (uint64_t)(p.cols >> 1), 0u, k0, k1, w);
      typedef unsigned int u2v __attribute__((ext_vector_type(2)));
      if constexpr (FAST) {
        *(__attribute__((address_space(1))) u2v*)(cbase_u + (uint64_t)(coff + (uint32_t)(4 * g) * (uint32_t)p.ld_row_codes)) =
            u2v{w[0], w[1]};
        store_row_scales(sbase_u + (uint64_t)(soff + (uint32_t)(4 * g) * (uint32_t)p.ld_row_scales), k, byte, true,
                         hl == 0);
      } else {
        const int64_t row = row0 + r, c0 = col0 + 32 * k;
        const bool valid = interior || (row < p.rows && c0 < p.cols);
        if (valid) *(u2v*)(cbase + 4 * g * p.ld_row_codes) = u2v{w[0], w[1]};
        store_row_scales(sbase + 4 * g * p.ld_row_scales, k, byte, wide_scales && full_width, valid && hl == 0);
      }
    }
  }
  if constexpr (kShare) {
    // every wave's low parts are in LDS before any column pass reads them (the
    // clobber keeps the compiler's LDS accesses on their side of the barrier)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if constexpr (DO_COL) {
    const int g16 = lane >> 4, s = lane & 15;
    // the lane's output column in group 0 and its addresses; group g is 32 columns further
    const int64_t cl = col0 + 64 * wave + n;
    uint8_t* const ccbase = p.col_codes + cl * p.ld_col_codes + row0 / 2 + 8 * hl;
    uint8_t* const csbase = p.col_scales + cl * p.ld_col_scales + row0 / 32;
    uint8_t* const ccbase_u = uniform_ptr(p.col_codes + col0 * p.ld_col_codes + row0 / 2);
    uint8_t* const csbase_u = uniform_ptr(p.col_scales + col0 * p.ld_col_scales + row0 / 32);
    const uint32_t ccoff = (uint32_t)(64 * wave + n) * (uint32_t)p.ld_col_codes + 8 * hl;
    const uint32_t csoff = (uint32_t)(64 * wave + n) * (uint32_t)p.ld_col_scales;
    const uint64_t cctr0 = (((uint64_t)cl * (uint64_t)p.rows + (uint64_t)row0) >> 3) + 2 * hl;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int col = 64 * wave + 32 * g + 16 * (g16 & 1) + 4 * (s & 3);    // this lane's source columns
      uint4 part[3][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t d[4], lo[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int row = 16 * h + 8 * (g16 >> 1) + 4 * half + (s >> 2);
          const uint32_t off = (uint32_t)(row * kRowBytes) + lds_col(col, row & 9);
          typedef short v4s __attribute__((ext_vector_type(4)));
          typedef __attribute__((address_space(3))) v4s* lds_v4s;
          const v4s q = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4s)((__attribute__((address_space(3))) uint8_t*)(uint8_t*)buf + off));
          d[2 * half] = (uint32_t)(uint16_t)q[0] | ((uint32_t)(uint16_t)q[1] << 16);
          d[2 * half + 1] = (uint32_t)(uint16_t)q[2] | ((uint32_t)(uint16_t)q[3] << 16);
          if constexpr (kShare) {
            const v4s ql = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s)((__attribute__((address_space(3))) uint8_t*)lowbuf + off));
            lo[2 * half] = (uint32_t)(uint16_t)ql[0] | ((uint32_t)(uint16_t)ql[1] << 16);
            lo[2 * half + 1] = (uint32_t)(uint16_t)ql[2] | ((uint32_t)(uint16_t)ql[3] << 16);
          }
        }
        if constexpr (kShare) {
          part[0][h] = uint4{d[0] ^ lo[0], d[1] ^ lo[1], d[2] ^ lo[2], d[3] ^ lo[3]};
          part[1][h] = uint4{lo[0], lo[1], lo[2], lo[3]};
        } else {
          uint4 ph[3];
          split_parts<PARTS>(uint4{d[0], d[1], d[2], d[3]}, t2, t3, ph);
#pragma unroll
          for (int q = 0; q < PARTS; ++q) part[q][h] = ph[q];
        }
      }
      float y[16];
      mfma_block_sums<PARTS>(ha, part, c, y);
      const int64_t cc = cl + 32 * g;
      uint32_t w[2];
      // counter: (cc * rows + row0) / 8 + 2 hl with cc 32 g columns further, and rows % 32 == 0 here
      const uint32_t byte = cast_half_block<GRID, ROUND>(y, cctr0 + (uint64_t)(4 * g) * (uint64_t)p.rows, 1u, k0,
                                                         k1, w);
      if constexpr (FAST) {
        typedef unsigned int u2c __attribute__((ext_vector_type(2)));
        *(__attribute__((address_space(1))) u2c*)(ccbase_u + (uint64_t)(ccoff + (uint32_t)(32 * g) * (uint32_t)p.ld_col_codes)) =
            u2c{w[0], w[1]};
        if (hl == 0)
          *(__attribute__((address_space(1))) uint8_t*)(csbase_u + (uint64_t)(csoff + (uint32_t)(32 * g) *
                                                                                   (uint32_t)p.ld_col_scales)) = (uint8_t)byte;
      } else if (cc < p.cols) {
        *(uint2*)(ccbase + 32 * g * p.ld_col_codes) = uint2{w[0], w[1]};
        if (hl == 0) csbase[32 * g * p.ld_col_scales] = (uint8_t)byte;
      }
    }
  }
}

template <int HAD, int GRID, int ROUND, bool DO_ROW, bool DO_COL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(wgs_per_cu(ROUND, HAD > 0 && DO_ROW && DO_COL))))
quant_kernel(const QuantParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kPartBytes];   // two tile buffers
  // the low parts of a two-part tile, handed from the row pass to the column pass
  __shared__ __attribute__((aligned(16))) uint8_t lowbuf[HAD > 0 && DO_ROW && DO_COL ? kPartBytes : 16];
  __shared__ uint32_t red[kThreads / 64];
  __shared__ uint4 htab[2 * 64];       // the sign-Hadamard MFMA operand of each lane (two K-halves)
  __shared__ uint16_t fix[2 * kThreads];   // blocks of a kClsSpecial tile to redo exactly
  __shared__ uint32_t fix_n;

  const int tid = threadIdx.x;
  const uint32_t xcd = blockIdx.x & 7u, J = gridDim.x >> 3;
  uint32_t tau = blockIdx.x >> 3;
  int64_t row0 = 0, col0 = 0;
  if (!next_tile(p, xcd, J, tau, row0, col0)) return;
  issue_tile(p, row0, col0, tid >> 6, tid & 63, lds);
  const bool wide_scales = DO_ROW && ((((uintptr_t)p.row_scales) | (uintptr_t)p.ld_row_scales) & 7u) == 0;
  if constexpr (HAD > 0) {
    if (tid < 64) {                    // read after the first barrier below
      bf16x8 ha[2];
      hadamard_operand<HAD>(p.sign_mask, tid, ha);
      htab[2 * tid] = __builtin_bit_cast(uint4, ha[0]);
      htab[2 * tid + 1] = __builtin_bit_cast(uint4, ha[1]);
    }
  }
  if (tid == 0) fix_n = 0u;            // read after the first barrier below
  int cur = 0;

  for (;;) {
    // Lane ids and the sign mask pass through an empty asm each tile, so that
    // the many addresses and sign constants derived from them are computed
    // where they are used instead of being held in registers across the loop.
    int t = tid;
    uint32_t mask = p.sign_mask;
    asm volatile("" : "+v"(t), "+v"(mask));
    const int lane = t & 63, wave = t >> 6;
    uint8_t* buf = lds + cur * kPartBytes;

    // ---- 1. this tile has landed in LDS (every wave's copies), and every wave
    // is done with the other buffer: start the next tile's copy into it
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    uint32_t tau_next = tau + J;
    int64_t nrow0 = 0, ncol0 = 0;
    const bool more = next_tile(p, xcd, J, tau_next, nrow0, ncol0);
    if (more) issue_tile(p, nrow0, ncol0, wave, lane, lds + (cur ^ 1) * kPartBytes);

    // ---- 2. packed 16-bit max / min-nonzero of |x| over the tile (any 16-byte
    // pieces will do: lane t reads pieces t, t + 256, ...)
    us2 mx2 = {0, 0}, mn2 = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = *(const uint4*)(buf + 16 * (t + kThreads * i));
      const uint32_t dw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const us2 m = __builtin_bit_cast(us2, dw[k] & 0x7FFF7FFFu);
        mx2 = __builtin_elementwise_max(mx2, m);
        mn2 = __builtin_elementwise_min(mn2, m - (us2){1, 1});  // zero wraps to 0xFFFF: ignored
      }
    }
    // both reductions in one: max |x| in the high half, 0xFFFF - (min nonzero |x| - 1) in the low
    const uint32_t lmx = max((uint32_t)mx2.x, (uint32_t)mx2.y), lmn = min((uint32_t)mn2.x, (uint32_t)mn2.y);
    const uint32_t both = wave_pk_max_u16((lmx << 16) | (0xFFFFu - lmn));
    if (lane == 0) red[wave] = both;
    // the wait and the barrier in one asm statement whose memory clobber keeps red[] accesses on their
    // side of it (the barrier builtin alone is not a memory operation)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const uint32_t all = pk_max_u16(pk_max_u16(red[0], red[1]), pk_max_u16(red[2], red[3]));
    const uint32_t mx = all >> 16, mn = 0xFFFFu - (all & 0xFFFFu);

    // ---- 3. classify by the exponent fields of the largest and smallest nonzero |x|
    int cls = kClsMfma1;
    uint32_t t2 = 0, t3 = 0;                        // split thresholds (both halves)
    if (mx >= (250u << 7)) {
      cls = kClsSpecial;                            // Inf/NaN or sums that could overflow
    } else if (HAD > 0 && mn != 0xFFFFu) {
      const int fmax = max((int)(mx >> 7), 1);
      const int fmin = max((int)((mn + 1u) >> 7), 1);
      const int span = fmax - fmin;
      if (span > 40) cls = kClsSpecial;
      else if (fmin < 8 || span > 35) cls = kClsF64;
      else if (span > 11) {
        cls = span > 23 ? kClsMfma3 : kClsMfma2;
        t2 = (uint32_t)(fmax - 11) << 7;
        t2 |= t2 << 16;
        t3 = (uint32_t)(fmax - 23) << 7;
        t3 |= t3 << 16;
      }
    }

    if (HAD > 0 && cls <= kClsMfma3) {
      if constexpr (HAD > 0) {
        const bool fast = p.fast_ok && (!DO_ROW || wide_scales) && row0 + kTileRows <= p.rows &&
                          col0 + kTileCols <= p.cols;
        if (fast) {
          if (cls == kClsMfma1) mfma_passes<HAD, GRID, ROUND, DO_ROW, DO_COL, 1, true>(p, buf, lowbuf, t, row0, col0, htab, t2, t3, true);
          else if (cls == kClsMfma2) mfma_passes<HAD, GRID, ROUND, DO_ROW, DO_COL, 2, true>(p, buf, lowbuf, t, row0, col0, htab, t2, t3, true);
          else mfma_passes<HAD, GRID, ROUND, DO_ROW, DO_COL, 3, true>(p, buf, lowbuf, t, row0, col0, htab, t2, t3, true);
        } else {
          if (cls == kClsMfma1) mfma_passes<HAD, GRID, ROUND, DO_ROW, DO_COL, 1, false>(p, buf, lowbuf, t, row0, col0, htab, t2, t3, wide_scales);
          else if (cls == kClsMfma2) mfma_passes<HAD, GRID, ROUND, DO_ROW, DO_COL, 2, false>(p, buf, lowbuf, t, row0, col0, htab, t2, t3, wide_scales);
          else mfma_passes<HAD, GRID, ROUND, DO_ROW, DO_COL, 3, false>(p, buf, lowbuf, t, row0, col0, htab, t2, t3, wide_scales);
        }
      }
    } else {
      // ---- 4c. no rotation, float64 butterflies or exact fixed point: each
      // lane casts whole blocks
      lane_block_passes<HAD, GRID, ROUND, DO_ROW, DO_COL>(p, buf, t, row0, col0, cls, mask, wide_scales, fix, &fix_n);
    }
    if (!more) break;
    tau = tau_next;
    row0 = nrow0;
    col0 = ncol0;
    cur ^= 1;
  }
}

// ---- host-side launch: pick the instantiation
template <int HAD, int GRID, int ROUND>
static hipError_t launch_axes(const QuantParams& p, bool do_row, bool do_col, dim3 grid, hipStream_t s) {
  if (do_row && do_col)
    hipLaunchKernelGGL((quant_kernel<HAD, GRID, ROUND, true, true>), grid, dim3(kThreads), 0, s, p);
  else if (do_row)
    hipLaunchKernelGGL((quant_kernel<HAD, GRID, ROUND, true, false>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((quant_kernel<HAD, GRID, ROUND, false, true>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int HAD>
static hipError_t launch_cast(const QuantParams& p, int grid_kind, int round, bool r, bool c, dim3 g, hipStream_t s) {
  if (grid_kind == MX_GRID_E2M1) {
    return round == MX_ROUND_RTNE ? launch_axes<HAD, MX_GRID_E2M1, MX_ROUND_RTNE>(p, r, c, g, s)
                                  : launch_axes<HAD, MX_GRID_E2M1, MX_ROUND_SR>(p, r, c, g, s);
  }
  return round == MX_ROUND_RTNE ? launch_axes<HAD, MX_GRID_E1M2, MX_ROUND_RTNE>(p, r, c, g, s)
                                : launch_axes<HAD, MX_GRID_E1M2, MX_ROUND_SR>(p, r, c, g, s);
}

hipError_t launch_quant(QuantParams p, int had_n, bool rht, int grid_kind, int round, bool do_row, bool do_col,
                        hipStream_t s) {
  p.n_row_tiles = (int32_t)((p.rows + kTileRows - 1) / kTileRows);
  p.n_col_tiles = (int32_t)((p.cols + kTileCols - 1) / kTileCols);
  p.n_row_groups = (p.n_row_tiles + kGroup - 1) / kGroup;
  // a tile's output lines lie within 32-bit offsets of its first line: up to 32 row-wise lines and 256
  // column-wise lines of the given pitches
  p.fast_ok = (!do_row || (p.ld_row_codes < (int64_t(1) << 26) && p.ld_row_scales < (int64_t(1) << 26))) &&
              (!do_col || (p.ld_col_codes < (int64_t(1) << 23) && p.ld_col_scales < (int64_t(1) << 23)));
  const int64_t regions = (int64_t)p.n_col_tiles * p.n_row_groups;
  // tiles each XCD walks: its regions (every 8th) x 8 row tiles
  const int64_t per_xcd = ((regions + 7) / 8) * kGroup;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int64_t wgs_per_xcd = std::max<int64_t>(1, (int64_t)cus * wgs_per_cu(round, had_n > 0 && do_row && do_col) / 8);
  const dim3 g((unsigned)(8 * std::min(per_xcd, wgs_per_xcd)));
  if (!rht) p.sign_mask = 0u;
  if (had_n == 0) return launch_cast<0>(p, grid_kind, round, do_row, do_col, g, s);
  if (had_n == 16) return launch_cast<16>(p, grid_kind, round, do_row, do_col, g, s);
  return launch_cast<32>(p, grid_kind, round, do_row, do_col, g, s);
}

}  // namespace mx

// ---------------------------------------------------------------------------
// The unfused path: the rotation alone, writing float32 y, and the MX cast of
// float32 lines ("Ripensare il Bias di Shrinkage ...", Efficienza: the random
// Hadamard transform fused with the FP4 quantization against the two run
// apart).  Rotating, then casting, gives the fused kernel's codes and scales
// bit for bit: y is the same RN32(RN32(S) * c) of the exact sum S.
namespace mx {

// A workgroup takes a 32-row x 256-column tile.  The bf16 tile is read with
// coalesced 16-byte loads into LDS; thread t then rotates one 32-value block
// (row axis: block t % 8 of tile row t / 8; column axis: tile column t) from
// LDS and writes its 32 results into an LDS tile of y, which the workgroup
// stores with coalesced 16-byte stores: whole 128-byte lines of y[r][...] (row
// axis) or of the transposed y[c][...] (column axis).  Blocks the float64
// butterflies could get wrong (more than 40 binades, non-finite or
// near-overflow inputs) are computed exactly, one output at a time.  Edge
// tiles of a ragged tensor store only what lies inside it.
template <int HAD>
__global__ void __launch_bounds__(kThreads) rotate_kernel(const RotateParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t xt[kTileRows][kTileCols];     // 16 KB of bf16
  __shared__ __attribute__((aligned(16))) float yt[kTileRows * kTileCols];       // 32 KB of results
  const int t = threadIdx.x;
  const int64_t tiles_c = (p.cols + kTileCols - 1) / kTileCols;
  const int64_t row0 = (int64_t)(blockIdx.x / tiles_c) * kTileRows, col0 = (int64_t)(blockIdx.x % tiles_c) * kTileCols;
  // load: piece i = t + 256 q (q = 0..3) is 8 values of row i / 32 at column 8 (i % 32)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = t + kThreads * q, r = i >> 5, c = 8 * (i & 31);
    uint4 v = uint4{0u, 0u, 0u, 0u};
    if (row0 + r < p.rows && col0 + c < p.cols) v = *(const uint4*)(p.x + (row0 + r) * p.ld_x + col0 + c);
    *(uint4*)&xt[r][c] = v;
  }
  __syncthreads();
  const int lr = p.col ? 0 : t >> 3, lc = p.col ? t : 32 * (t & 7);
  auto get = [&](int j) { return (uint32_t)(p.col ? xt[j][lc] : xt[lr][lc + j]); };
  float y[32];
  if (block_needs_exact<HAD>(get)) {
#pragma unroll 1
    for (int i = 0; i < 32; ++i) y[i] = special_value<HAD>(get, i, p.sign_mask);
  } else {
    load_rotate<HAD>(
        [&](int h, float (&x)[16]) {
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = __uint_as_float(get(16 * h + i) << 16);
        },
        p.sign_mask, y);
  }
  // thread t's 32 results are line t / 8, values 32 (t % 8) .. of the row-axis tile (32 lines of 256), or
  // line t of the column-axis tile (256 lines of 32); either way 128 contiguous bytes, block t of yt.  Its
  // 16-byte piece s sits at slot (s + t) % 8 of the block, so that a wave's writes spread over the banks.
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *(float4*)&yt[32 * t + 4 * ((i + t) & 7)] = float4{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]};
  __syncthreads();
  // store: piece i = t + 256 q of the 2048 16-byte pieces, piece i % 8 of block i / 8; row axis: tile row
  // i / 64, columns 4 (i % 64); column axis: tile column i / 8, rows 4 (i % 8)
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = t + kThreads * q, b = i >> 3;
    const int64_t line = p.col ? col0 + b : row0 + (i >> 6);
    const int64_t pos = p.col ? row0 + 4 * (i & 7) : col0 + 4 * (i & 63);
    const bool inside = p.col ? (line < p.cols && pos < p.rows) : (line < p.rows && pos < p.cols);
    if (inside) *(float4*)(p.y + line * p.ld_y + pos) = *(const float4*)&yt[32 * b + 4 * ((i + b) & 7)];
  }
}

// One thread per 32-value block of a float32 line: block absmax, E8M0 scale,
// cast, as the fused kernel's cast of the same y (stochastic-rounding element
// index line * len + j in `stream`).  A block holding a non-finite value gets
// scale 0xFF and zero codes.
template <int GRID, int ROUND>
__global__ void __launch_bounds__(kThreads) quant_f32_kernel(const QuantF32Params p) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t nblk = p.len / 32;
  if (idx >= p.lines * nblk) return;
  const int64_t line = idx / nblk, k = idx % nblk;
  const float4* src = (const float4*)(p.y + line * p.ld_y + 32 * k);
  float y[32];
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = src[i];
    y[4 * i] = v.x;
    y[4 * i + 1] = v.y;
    y[4 * i + 2] = v.z;
    y[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) mx = max(mx, __float_as_uint(y[i]) & 0x7FFFFFFFu);
  uint32_t w[4];
  uint32_t byte = cast_block<GRID, ROUND>(y, (uint64_t)(line * p.len + 32 * k) >> 3, p.stream, (uint32_t)p.seed,
                                          (uint32_t)(p.seed >> 32), w);
  if (mx >= 0x7F800000u) {
    byte = 0xFFu;
    w[0] = w[1] = w[2] = w[3] = 0u;
  }
  *(uint4*)(p.codes + line * p.ld_codes + 16 * k) = uint4{w[0], w[1], w[2], w[3]};
  p.scales[line * p.ld_scales + k] = (uint8_t)byte;
}

hipError_t launch_rotate(RotateParams p, int had_n, bool rht, hipStream_t s) {
  if (!rht) p.sign_mask = 0u;
  const int64_t tiles = ((p.rows + kTileRows - 1) / kTileRows) * ((p.cols + kTileCols - 1) / kTileCols);
  const dim3 g((unsigned)tiles);
  if (had_n == 16) hipLaunchKernelGGL(rotate_kernel<16>, g, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(rotate_kernel<32>, g, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_quant_f32(const QuantF32Params& p, int grid_kind, int round, hipStream_t s) {
  const int64_t blocks = p.lines * (p.len / 32);
  const dim3 g((unsigned)((blocks + kThreads - 1) / kThreads));
  if (grid_kind == MX_GRID_E2M1) {
    if (round == MX_ROUND_RTNE) hipLaunchKernelGGL((quant_f32_kernel<MX_GRID_E2M1, MX_ROUND_RTNE>), g, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((quant_f32_kernel<MX_GRID_E2M1, MX_ROUND_SR>), g, dim3(kThreads), 0, s, p);
  } else {
    if (round == MX_ROUND_RTNE) hipLaunchKernelGGL((quant_f32_kernel<MX_GRID_E1M2, MX_ROUND_RTNE>), g, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((quant_f32_kernel<MX_GRID_E1M2, MX_ROUND_SR>), g, dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mx
