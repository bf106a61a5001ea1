// 16-value block quantization: MX scales per 16 values, and NVFP4-style
// double-block scaling ("Résumé Technique : TetraJet-v2", section 2.A:
// 16-value groups under an 8-bit scale inside 128-value outer blocks that
// carry a scale of their own, no tensor-wide absmax).
//
// MX16:   per 16 values, e = clamp(floor(log2 amax) - emax, -127, 127) as an
//         E8M0 byte, then the MX cast (the 32-value kernel's rules).
// Double: per 128 values s_o = RN32(amax128 / 2688) (float32); per 16 values
//         s_i = E4M3 nearest to amax16 / (6 s_o) (ties to even, saturating at
//         448); y = RN32(RN64(x * RN64(1 / (s_i s_o)))) cast to E2M1 at unit
//         scale.  s_i = 0 leaves only the sign; an outer block with Inf/NaN
//         gets s_o = NaN, inner 0x7F, codes 0.
//
// s_o is a product, RN32(amax * RN64(1/2688)): amax / 21 for an 8-bit
// significand is exact or has a 6-bit periodic binary expansion, so it never
// lies within a few float64 ulps of a float32 midpoint (checked for every
// finite bf16).  The E4M3 argument stays a correctly rounded float64 division:
// it can fall exactly on an E4M3 midpoint (amax16 6.375 under s_o 1), where a
// product with an inexact reciprocal would break the tie either way; off the
// midpoints it is at least 2^-32 of amax16 away from one.
//
// These scales are not what gfx950's scaled MFMA consumes (32-value blocks,
// E8M0), so this is a quantizer only.
//
// Work split: a lane owns inner blocks whole, so the 16-value maxima need no
// lane exchange, and the eight lanes of one outer block sit in one DPP row
// group of 8 (max over lanes l^1, l^2 by quad permutes, then the half-row
// mirror).
//  - Row axis: a lane takes 16 contiguous values (two 16-byte loads); a
//    workgroup takes 4096 values of one row, so a wave reads 2 KB contiguous
//    and writes 512 contiguous code bytes.
//  - Column axis: a lane takes a 16-row x 8-column tile (sixteen 16-byte row
//    loads, one inner block per column); lanes l..l+7 stack 128 rows, the 8
//    groups of a wave sit side by side (64 columns, 128 bytes per row read),
//    and a workgroup's 4 waves cover 256 columns.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

constexpr int kB16Threads = 256;
constexpr int kRowSpan = 16 * kB16Threads;     // values of a row per workgroup tile
constexpr int kColRows = 128, kColCols = 256;  // column-axis workgroup tile

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes read once: a non-temporal load
__device__ __forceinline__ uint4 load_once(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return uint4{v.x, v.y, v.z, v.w};
}

// lane-wise max of two pairs of 16-bit magnitudes
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// max over the 8 lanes l & ~7 .. l | 7 (packed 16-bit pairs)
__device__ __forceinline__ uint32_t oct_max_pk(uint32_t v) {
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // l ^ 1
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // l ^ 2
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // 7 - l within 8
  return v;
}

// nearest E4M3 code of q >= 0 (float64), ties to the even code, saturating at
// 448.  Normal range: the float64 significand rounded to 3 bits in place (add
// half an E4M3 ulp minus one, plus the kept lsb, then truncate; a carry bumps
// the exponent).  Below 2^-6 the E4M3 step is 2^-9: k = q * 2^9 rounded by the
// 2^52 add-subtract (k = 8 is the code of 2^-6).  Branch-free.
__device__ __forceinline__ uint32_t e4m3_code(double q) {
  uint64_t b = (uint64_t)__double_as_longlong(q);
  b += 0x0000FFFFFFFFFFFFull + ((b >> 49) & 1u);
  const uint32_t hi = (uint32_t)(b >> 32);
  const uint32_t normal = ((((hi >> 20) - 1016u) & 0x1Fu) << 3) | ((hi >> 17) & 7u);   // (E + 7) << 3 | m
  const uint32_t sub = (uint32_t)((q * 512.0 + 0x1p52) - 0x1p52);
  const uint32_t code = q < 0x1p-6 ? sub : normal;
  return q < 448.0 ? code : 0x7Eu;
}

__device__ __forceinline__ double e4m3_value(uint32_t code) {
  const uint32_t e = code >> 3, m = code & 7u;
  return e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + 0.125 * (double)m, (int)e - 7);
}

__device__ __forceinline__ double bf16_value(uint32_t mag) { return (double)__uint_as_float(mag << 16); }

// a / b for tile indices (uniform): 32-bit when both fit
__device__ __forceinline__ int64_t tile_div(int64_t a, int64_t b) {
  if (((a | b) >> 32) == 0) return (int64_t)((uint32_t)a / (uint32_t)b);
  return a / b;
}

// One inner block of 16 values.  get(k) gives value k as float bits (the
// bf16 pattern in the high half); amax16 / amax128 are the |x| maxima of the
// inner and outer block as bf16 magnitude patterns (>= 0x7F80: Inf/NaN
// present).  ctr8: Philox counter of value 0 (its element index / 8).
// Returns the 8 code bytes; sets the scale byte and (double block) s_o.
template <int MODE, int GRID, int ROUND, class Get>
__device__ __forceinline__ uint2 quant16(Get get, uint32_t amax16, uint32_t amax128, uint64_t ctr8, uint32_t stream,
                                         uint32_t k0, uint32_t k1, uint32_t& scale, float& so_out) {
  // stochastic rounding: the E2M1 casts take whole Philox blocks (sr_e2m1_8), the E1M2 one per-element draws
  constexpr bool kSrE2M1 = ROUND == MX_ROUND_SR && (GRID == MX_GRID_E2M1 || MODE != 0);
  uint32_t u[16] = {};
  U4 ph[2];
  if constexpr (kSrE2M1) philox4x32_10_xn<2>(ctr8, stream, k0, k1, ph);
  else if constexpr (ROUND == MX_ROUND_SR) sr_draws<2>(ctr8, stream, k0, k1, u);
  uint32_t w[2] = {0u, 0u};
  bool zero_codes;
  if constexpr (MODE == 0) {
    zero_codes = amax16 >= 0x7F80u;
    const uint32_t byte = zero_codes ? 0xFFu : scale_byte<GRID>(amax16 >> 7);
    scale = byte;
    if constexpr (GRID == MX_GRID_E2M1 && ROUND == MX_ROUND_RTNE) {
      const float sc = __uint_as_float(e8m0_scale_bits(byte));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t r = 0;
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(get(8 * h)), __uint_as_float(get(8 * h + 1)), sc, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(get(8 * h + 2)), __uint_as_float(get(8 * h + 3)), sc, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(get(8 * h + 4)), __uint_as_float(get(8 * h + 5)), sc, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(get(8 * h + 6)), __uint_as_float(get(8 * h + 7)), sc, 3);
        w[h] = r;
      }
    } else if constexpr (kSrE2M1) {
      const float sc = __uint_as_float(e8m0_scale_bits(byte));      // non-finite blocks are zeroed below
      float yy[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) yy[k] = __uint_as_float(get(k));
      w[0] = sr_e2m1_8(&yy[0], ph[0], sc);
      w[1] = sr_e2m1_8(&yy[8], ph[1], sc);
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) w[k >> 3] |= cast_one<GRID, ROUND>(__uint_as_float(get(k)), byte, u[k]) << (4 * (k & 7));
    }
  } else {
    zero_codes = amax128 >= 0x7F80u;
    const float so = zero_codes ? __uint_as_float(0x7FC00000u) : (float)(bf16_value(amax128) * (1.0 / 2688.0));
    so_out = so;
    uint32_t code = 0x7Fu;
    double r = 0.0;
    if (!zero_codes) {
      const double am = bf16_value(amax16);
      code = so > 0.0f ? e4m3_code(am / (6.0 * (double)so)) : 0u;
      const double d = e4m3_value(code) * (double)so;       // exact: 4 x 24 significant bits
      r = d > 0.0 ? 1.0 / d : 0.0;
    }
    scale = code;
    // s_i = 0 gives r = 0, and x * 0 is the zero with x's sign (x finite here)
    float y[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) y[k] = (float)((double)__uint_as_float(get(k)) * r);
    if constexpr (ROUND == MX_ROUND_RTNE) {
      const float one = 1.0f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t q = 0;
        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[8 * h], y[8 * h + 1], one, 0);
        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[8 * h + 2], y[8 * h + 3], one, 1);
        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[8 * h + 4], y[8 * h + 5], one, 2);
        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[8 * h + 6], y[8 * h + 7], one, 3);
        w[h] = q;
      }
    } else {
      w[0] = sr_e2m1_8(&y[0], ph[0], 1.0f);                         // unit scale: byte 127
      w[1] = sr_e2m1_8(&y[8], ph[1], 1.0f);
    }
  }
  if (zero_codes) w[0] = w[1] = 0u;
  return uint2{w[0], w[1]};
}

// Row axis: tile = (row, 4096-value segment); lane t takes values 16t..16t+15 of the segment.
template <int MODE, int GRID, int ROUND>
__device__ __forceinline__ void block16_row(const Block16Params& p, int64_t tile, int t) {
  const int64_t segs = (p.cols + kRowSpan - 1) / kRowSpan;
  const int64_t row = tile_div(tile, segs);
  const int64_t pos0 = (tile - row * segs) * kRowSpan + 16 * t;
  if (pos0 >= p.cols) return;                     // whole inner (and, double block, outer) blocks only
  const uint16_t* src = p.x + row * p.ld_x + pos0;
  // read once: non-temporal loads (and row-wise code stores, whole lines written once)
  const uint4 a = load_once(src), b = load_once(src + 8);
  const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t m = v[0] & 0x7FFF7FFFu;
#pragma unroll
  for (int i = 1; i < 8; ++i) m = pk_max_u16(m, v[i] & 0x7FFF7FFFu);
  const uint32_t amax16 = max(m & 0xFFFFu, m >> 16);
  const uint32_t amax128 = MODE == 1 ? oct_max_pk(amax16) : 0u;
  auto get = [&](int k) { return (k & 1) ? (v[k >> 1] & 0xFFFF0000u) : (v[k >> 1] << 16); };
  uint32_t scale;
  float so = 0.0f;
  const uint64_t ctr8 = ((uint64_t)row * (uint64_t)p.cols + (uint64_t)pos0) >> 3;
  const uint2 c = quant16<MODE, GRID, ROUND>(get, amax16, amax128, ctr8, 0u, (uint32_t)p.seed,
                                            (uint32_t)(p.seed >> 32), scale, so);
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(u32x2{c.x, c.y}, (u32x2*)(p.codes + row * p.ld_codes + pos0 / 2));
  p.scales[row * p.ld_scales + pos0 / 16] = (uint8_t)scale;
  if (MODE == 1 && (t & 7) == 0) p.outer[row * p.ld_outer + pos0 / 128] = so;
}

// Column axis: tile = (128-row band, 256-column band).
template <int MODE, int GRID, int ROUND>
__device__ __forceinline__ void block16_col(const Block16Params& p, int64_t tile, int t) {
  const int64_t ctiles = (p.cols + kColCols - 1) / kColCols;
  const int64_t rt = tile_div(tile, ctiles);
  const int lane = t & 63;
  const int64_t col = (tile - rt * ctiles) * kColCols + 64 * (t >> 6) + 8 * (lane >> 3);
  const int64_t row = rt * kColRows + 16 * (lane & 7);
  if (col >= p.cols || row >= p.rows) return;      // cols % 8 == 0; whole inner / outer blocks
  const uint16_t* src = p.x + row * p.ld_x + col;
  uint32_t v[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint4 q = load_once(src + i * p.ld_x);
    v[i][0] = q.x;
    v[i][1] = q.y;
    v[i][2] = q.z;
    v[i][3] = q.w;
  }
  // |x| maxima of the 8 columns over the 16 rows, two columns per dword
  uint32_t m[4], mo[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    m[d] = v[0][d] & 0x7FFF7FFFu;
#pragma unroll
    for (int i = 1; i < 16; ++i) m[d] = pk_max_u16(m[d], v[i][d] & 0x7FFF7FFFu);
    mo[d] = MODE == 1 ? oct_max_pk(m[d]) : 0u;
  }
  const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
  uint8_t* const cbase = p.codes + col * p.ld_codes + row / 2;
  uint8_t* const sbase = p.scales + col * p.ld_scales + row / 16;
  float* const obase = p.outer + col * p.ld_outer + row / 128;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = j >> 1;
    const uint32_t amax16 = (j & 1) ? m[d] >> 16 : m[d] & 0xFFFFu;
    const uint32_t amax128 = (j & 1) ? mo[d] >> 16 : mo[d] & 0xFFFFu;
    auto get = [&](int k) { return (j & 1) ? (v[k][d] & 0xFFFF0000u) : (v[k][d] << 16); };
    uint32_t scale;
    float so = 0.0f;
    const int64_t line = col + j;
    const uint64_t ctr8 = ((uint64_t)line * (uint64_t)p.rows + (uint64_t)row) >> 3;
    const uint2 c = quant16<MODE, GRID, ROUND>(get, amax16, amax128, ctr8, 1u, k0, k1, scale, so);
    *(uint2*)(cbase + j * p.ld_codes) = c;
    sbase[j * p.ld_scales] = (uint8_t)scale;
    if (MODE == 1 && (lane & 7) == 0) obase[j * p.ld_outer] = so;
  }
}

// MODE 0: MX16 (E8M0 per 16); MODE 1: double block (float32 per 128, E4M3 per 16)
template <int MODE, int GRID, int ROUND, bool COL>
__global__ void __launch_bounds__(kB16Threads) block16_kernel(const Block16Params p, int64_t tiles) {
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    if constexpr (COL) block16_col<MODE, GRID, ROUND>(p, tile, threadIdx.x);
    else block16_row<MODE, GRID, ROUND>(p, tile, threadIdx.x);
  }
}

template <int MODE, int GRID, int ROUND>
static void launch_axis(const Block16Params& p, bool col, hipStream_t s) {
  const int64_t tiles = col ? ((p.rows + kColRows - 1) / kColRows) * ((p.cols + kColCols - 1) / kColCols)
                            : p.rows * ((p.cols + kRowSpan - 1) / kRowSpan);
  const dim3 g((unsigned)min(tiles, (int64_t)1 << 20));
  if (col) hipLaunchKernelGGL((block16_kernel<MODE, GRID, ROUND, true>), g, dim3(kB16Threads), 0, s, p, tiles);
  else hipLaunchKernelGGL((block16_kernel<MODE, GRID, ROUND, false>), g, dim3(kB16Threads), 0, s, p, tiles);
}

hipError_t launch_block16(const Block16Params& p, bool double_block, int grid_kind, int round, bool col,
                          hipStream_t s) {
  if (double_block) {
    if (round == MX_ROUND_SR) launch_axis<1, MX_GRID_E2M1, MX_ROUND_SR>(p, col, s);
    else launch_axis<1, MX_GRID_E2M1, MX_ROUND_RTNE>(p, col, s);
  } else if (grid_kind == MX_GRID_E2M1) {
    if (round == MX_ROUND_SR) launch_axis<0, MX_GRID_E2M1, MX_ROUND_SR>(p, col, s);
    else launch_axis<0, MX_GRID_E2M1, MX_ROUND_RTNE>(p, col, s);
  } else {
    if (round == MX_ROUND_SR) launch_axis<0, MX_GRID_E1M2, MX_ROUND_SR>(p, col, s);
    else launch_axis<0, MX_GRID_E1M2, MX_ROUND_RTNE>(p, col, s);
  }
  return hipGetLastError();
}

}  // namespace mx
