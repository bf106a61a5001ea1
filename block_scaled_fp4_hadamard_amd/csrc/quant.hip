// Fused block-Hadamard + block-absmax + 4-bit cast for gfx950 (MI355X).
//
// One workgroup (256 lanes) owns a 32-row x 256-column bf16 tile:
//   1. coalesced 16-byte loads of the tile (each row segment is 512 contiguous
//      bytes), widened to fp32 once and staged in LDS (padded chunks so both
//      the row-chunk reads and the column reads are bank-conflict free);
//      the same pass takes a tile-wide max / min-nonzero of |x| that decides
//      whether float64 butterflies are exact for every chunk of the tile;
//   2. row pass: lane (r, k) rotates, scales and casts the 32-element chunk k
//      of row r and writes 16 code bytes + 1 scale byte;
//   3. column pass: lane c does the same for column c over the tile's 32 rows
//      (the Wgrad operand, blocked along tokens) and writes the transposed
//      output.
// The rotation (deterministic H16/H32 or random-sign RHT, "Pre-addestramento
// ... con MXFP4", Metodologia) runs as an in-register Walsh-Hadamard
// butterfly in float64: with the tile's inputs spanning <= 40 binades every
// partial sum is exact, so y = RN32(RN32(S) * c) matches the exact-sum
// definition bit for bit.  Tiles outside that (wide spans, Inf/NaN, values near
// the top of the range) take an exact fixed-point path instead.
// The E2M1 round-to-nearest-even cast uses gfx950's scaled fp4 conversion
// (ties to even, saturating, dividing by the power-of-two scale given as a
// float); stochastic rounding and the uniform grid run in plain VALU code.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kTileRows = 32;
constexpr int kTileCols = 256;
constexpr int kThreads = 256;
constexpr int kChunkPitch = 36;                    // floats per 32-float chunk in LDS (+16 B pad)
constexpr int kRowPitch = 8 * kChunkPitch;         // floats per tile row in LDS
constexpr int kGroup = 8;                          // row tiles sharing one XCD (a 256x256 region)

// fp32 RN32(1/sqrt(32)) = sqrt(2)/8 and 1/sqrt(16)
constexpr float kInvSqrt32 = 0x1.6a09e6p-3f;
constexpr float kInvSqrt16 = 0.25f;

__device__ __forceinline__ uint32_t e8m0_scale_bits(uint32_t byte) {
  // the float whose exponent the scaled conversions divide by: 2^(byte-127)
  return byte ? (byte << 23) : 0x00400000u;        // 2^-127 is a subnormal float
}

// Cast one 32-element block y[] (E2M1 or E1M2, RTNE or SR) into 4 code
// dwords; returns the scale byte.  `careful` blocks may hold non-finite y.
template <int GRID, int ROUND>
__device__ __forceinline__ uint32_t cast_block(const float (&y)[32], bool careful, const uint32_t (&u)[32],
                                               uint32_t (&w)[4]) {
  constexpr int kEmax = GRID == MX_GRID_E2M1 ? 2 : 0;
  uint32_t expf;
  bool nonfinite = false;
  if (!careful) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(y[i]));
    expf = __float_as_uint(m) >> 23;
  } else {
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) mb = max(mb, __float_as_uint(y[i]) & 0x7FFFFFFFu);
    nonfinite = mb >= 0x7F800000u;
    expf = mb >> 23;
  }
  const uint32_t byte = expf > (uint32_t)kEmax ? expf - kEmax : 0u;
  if (nonfinite) {
    w[0] = w[1] = w[2] = w[3] = 0u;
    return 0xFFu;
  }
  if constexpr (GRID == MX_GRID_E2M1) {
    const float sc = __uint_as_float(e8m0_scale_bits(byte));
    if constexpr (ROUND == MX_ROUND_RTNE) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t r = 0;
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 0], y[8 * d + 1], sc, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 2], y[8 * d + 3], sc, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 4], y[8 * d + 5], sc, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * d + 6], y[8 * d + 7], sc, 3);
        w[d] = r;
      }
    } else {
      // Stochastic rounding in plain arithmetic.  v = |y| / 2^e (exact unless
      // v < 2^-126, where P below is 0 either way); the quantum q is 1/2 on
      // [0,2), 1 on [2,4), 2 on [4,8); t = v / q, lo = floor(t) and
      // P = floor((t - lo) * 2^32) (t - lo is exact); round up iff u < P.
      // The magnitude code of lo is floor(t) + 2*log2(q) + 2 on every piece.
      // (gfx950's stochastic fp4 conversion is not used: it draws only 22 of
      // the 32 random bits, a coarser rule than this one.)
      const int ebias = (int)byte - 127;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t r = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float yy = y[8 * d + q];
          const float v = ldexpf(fabsf(yy), -ebias);
          const int qexp = max((int)(__float_as_uint(v) >> 23) - 128, -1);
          const float t = ldexpf(v, -qexp);
          const float fl = floorf(t);
          const uint32_t pr = (uint32_t)ldexpf(t - fl, 32);
          uint32_t k = (uint32_t)fl + (uint32_t)(2 * qexp + 2) + (u[8 * d + q] < pr ? 1u : 0u);
          k = min(k, 7u) | ((__float_as_uint(yy) >> 28) & 8u);
          r |= k << (4 * q);
        }
        w[d] = r;
      }
    }
  } else {
    // uniform grid: magnitude code k = v*4 rounded, v = |y| / 2^e; t = |y| * 2^(2-e)
    const int sh = 2 - ((int)byte - 127);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t r = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float yy = y[8 * d + q];
        const float t = ldexpf(fabsf(yy), sh);
        uint32_t k;
        if constexpr (ROUND == MX_ROUND_RTNE) {
          k = (uint32_t)rintf(t);
        } else {
          const float fl = floorf(t);
          const uint32_t p = (uint32_t)ldexpf(t - fl, 32);     // floor(frac * 2^32)
          k = (uint32_t)fl + (u[8 * d + q] < p ? 1u : 0u);
        }
        k = min(k, 7u) | ((__float_as_uint(yy) >> 28) & 8u);
        r |= k << (4 * q);
      }
      w[d] = r;
    }
  }
  return byte;
}

// Rotate 32 fp32 inputs (exact bf16 values) in place along the chunk.
template <int HAD, bool RHT>
__device__ __forceinline__ void rotate_fast(float (&y)[32], uint32_t mask) {
  double v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float x = y[i];
    if constexpr (RHT) x = __uint_as_float(__float_as_uint(x) ^ (((mask >> (i % HAD)) & 1u) << 31));
    v[i] = (double)x;
  }
#pragma unroll
  for (int h = 1; h < HAD; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const double a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  const float c = HAD == 32 ? kInvSqrt32 : kInvSqrt16;
#pragma unroll
  for (int i = 0; i < 32; ++i) y[i] = __builtin_fmaf((float)v[i], c, 0.0f);   // +0 addend: a zero sum gives +0
}

// Exact rotation for special tiles; a chunk with a non-finite input gives NaN.
template <int HAD>
__device__ __noinline__ void rotate_exact(float (&y)[32], uint32_t mask) {
  const float c = HAD == 32 ? kInvSqrt32 : kInvSqrt16;
#pragma unroll 1
  for (int base = 0; base < 32; base += HAD) {
    uint32_t xb[HAD];
    bool nonfinite = false;
    for (int j = 0; j < HAD; ++j) {
      xb[j] = __float_as_uint(y[base + j]) >> 16;
      nonfinite |= ((xb[j] >> 7) & 0xFFu) == 0xFFu;
    }
#pragma unroll 1
    for (int i = 0; i < HAD; ++i) {
      const float s = nonfinite ? __uint_as_float(0x7FC00000u) : exact_hadamard_rn32<HAD>(xb, i, mask);
      y[base + i] = __builtin_fmaf(s, c, 0.0f);
    }
  }
}

// 32 Philox words for elements [i0, i0+32) of a stream (i0 % 4 == 0).
__device__ __forceinline__ void philox_words32(uint64_t i0, uint32_t stream, uint32_t k0, uint32_t k1,
                                               uint32_t (&u)[32]) {
  const uint64_t b0 = i0 >> 2;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint64_t b = b0 + q;
    const U4 r = philox4x32_10((uint32_t)b, (uint32_t)(b >> 32), stream, 0u, k0, k1);
    u[4 * q + 0] = r.x;
    u[4 * q + 1] = r.y;
    u[4 * q + 2] = r.z;
    u[4 * q + 3] = r.w;
  }
}

template <int HAD, bool RHT, int GRID, int ROUND, bool DO_ROW, bool DO_COL>
__global__ void __launch_bounds__(kThreads)
quant_tile_kernel(const QuantParams p) {
  __shared__ __attribute__((aligned(16))) float tile[kTileRows * kRowPitch];
  __shared__ uint32_t red[2 * (kThreads / 64)];

  // ---- XCD-aware tile order: the 8 row tiles of a 256x256 region run on one
  // XCD back to back, so the column-wise output's 16-byte pieces of one
  // 128-byte line are merged in that XCD's L2.
  const uint32_t wg = blockIdx.x;
  const uint32_t xcd = wg & 7u, j = wg >> 3;
  const uint32_t region = (j >> 3) * 8u + xcd, member = j & 7u;
  const uint32_t n_regions = (uint32_t)p.n_col_tiles * (uint32_t)p.n_row_groups;
  if (region >= n_regions) return;
  const uint32_t col_tile = region / (uint32_t)p.n_row_groups;
  const uint32_t row_tile = (region % (uint32_t)p.n_row_groups) * kGroup + member;
  if (row_tile >= (uint32_t)p.n_row_tiles) return;
  const int64_t row0 = (int64_t)row_tile * kTileRows;
  const int64_t col0 = (int64_t)col_tile * kTileCols;
  const int t = threadIdx.x;

  // ---- 1. load (16 B per lane per row segment), range check, stage fp32 in LDS
  us2 mx2 = {0, 0}, mn2 = {0xFFFF, 0xFFFF};
  {
    const int q = t & 31;                       // 16-byte piece within a 512-byte row segment
    const int64_t c = col0 + q * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (t >> 5) + 8 * i;
      const int64_t row = row0 + r;
      uint4 d = {0u, 0u, 0u, 0u};
      if (row < p.rows && c < p.cols) d = *(const uint4*)(p.x + row * p.ld_x + c);
      const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        us2 m = __builtin_bit_cast(us2, dw[k] & 0x7FFF7FFFu);
        mx2 = __builtin_elementwise_max(mx2, m);
        mn2 = __builtin_elementwise_min(mn2, m - (us2){1, 1});  // zero wraps to 0xFFFF: ignored
      }
      float* dst = tile + r * kRowPitch + (q >> 2) * kChunkPitch + (q & 3) * 8;
      float4 lo = {__uint_as_float(d.x << 16), __uint_as_float(d.x & 0xFFFF0000u),
                   __uint_as_float(d.y << 16), __uint_as_float(d.y & 0xFFFF0000u)};
      float4 hi = {__uint_as_float(d.z << 16), __uint_as_float(d.z & 0xFFFF0000u),
                   __uint_as_float(d.w << 16), __uint_as_float(d.w & 0xFFFF0000u)};
      *(float4*)dst = lo;
      *(float4*)(dst + 4) = hi;
    }
  }
  uint32_t mx = max((uint32_t)mx2.x, (uint32_t)mx2.y);
  uint32_t mn = min((uint32_t)mn2.x, (uint32_t)mn2.y);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
  }
  if ((t & 63) == 0) {
    red[t >> 6] = mx;
    red[4 + (t >> 6)] = mn;
  }
  __syncthreads();
  mx = max(max(red[0], red[1]), max(red[2], red[3]));
  mn = min(min(red[4], red[5]), min(red[6], red[7]));
  // special tile: non-finite or near-overflow inputs, or (rotating) a span the
  // float64 butterfly cannot hold exactly
  bool careful = mx >= (250u << 7);
  if constexpr (HAD > 0) {
    if (mn != 0xFFFFu) {
      const int fmax = max((int)(mx >> 7), 1);
      const int fmin = max((int)((mn + 1u) >> 7), 1);
      careful |= (fmax - fmin) > 40;
    }
  }

  const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);

  // ---- 2. row pass: lane (r, k) owns chunk k of row r
  if constexpr (DO_ROW) {
    const int r = t >> 3, k = t & 7;
    const int64_t row = row0 + r, c0 = col0 + k * 32;
    if (row < p.rows && c0 < p.cols) {
      float y[32];
      const float* src = tile + r * kRowPitch + k * kChunkPitch;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 v = *(const float4*)(src + 4 * i);
        y[4 * i] = v.x; y[4 * i + 1] = v.y; y[4 * i + 2] = v.z; y[4 * i + 3] = v.w;
      }
      if constexpr (HAD > 0) {
        if (!careful) rotate_fast<HAD, RHT>(y, p.sign_mask);
        else rotate_exact<HAD>(y, RHT ? p.sign_mask : 0u);
      }
      uint32_t u[32];
      if constexpr (ROUND == MX_ROUND_SR) philox_words32((uint64_t)row * (uint64_t)p.cols + (uint64_t)c0, 0u, k0, k1, u);
      uint32_t w[4];
      const uint32_t byte = cast_block<GRID, ROUND>(y, careful, u, w);
      *(uint4*)(p.row_codes + row * p.ld_row_codes + c0 / 2) = uint4{w[0], w[1], w[2], w[3]};
      p.row_scales[row * p.ld_row_scales + c0 / 32] = (uint8_t)byte;
    }
  }

  // ---- 3. column pass: lane c owns column c of the tile (32 rows = one block)
  if constexpr (DO_COL) {
    const int64_t col = col0 + t;
    if (col < p.cols) {
      float y[32];
      const float* src = tile + (t >> 5) * kChunkPitch + (t & 31);
#pragma unroll
      for (int i = 0; i < 32; ++i) y[i] = src[i * kRowPitch];
      if constexpr (HAD > 0) {
        if (!careful) rotate_fast<HAD, RHT>(y, p.sign_mask);
        else rotate_exact<HAD>(y, RHT ? p.sign_mask : 0u);
      }
      uint32_t u[32];
      if constexpr (ROUND == MX_ROUND_SR) philox_words32((uint64_t)col * (uint64_t)p.rows + (uint64_t)row0, 1u, k0, k1, u);
      uint32_t w[4];
      const uint32_t byte = cast_block<GRID, ROUND>(y, careful, u, w);
      *(uint4*)(p.col_codes + col * p.ld_col_codes + row0 / 2) = uint4{w[0], w[1], w[2], w[3]};
      p.col_scales[col * p.ld_col_scales + row0 / 32] = (uint8_t)byte;
    }
  }
}

// ---- host-side launch: pick the instantiation
template <int HAD, bool RHT, int GRID, int ROUND>
static hipError_t launch_axes(const QuantParams& p, bool do_row, bool do_col, dim3 grid, hipStream_t s) {
  if (do_row && do_col)
    hipLaunchKernelGGL((quant_tile_kernel<HAD, RHT, GRID, ROUND, true, true>), grid, dim3(kThreads), 0, s, p);
  else if (do_row)
    hipLaunchKernelGGL((quant_tile_kernel<HAD, RHT, GRID, ROUND, true, false>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((quant_tile_kernel<HAD, RHT, GRID, ROUND, false, true>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int HAD, bool RHT>
static hipError_t launch_cast(const QuantParams& p, int grid_kind, int round, bool r, bool c, dim3 g, hipStream_t s) {
  if (grid_kind == MX_GRID_E2M1) {
    return round == MX_ROUND_RTNE ? launch_axes<HAD, RHT, MX_GRID_E2M1, MX_ROUND_RTNE>(p, r, c, g, s)
                                  : launch_axes<HAD, RHT, MX_GRID_E2M1, MX_ROUND_SR>(p, r, c, g, s);
  }
  return round == MX_ROUND_RTNE ? launch_axes<HAD, RHT, MX_GRID_E1M2, MX_ROUND_RTNE>(p, r, c, g, s)
                                : launch_axes<HAD, RHT, MX_GRID_E1M2, MX_ROUND_SR>(p, r, c, g, s);
}

hipError_t launch_quant(QuantParams p, int had_n, bool rht, int grid_kind, int round, bool do_row, bool do_col,
                        hipStream_t s) {
  p.n_row_tiles = (int32_t)((p.rows + kTileRows - 1) / kTileRows);
  p.n_col_tiles = (int32_t)((p.cols + kTileCols - 1) / kTileCols);
  p.n_row_groups = (p.n_row_tiles + kGroup - 1) / kGroup;
  const int64_t regions = (int64_t)p.n_col_tiles * p.n_row_groups;
  // WG ids: 8 consecutive regions x 8 members per 64 ids
  const int64_t wgs = ((regions + 7) / 8) * 64;
  const dim3 g((unsigned)wgs);
  if (had_n == 0) return launch_cast<0, false>(p, grid_kind, round, do_row, do_col, g, s);
  if (had_n == 16) return rht ? launch_cast<16, true>(p, grid_kind, round, do_row, do_col, g, s)
                              : launch_cast<16, false>(p, grid_kind, round, do_row, do_col, g, s);
  return rht ? launch_cast<32, true>(p, grid_kind, round, do_row, do_col, g, s)
             : launch_cast<32, false>(p, grid_kind, round, do_row, do_col, g, s);
}

}  // namespace mx
