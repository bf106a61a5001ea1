// MXNorm fused with the MX cast: each row is scaled by an estimate of its
// inverse RMS built from its own block maxima, then quantized row-wise
// ("MXNorm: Reusing MXFP block scales for efficient tensor normalisation",
// Sommario tecnico 2: rho = c(p, B) * ((1/K) sum_k m_k^p)^(-1/p), the
// normalization and the MX cast fused into one operation, the gain folded
// into the next layer's weights).
//
// Arithmetic, fixed so that every bit is reproducible:
//   m_k   absmax of bf16 block k (32 values) of the row, NaN counting as +inf;
//   S     sum of m_k^p in float64 as a balanced binary tree over the blocks in
//         order (pairs of neighbours, then pairs of pairs, ...), missing
//         blocks of a power-of-two count being zeros;
//   q     RN64(S / K);
//   rho   RN32 of the exact real number c * q^(-1/p) (ties to even), or 0 when
//         q is 0 or +inf;
//   y     RN32(x * rho), then the cast of the row-wise quantizer (block
//         absmax, E8M0 scale, RTNE or stochastic rounding on stream 0, pack).
//
// One wave per row.  The row is read in groups of 8 chunks of 512 values
// (16 bytes per lane per chunk, 16 blocks per chunk, four lanes per block),
// all 8 loads of a group in flight together.  A chunk's 16 block values meet
// in a butterfly across lanes 4, 8, 16 and 32 apart, which is the balanced
// tree over those 16 blocks; the 8 chunk sums add as a tree in registers, and
// the sums of up to 16 groups in a butterfly through LDS: one balanced tree
// over 2048 block slots, the empty ones zero.  rho starts from a float64
// estimate and is corrected to the exactly rounded value with midpoint tests
// whose sign an FMA gives exactly.  The first group (rows up to 4096 values:
// the whole row) stays in registers for the second pass; later groups are
// read again.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

constexpr int kNormWaves = 4;                 // rows per 256-lane workgroup
constexpr int kChunk = 512;                   // values per chunk: 64 lanes x 8
constexpr int kGroupChunks = 8;               // chunks loaded together (4096 values)
constexpr int kMaxGroups = 16;                // cols <= 65536

// |x| of 8 bf16 values as magnitude bits; the largest, with NaN above +inf
__device__ __forceinline__ uint32_t max_mag8(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  return m;
}

// maximum over the four lanes of a quad (lanes 4b .. 4b+3 hold block b)
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // lanes l ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // lanes l ^ 2
  return v;
}

// sign(t - z) for z = c * q^(-1/p), t >= 0 dyadic with at most 25 significant
// bits: p = 1 compares t*q with c, p = 2 compares t^2*q with c^2.  t*t and c*c
// are exact in float64, and an FMA rounds the exact difference once, which
// keeps its sign.
template <int P>
__device__ __forceinline__ int cmp_to_estimate(double t, double q, double c) {
  const double r = P == 1 ? fma(t, q, -c) : fma(t * t, q, -(c * c));
  return (r > 0.0) - (r < 0.0);
}

template <int P>
__device__ float estimate_rho(double q, float c) {
  if (q == 0.0 || isinf(q)) return 0.0f;
  const double cd = (double)c;
  constexpr double kOverflow = 340282356779733661637539395458142568448.0;   // 2^128 - 2^103: rounds to +inf
  float f = P == 1 ? (float)(cd / q) : (float)(cd / sqrt(q));
  if (isinf(f)) {
    if (cmp_to_estimate<P>(kOverflow, q, cd) <= 0) return f;                  // z >= the overflow midpoint
    f = 3.40282346638528859811704183484516925440e38f;
  }
  for (int it = 0; it < 8; ++it) {
    const float up = nextafterf(f, INFINITY), dn = nextafterf(f, 0.0f);
    const double hi = isinf(up) ? kOverflow : ((double)f + (double)up) * 0.5;   // exact midpoints
    const double lo = ((double)f + (double)dn) * 0.5;
    const int ch = cmp_to_estimate<P>(hi, q, cd), cl = cmp_to_estimate<P>(lo, q, cd);
    if (ch < 0) {
      f = up;                          // z above the upper midpoint
    } else if (cl > 0) {
      f = dn;                          // z below the lower midpoint
    } else {
      if (ch == 0 && (__float_as_uint(f) & 1u)) f = up;   // a tie goes to the even neighbour
      if (cl == 0 && (__float_as_uint(f) & 1u)) f = dn;
      break;
    }
  }
  return f;
}

// chunk ch (0 .. 7) of group g of a row: 8 bf16 per lane, zeros past the row's end
__device__ __forceinline__ void load_group(const uint16_t* xr, int64_t cols, int g, int lane, uint4 (&v)[kGroupChunks]) {
#pragma unroll
  for (int ch = 0; ch < kGroupChunks; ++ch) {
    const int64_t col = ((int64_t)g * kGroupChunks + ch) * kChunk + 8 * lane;
    v[ch] = col < cols ? *(const uint4*)(xr + col) : uint4{0u, 0u, 0u, 0u};
  }
}

// tree sum of m^p over the 128 blocks of a group: within each chunk by a lane
// butterfly (quads 1, 2, 4, 8 apart), then over the 8 chunks in registers.
// bmax: each chunk's block absmax as bf16 magnitude bits (NaN kept)
template <int P>
__device__ __forceinline__ double group_sum(const uint4 (&v)[kGroupChunks], uint32_t (&bmax)[kGroupChunks]) {
  double s[kGroupChunks];
#pragma unroll
  for (int ch = 0; ch < kGroupChunks; ++ch) {
    uint32_t mb = quad_max(max_mag8(v[ch]));
    bmax[ch] = mb;
    if (mb > 0x7F80u) mb = 0x7F80u;                           // NaN counts as +inf
    const double m = (double)__uint_as_float(mb << 16);
    s[ch] = P == 1 ? m : m * m;                               // exact
  }
#pragma unroll
  for (int d = 4; d <= 32; d <<= 1)
#pragma unroll
    for (int ch = 0; ch < kGroupChunks; ++ch) s[ch] += __shfl_xor(s[ch], d);
  return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

// cast 8 values of one lane (a quarter of block col / 32) into a code word;
// returns the block's scale byte.  xmax: the block's absmax as bf16 magnitude
// bits.  Since rho >= 0 and rounding is monotonic and odd, the block's
// max |y| = max RN32(|x| rho) is RN32(max |x| * rho), NaN and inf included.
template <int GRID, int ROUND>
__device__ __forceinline__ uint32_t cast8(const uint4& v, uint32_t xmax, float rho, int64_t elem, uint32_t k0,
                                          uint32_t k1, uint32_t& word) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = __uint_as_float(w[i] << 16) * rho;
    y[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u) * rho;
  }
  const uint32_t mb = __float_as_uint(__uint_as_float(xmax << 16) * rho) & 0x7FFFFFFFu;
  const bool nonfinite = mb >= 0x7F800000u;
  const uint32_t byte = nonfinite ? 0xFFu : scale_byte<GRID>(mb >> 23);
  uint32_t r = 0;
  if constexpr (GRID == MX_GRID_E2M1 && ROUND == MX_ROUND_RTNE) {
    const float sc = __uint_as_float(e8m0_scale_bits(byte));
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[0], y[1], sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[2], y[3], sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[4], y[5], sc, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[6], y[7], sc, 3);
  } else if constexpr (GRID == MX_GRID_E2M1) {
    // stochastic rounding, a pair per conversion twice over (non-finite blocks are zeroed below)
    U4 ph[1];
    philox4x32_10_xn<1>((uint64_t)elem >> 3, 0u, k0, k1, ph);                 // elem % 8 == 0
    r = sr_e2m1_8(y, ph[0], __uint_as_float(e8m0_scale_bits(byte)));
  } else {
    uint32_t u[8] = {};
    if constexpr (ROUND == MX_ROUND_SR) sr_draws<1>((uint64_t)elem >> 3, 0u, k0, k1, u);   // elem % 8 == 0
#pragma unroll
    for (int i = 0; i < 8; ++i) r |= cast_one<GRID, ROUND>(y[i], byte, u[i]) << (4 * i);
  }
  word = nonfinite ? 0u : r;
  return byte;
}

template <int GRID, int ROUND, int P>
__global__ void __launch_bounds__(64 * kNormWaves) mxnorm_kernel(const MxNormParams p) {
  __shared__ double group_sums[kNormWaves][kMaxGroups];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kNormWaves + wave;
  if (row >= p.rows) return;                                   // the whole wave
  const int ngroups = (int)((p.cols + kGroupChunks * kChunk - 1) / (kGroupChunks * kChunk));
  const uint16_t* xr = p.x + row * p.ld_x;

  // ---- pass 1: block maxima, m^p, the tree sum (groups of 8 chunks; the
  // group sums meet in a 16-slot butterfly)
  uint4 v[kGroupChunks];
  uint32_t bmax[kGroupChunks];
  load_group(xr, p.cols, 0, lane, v);
  double total = group_sum<P>(v, bmax);
  if (ngroups > 1) {
    if (lane == 0) group_sums[wave][0] = total;
    for (int g = 1; g < ngroups; ++g) {
      uint4 w[kGroupChunks];
      uint32_t wmax[kGroupChunks];
      load_group(xr, p.cols, g, lane, w);
      const double gs = group_sum<P>(w, wmax);
      if (lane == 0) group_sums[wave][g] = gs;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                        // lgkmcnt(0): the sums are in LDS
    __builtin_amdgcn_wave_barrier();
    // a butterfly over all 64 lanes (slots past the groups are zeros), so
    // that every lane ends with the same total
    double t = lane < ngroups ? group_sums[wave][lane] : 0.0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) t += __shfl_xor(t, d);
    total = t;
  }
  const double q = total / (double)(p.cols / 32);
  const float rho = estimate_rho<P>(q, p.c);
  if (lane == 0) p.rho[row] = rho;

  // ---- pass 2: y = RN32(x * rho), block scale, cast, pack (the first
  // group is still in registers)
  const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
  uint32_t* const crow = (uint32_t*)(p.codes + row * p.ld_codes) + lane;    // 4 code bytes per lane and chunk
  uint8_t* const srow = p.scales + row * p.ld_scales + lane / 4;
  for (int g = 0; g < ngroups; ++g) {
    if (g > 0) {
      load_group(xr, p.cols, g, lane, v);
#pragma unroll
      for (int ch = 0; ch < kGroupChunks; ++ch) bmax[ch] = quad_max(max_mag8(v[ch]));
    }
#pragma unroll
    for (int ch = 0; ch < kGroupChunks; ++ch) {
      const int64_t col = ((int64_t)g * kGroupChunks + ch) * kChunk + 8 * lane;
      uint32_t word;
      const uint32_t byte = cast8<GRID, ROUND>(v[ch], bmax[ch], rho, row * p.cols + col, k0, k1, word);
      if (col < p.cols) {
        const int c = g * kGroupChunks + ch;
        __builtin_nontemporal_store(word, crow + 64 * c);                       // written once
        if ((lane & 3) == 0) srow[16 * c] = (uint8_t)byte;
      }
    }
  }
}

template <int GRID, int ROUND, int P>
static void launch_p(const MxNormParams& p, dim3 g, hipStream_t s) {
  hipLaunchKernelGGL((mxnorm_kernel<GRID, ROUND, P>), g, dim3(64 * kNormWaves), 0, s, p);
}

template <int GRID, int ROUND>
static void launch_gr(const MxNormParams& p, int power, dim3 g, hipStream_t s) {
  if (power == 1) launch_p<GRID, ROUND, 1>(p, g, s);
  else launch_p<GRID, ROUND, 2>(p, g, s);
}

hipError_t launch_mxnorm(const MxNormParams& p, int power, int grid_kind, int round, hipStream_t s) {
  const dim3 g((unsigned)((p.rows + kNormWaves - 1) / kNormWaves));
  if (grid_kind == MX_GRID_E2M1) {
    if (round == MX_ROUND_SR) launch_gr<MX_GRID_E2M1, MX_ROUND_SR>(p, power, g, s);
    else launch_gr<MX_GRID_E2M1, MX_ROUND_RTNE>(p, power, g, s);
  } else {
    if (round == MX_ROUND_SR) launch_gr<MX_GRID_E1M2, MX_ROUND_SR>(p, power, g, s);
    else launch_gr<MX_GRID_E1M2, MX_ROUND_RTNE>(p, power, g, s);
  }
  return hipGetLastError();
}

}  // namespace mx
