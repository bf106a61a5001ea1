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
// One wave per row.  The row is read in chunks of 512 values (16 bytes per
// lane, 16 blocks per chunk, four lanes per block).  A chunk's 16 block
// values meet in a butterfly across lanes 4, 8, 16 and 32 apart, which is the
// balanced tree over those 16 blocks; the chunk sums go to LDS and a second
// butterfly over up to 128 chunk slots finishes the tree.  rho starts from a
// float64 estimate and is corrected to the exactly rounded value with
// midpoint tests whose sign an FMA gives exactly.  Rows of up to 4096 values
// stay in registers for the second pass; longer rows are read again.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

constexpr int kNormWaves = 4;                 // rows per 256-lane workgroup
constexpr int kChunk = 512;                   // values per chunk: 64 lanes x 8
constexpr int kMaxChunks = 128;               // cols <= 65536
constexpr int kRegChunks = 8;                 // rows up to 4096 values stay in registers

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

template <int GRID, int ROUND, int P, bool REGS>
__global__ void __launch_bounds__(64 * kNormWaves) mxnorm_kernel(const MxNormParams p) {
  __shared__ double chunk_sums[kNormWaves][kMaxChunks];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kNormWaves + wave;
  if (row >= p.rows) return;                                   // the whole wave
  const int nch = (int)((p.cols + kChunk - 1) / kChunk);
  const uint16_t* xr = p.x + row * p.ld_x;
  double* sums = chunk_sums[wave];

  // ---- pass 1: block maxima, m^p, the tree sum
  uint4 keep[REGS ? kRegChunks : 1];
#pragma unroll
  for (int i = 0; i < (REGS ? kRegChunks : 1); ++i) keep[i] = uint4{0u, 0u, 0u, 0u};
  for (int ch = 0; ch < nch; ++ch) {
    const int64_t col = (int64_t)ch * kChunk + 8 * lane;
    uint4 v = uint4{0u, 0u, 0u, 0u};
    if (col < p.cols) v = *(const uint4*)(xr + col);
    if constexpr (REGS) {
#pragma unroll
      for (int i = 0; i < kRegChunks; ++i)
        if (i == ch) keep[i] = v;
    }
    uint32_t mb = quad_max(max_mag8(v));
    if (mb > 0x7F80u) mb = 0x7F80u;                           // NaN counts as +inf
    const double m = (double)__uint_as_float(mb << 16);
    double s = P == 1 ? m : m * m;                            // exact
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (lane == 0) sums[ch] = s;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);                          // lgkmcnt(0): the sums are in LDS
  __builtin_amdgcn_wave_barrier();
  double t = (2 * lane < nch ? sums[2 * lane] : 0.0) + (2 * lane + 1 < nch ? sums[2 * lane + 1] : 0.0);
  t += __shfl_xor(t, 1);
  t += __shfl_xor(t, 2);
  t += __shfl_xor(t, 4);
  t += __shfl_xor(t, 8);
  t += __shfl_xor(t, 16);
  t += __shfl_xor(t, 32);
  const double q = t / (double)(p.cols / 32);
  const float rho = estimate_rho<P>(q, p.c);
  if (lane == 0) p.rho[row] = rho;

  // ---- pass 2: y = RN32(x * rho), block scale, cast, pack
  const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
  for (int ch = 0; ch < nch; ++ch) {
    const int64_t col = (int64_t)ch * kChunk + 8 * lane;
    uint4 v = uint4{0u, 0u, 0u, 0u};
    if constexpr (REGS) {
#pragma unroll
      for (int i = 0; i < kRegChunks; ++i)
        if (i == ch) v = keep[i];
    } else {
      if (col < p.cols) v = *(const uint4*)(xr + col);
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float y[8];
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[2 * i] = __uint_as_float(w[i] << 16) * rho;
      y[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u) * rho;
      mb = max(mb, max(__float_as_uint(y[2 * i]) & 0x7FFFFFFFu, __float_as_uint(y[2 * i + 1]) & 0x7FFFFFFFu));
    }
    mb = quad_max(mb);
    const bool nonfinite = mb >= 0x7F800000u;
    const uint32_t byte = nonfinite ? 0xFFu : scale_byte<GRID>(mb >> 23);
    uint32_t u[8] = {};
    if constexpr (ROUND == MX_ROUND_SR) {
      const uint64_t i0 = ((uint64_t)row * (uint64_t)p.cols + (uint64_t)col) >> 2;   // element index / 4
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const U4 r = philox4x32_10((uint32_t)(i0 + h), (uint32_t)((i0 + h) >> 32), 0u, 0u, k0, k1);
        u[4 * h] = r.x;
        u[4 * h + 1] = r.y;
        u[4 * h + 2] = r.z;
        u[4 * h + 3] = r.w;
      }
    }
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= cast_one<GRID, ROUND>(y[i], byte, u[i]) << (4 * i);
    if (nonfinite) word = 0;
    if (col < p.cols) {
      *(uint32_t*)(p.codes + row * p.ld_codes + col / 2) = word;
      if ((lane & 3) == 0) p.scales[row * p.ld_scales + col / 32] = (uint8_t)byte;
    }
  }
}

template <int GRID, int ROUND, int P>
static void launch_p(const MxNormParams& p, dim3 g, hipStream_t s) {
  if (p.cols <= (int64_t)kRegChunks * kChunk)
    hipLaunchKernelGGL((mxnorm_kernel<GRID, ROUND, P, true>), g, dim3(64 * kNormWaves), 0, s, p);
  else
    hipLaunchKernelGGL((mxnorm_kernel<GRID, ROUND, P, false>), g, dim3(64 * kNormWaves), 0, s, p);
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
