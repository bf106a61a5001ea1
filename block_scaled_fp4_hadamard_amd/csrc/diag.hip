// Quantization diagnostics of an MX-quantized tensor: signal energy, noise
// energy and the histogram of magnitude codes ("Ripensare il Bias di
// Shrinkage nel Pretraining di LLM in FP4", Risultati Sperimentali,
// Diagnostica di Quantizzazione: SQNR and bucket usage with and without the
// random Hadamard rotation, for E2M1 and the uniform E1M2 grid).
//
// The signal is y, the values the cast received: the bf16 inputs, or with a
// rotation y = RN32(RN32(S) * RN32(1/sqrt(n))) with S formed by float64
// butterflies (exact when a chunk spans at most 40 binades, as in the
// quantizer's float64 class; within float64 rounding otherwise).  The noise is
// y - y_hat, y_hat = grid level * 2^(scale byte - 127).  Blocks whose scale
// byte is 0xFF are left out.
//
// One thread per block of 32 values, blocks walked grid-stride with an
// incremental (line, block) cursor.  Row axis: consecutive threads take
// consecutive blocks of a row, each reading its 64 contiguous input bytes as
// four 16-byte loads when the rows allow it; column axis: consecutive threads
// take the same block of consecutive columns, so each of the 32 row reads is
// contiguous across the wave.  The decoded level is formed in float (exact)
// and scaled in float64; the error, the squares and their sums are float64 per
// thread, reduced over the wave and added to the caller's totals with one
// atomic per quantity per wave.  Code counts go into eight 8-bit lanes of a
// 64-bit counter per block (32 codes cannot overflow one), unpacked into the
// thread's totals once per block.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

constexpr int kDiagThreads = 1024;   // one workgroup per CU, four waves per SIMD

template <int HAD>
__device__ __forceinline__ void fwht_chunks(double (&v)[32]) {
#pragma unroll
  for (int h = 1; h < HAD; h <<= 1)
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if ((i & h) == 0) {
        const double a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
}

// float bits of the magnitude of code mag (3 bits): E2M1 0, 0.5, 1, 1.5, 2, 3, 4, 6 (from 2 up, exponent
// field mag >> 1 and mantissa bit mag & 1 sit at bits 23 and 22); the uniform grid mag / 4
template <int GRID>
__device__ __forceinline__ uint32_t level_bits(uint32_t mag) {
  if constexpr (GRID == MX_GRID_E2M1) {
    const uint32_t wide = (mag << 22) + 0x3F000000u;
    return mag >= 2u ? wide : (mag == 1u ? 0x3F000000u : 0u);
  } else {
    return __float_as_uint(0.25f * (float)mag);
  }
}

// COL: blocks run down columns; VEC: row-axis inputs read 16 bytes at a time (16-byte aligned rows)
template <int HAD, int GRID, bool COL, bool VEC>
__global__ void __launch_bounds__(kDiagThreads) __attribute__((amdgpu_waves_per_eu(4)))
quant_stats_kernel(const QuantStatsParams p) {
  const int64_t len = COL ? p.rows : p.cols;       // along the quantization axis
  const int64_t lines = COL ? p.cols : p.rows;
  const int64_t nb = len / 32;                    // blocks per line
  const int64_t nblk = lines * nb;
  // block b = major * nminor + minor: row axis (line, k) = (major, minor), column axis (k, line)
  const int64_t nminor = COL ? lines : nb;
  const int64_t b0 = (int64_t)blockIdx.x * kDiagThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kDiagThreads;
  int64_t major = b0 / nminor, minor = b0 % nminor;
  const int64_t smajor = stride / nminor, sminor = stride % nminor;
  double sum_sq = 0.0, sum_err = 0.0;
  uint32_t hist[8] = {};
  uint32_t blocks = 0;
  for (int64_t b = b0; b < nblk; b += stride) {
    const int64_t line = COL ? minor : major, k = COL ? major : minor;
    const uint32_t byte = p.scales[line * p.ld_scales + k];
    if (byte != 0xFFu) {
      uint32_t bits[32];
      if constexpr (!COL && VEC) {
        const uint4* src = (const uint4*)(p.x + line * p.ld_x + 32 * k);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = src[q];
          const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bits[8 * q + 2 * e] = d[e] & 0xFFFFu;
            bits[8 * q + 2 * e + 1] = d[e] >> 16;
          }
        }
      } else if constexpr (COL) {
        // one running address down the column, so that 32 addresses are not held at once
        const uint16_t* src = p.x + 32 * k * p.ld_x + line;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          bits[j] = *src;
          src += p.ld_x;
        }
      } else {
        const uint16_t* src = p.x + line * p.ld_x + 32 * k;
#pragma unroll
        for (int j = 0; j < 32; ++j) bits[j] = src[j];
      }
      double v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        uint32_t w = bits[j];
        if constexpr (HAD > 0) w ^= ((p.sign_mask >> (j % HAD)) & 1u) << 15;
        v[j] = (double)__uint_as_float(w << 16);
      }
      if constexpr (HAD > 0) {
        fwht_chunks<HAD>(v);
        const float c = HAD == 32 ? 0x1.6a09e6p-3f : 0.25f;
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = (double)(__builtin_fmaf((float)v[j], c, 0.0f));
      }
      const uint4 cw = *(const uint4*)(p.codes + line * p.ld_codes + 16 * k);
      const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
      // 2^(byte - 127) as a float64 (normal for every byte below 0xFF)
      const double sc = __longlong_as_double((long long)((uint64_t)(byte + 896u) << 52));
      uint64_t cnt = 0;
      // four partial sums per quantity: short dependence chains, so the float64 work need not be held
      // in registers to cover their latency
      double psq[4] = {}, perr[4] = {};
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t nib = (w[j >> 3] >> (4 * (j & 7))) & 0xFu;
        const uint32_t mag = nib & 7u;
        const float lv = __uint_as_float(level_bits<GRID>(mag) | ((nib & 8u) << 28));
        const double e = v[j] - (double)lv * sc;
        psq[j & 3] = __builtin_fma(v[j], v[j], psq[j & 3]);
        perr[j & 3] = __builtin_fma(e, e, perr[j & 3]);
        cnt += (uint64_t)1 << (8 * mag);
      }
      sum_sq += (psq[0] + psq[1]) + (psq[2] + psq[3]);
      sum_err += (perr[0] + perr[1]) + (perr[2] + perr[3]);
#pragma unroll
      for (int m = 0; m < 8; ++m) hist[m] += (uint32_t)(cnt >> (8 * m)) & 0xFFu;
      ++blocks;
    }
    major += smajor;
    minor += sminor;
    if (minor >= nminor) {
      minor -= nminor;
      ++major;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sum_sq += __shfl_xor(sum_sq, o);
    sum_err += __shfl_xor(sum_err, o);
    blocks += (uint32_t)__shfl_xor((int)blocks, o);
#pragma unroll
    for (int m = 0; m < 8; ++m) hist[m] += (uint32_t)__shfl_xor((int)hist[m], o);
  }
  // the workgroup's waves combine in LDS, and one lane per quantity adds the workgroup's total: eleven
  // atomics per workgroup, since atomics on the same few addresses are serialized
  __shared__ double wsum[kDiagThreads / 64][2];
  __shared__ uint32_t wcnt[kDiagThreads / 64][9];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    wsum[wave][0] = sum_sq;
    wsum[wave][1] = sum_err;
#pragma unroll
    for (int m = 0; m < 8; ++m) wcnt[wave][m] = hist[m];
    wcnt[wave][8] = blocks;
  }
  __syncthreads();
  const int q = threadIdx.x;
  if (q < 11) {
    double ds = 0.0;
    unsigned long long us = 0;
    for (int i = 0; i < kDiagThreads / 64; ++i) {
      if (q < 2) ds += wsum[i][q];
      else us += wcnt[i][q - 2];
    }
    if (q < 2) {
      if (ds != 0.0) atomicAdd(q == 0 ? &p.out->sum_sq : &p.out->sum_err_sq, ds);
    } else if (us != 0) {
      atomicAdd((unsigned long long*)(q == 10 ? &p.out->blocks : &p.out->hist[q - 2]), us);
    }
  }
}

template <int HAD, int GRID>
static void launch_stats(const QuantStatsParams& p, dim3 g, hipStream_t s) {
  const bool vec = ((uintptr_t)p.x % 16 == 0) && p.ld_x % 8 == 0;
  if (p.axis_col) hipLaunchKernelGGL((quant_stats_kernel<HAD, GRID, true, false>), g, dim3(kDiagThreads), 0, s, p);
  else if (vec) hipLaunchKernelGGL((quant_stats_kernel<HAD, GRID, false, true>), g, dim3(kDiagThreads), 0, s, p);
  else hipLaunchKernelGGL((quant_stats_kernel<HAD, GRID, false, false>), g, dim3(kDiagThreads), 0, s, p);
}

template <int HAD>
static void launch_stats_had(const QuantStatsParams& p, dim3 g, hipStream_t s) {
  if (p.grid == MX_GRID_E2M1) launch_stats<HAD, MX_GRID_E2M1>(p, g, s);
  else launch_stats<HAD, MX_GRID_E1M2>(p, g, s);
}

hipError_t launch_quant_stats(const QuantStatsParams& p, int had_n, hipStream_t s) {
  const int64_t len = p.axis_col ? p.rows : p.cols, lines = p.axis_col ? p.cols : p.rows;
  const int64_t nblk = lines * (len / 32);
  int64_t wgs = (nblk + kDiagThreads - 1) / kDiagThreads;
  if (wgs > 256) wgs = 256;          // persistent: one workgroup per CU walks its blocks grid-stride
  const dim3 g((unsigned)wgs);
  if (had_n == 32) launch_stats_had<32>(p, g, s);
  else if (had_n == 16) launch_stats_had<16>(p, g, s);
  else launch_stats_had<0>(p, g, s);
  return hipGetLastError();
}

}  // namespace mx
