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
// One thread per block of 32 values, blocks walked grid-stride.  Row axis:
// consecutive threads take consecutive blocks of a row (64 contiguous
// bytes each); column axis: consecutive threads take the same block of
// consecutive columns, so each of the 32 row reads is contiguous across the
// wave.  Sums are float64 per thread, reduced over the wave and added to the
// caller's totals with one atomic per quantity per wave.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

constexpr int kDiagThreads = 256;

__device__ __forceinline__ double grid_level(uint32_t mag, int grid) {
  if (grid == MX_GRID_E2M1) {
    // E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6: exponent field mag >> 1, mantissa bit mag & 1
    const uint32_t e = mag >> 1, m = mag & 1u;
    return e == 0 ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  }
  return 0.25 * (double)mag;
}

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

template <int HAD>
__global__ void __launch_bounds__(kDiagThreads) quant_stats_kernel(const QuantStatsParams p) {
  const int64_t len = p.axis_col ? p.rows : p.cols;       // along the quantization axis
  const int64_t lines = p.axis_col ? p.cols : p.rows;
  const int64_t nblk = lines * (len / 32);
  double sum_sq = 0.0, sum_err = 0.0;
  uint32_t hist[8] = {};
  uint32_t blocks = 0;
  for (int64_t b = (int64_t)blockIdx.x * kDiagThreads + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * kDiagThreads) {
    int64_t line, k;
    if (p.axis_col) {
      k = b / lines;
      line = b % lines;
    } else {
      line = b / (len / 32);
      k = b % (len / 32);
    }
    const uint32_t byte = p.scales[line * p.ld_scales + k];
    if (byte == 0xFFu) continue;
    double v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int64_t r = p.axis_col ? 32 * k + j : line, c = p.axis_col ? line : 32 * k + j;
      uint32_t bits = p.x[r * p.ld_x + c];
      if constexpr (HAD > 0) bits ^= ((p.sign_mask >> (j % HAD)) & 1u) << 15;
      v[j] = (double)__uint_as_float(bits << 16);
    }
    if constexpr (HAD > 0) {
      fwht_chunks<HAD>(v);
      const float c = HAD == 32 ? 0x1.6a09e6p-3f : 0.25f;
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = (double)(__builtin_fmaf((float)v[j], c, 0.0f));
    }
    const uint4 cw = *(const uint4*)(p.codes + line * p.ld_codes + 16 * k);
    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
    const double sc = ldexp(1.0, (int)byte - 127);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t nib = (w[j >> 3] >> (4 * (j & 7))) & 0xFu;
      const double lv = grid_level(nib & 7u, p.grid) * sc;
      const double yh = (nib & 8u) ? -lv : lv;
      const double e = v[j] - yh;
      sum_sq += v[j] * v[j];
      sum_err += e * e;
#pragma unroll
      for (int m = 0; m < 8; ++m) hist[m] += (nib & 7u) == (uint32_t)m;
    }
    ++blocks;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sum_sq += __shfl_xor(sum_sq, o);
    sum_err += __shfl_xor(sum_err, o);
    blocks += (uint32_t)__shfl_xor((int)blocks, o);
#pragma unroll
    for (int m = 0; m < 8; ++m) hist[m] += (uint32_t)__shfl_xor((int)hist[m], o);
  }
  if ((threadIdx.x & 63) == 0 && blocks) {
    atomicAdd(&p.out->sum_sq, sum_sq);
    atomicAdd(&p.out->sum_err_sq, sum_err);
    atomicAdd((unsigned long long*)&p.out->blocks, (unsigned long long)blocks);
#pragma unroll
    for (int m = 0; m < 8; ++m) atomicAdd((unsigned long long*)&p.out->hist[m], (unsigned long long)hist[m]);
  }
}

hipError_t launch_quant_stats(const QuantStatsParams& p, int had_n, hipStream_t s) {
  const int64_t len = p.axis_col ? p.rows : p.cols, lines = p.axis_col ? p.cols : p.rows;
  const int64_t nblk = lines * (len / 32);
  int64_t wgs = (nblk + kDiagThreads - 1) / kDiagThreads;
  if (wgs > 2048) wgs = 2048;
  const dim3 g((unsigned)wgs);
  if (had_n == 32) hipLaunchKernelGGL((quant_stats_kernel<32>), g, dim3(kDiagThreads), 0, s, p);
  else if (had_n == 16) hipLaunchKernelGGL((quant_stats_kernel<16>), g, dim3(kDiagThreads), 0, s, p);
  else hipLaunchKernelGGL((quant_stats_kernel<0>), g, dim3(kDiagThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mx
