// OsciReset ("Résumé Technique : TetraJet-v2", 2. Méthodologie, B): per
// element, the distance the quantized weight travels over the distance the
// master weight travels; at a check chosen by the caller (small learning
// rate), a weight whose ratio exceeds the threshold is reset to the value of
// its current quantization bin, and every element starts a new window.
//
// One thread per 8 consecutive weights of a row: they share one code dword
// and one E8M0 block scale.  Every array is read and written with 16-byte
// accesses, consecutive threads on consecutive 32-byte pieces of a row.  The
// arithmetic is float32 with one rounding per operation, in the order the
// method states it (no fused multiply-adds), so that the results are exactly
// reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_kernels.h"

namespace mx {

constexpr int kOsciThreads = 256;

// the decoded value of one 4-bit code at block scale sc (a power of two as a
// float, NaN for the E8M0 NaN byte): grid level times sc, sign from bit 3;
// exact in float32 for every scale the quantizer writes
template <int GRID>
__device__ __forceinline__ float decode_code(uint32_t code, float sc) {
  const uint32_t k = code & 7u;
  float level;
  if constexpr (GRID == MX_GRID_E2M1) {
    // 0, 0.5, 1, 1.5, 2, 3, 4, 6: exponent field k >> 1, mantissa bit k & 1 (subnormal for k < 2)
    level = k < 2 ? 0.5f * (float)k : __uint_as_float(((k >> 1) + 126u) << 23 | (k & 1u) << 22);
  } else {
    level = 0.25f * (float)k;
  }
  const float v = __fmul_rn(level, sc);
  return (code & 8u) ? -v : v;
}

template <int GRID>
__global__ void __launch_bounds__(kOsciThreads) osci_kernel(const OsciParams p) {
  const int64_t per_row = p.cols / 8;
  const int64_t idx = (int64_t)blockIdx.x * kOsciThreads + threadIdx.x;
  if (idx >= p.rows * per_row) return;
  const int64_t row = idx / per_row, c = 8 * (idx % per_row);
  const uint32_t codes = *(const uint32_t*)(p.codes + row * p.ld_codes + c / 2);
  const uint32_t byte = p.scales[row * p.ld_scales + c / 32];
  const float sc = byte == 0xFFu ? __uint_as_float(0x7FC00000u)
                                 : __uint_as_float(byte ? byte << 23 : 0x00400000u);   // 2^(byte - 127)
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = decode_code<GRID>(codes >> (4 * i), sc);

  float4* wp = (float4*)(p.w + row * p.ld_w + c);
  const int64_t so = row * p.ld_s + c;
  float4* wprev = (float4*)(p.w_prev + so);
  float4* qprev = (float4*)(p.q_prev + so);
  float4* dmp = (float4*)(p.dist_m + so);
  float4* dqp = (float4*)(p.dist_q + so);
  float w[8];
  {
    const float4 a = wp[0], b = wp[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  float dm[8], dq[8];
  if (p.mode == MX_OSCI_INIT) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dm[i] = dq[i] = 0.0f;
  } else {
    float wpv[8], qpv[8], dmv[8], dqv[8];
    auto load8 = [](const float4* src, float (&v)[8]) {
      const float4 a = src[0], b = src[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    };
    load8(wprev, wpv);
    load8(qprev, qpv);
    load8(dmp, dmv);
    load8(dqp, dqv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dm[i] = __fadd_rn(dmv[i], fabsf(__fsub_rn(w[i], wpv[i])));
      dq[i] = __fadd_rn(dqv[i], fabsf(__fsub_rn(q[i], qpv[i])));
    }
    if (p.mode == MX_OSCI_CHECK) {
      uint32_t n = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool reset = dq[i] > __fmul_rn(p.threshold, dm[i]);
        if (reset) {
          w[i] = q[i];
          ++n;
        }
        dm[i] = dq[i] = 0.0f;
      }
      if (n) {
        wp[0] = float4{w[0], w[1], w[2], w[3]};
        wp[1] = float4{w[4], w[5], w[6], w[7]};
        if (p.resets) atomicAdd(p.resets, (unsigned long long)n);
      }
    }
  }
  wprev[0] = float4{w[0], w[1], w[2], w[3]};
  wprev[1] = float4{w[4], w[5], w[6], w[7]};
  qprev[0] = float4{q[0], q[1], q[2], q[3]};
  qprev[1] = float4{q[4], q[5], q[6], q[7]};
  dmp[0] = float4{dm[0], dm[1], dm[2], dm[3]};
  dmp[1] = float4{dm[4], dm[5], dm[6], dm[7]};
  dqp[0] = float4{dq[0], dq[1], dq[2], dq[3]};
  dqp[1] = float4{dq[4], dq[5], dq[6], dq[7]};
}

hipError_t launch_osci(const OsciParams& p, int grid_kind, hipStream_t s) {
  const int64_t threads = p.rows * (p.cols / 8);
  const dim3 g((unsigned)((threads + kOsciThreads - 1) / kOsciThreads));
  if (grid_kind == MX_GRID_E2M1) hipLaunchKernelGGL(osci_kernel<MX_GRID_E2M1>, g, dim3(kOsciThreads), 0, s, p);
  else hipLaunchKernelGGL(osci_kernel<MX_GRID_E1M2>, g, dim3(kOsciThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mx
