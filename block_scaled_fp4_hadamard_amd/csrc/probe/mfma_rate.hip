// Sustained rate of gfx950's block-scaled FP4 matrix instruction
// (V_MFMA_SCALE_F32_32X32X64_F8F6F4 with 4-bit E2M1 operands) on
// register-resident operands, as a ceiling for the MXFP4 GEMM.
//
// A measurement aid, not part of the quantize/GEMM path: each wave loads one
// A and one B fragment (16 code bytes per lane) and their scale words from a
// table of 256 operand slots, then issues `iters` rounds of four independent
// MFMAs into four accumulators (no memory traffic inside the loop).  The
// operand bits set the power draw and with it the clock the chip holds, so
// the caller times the same launch on zero, constant and random operands.
//
//   mxp_mfma_rate(frags, scales, iters, workgroups, threads, sink, stream)
//     frags   device, 256 slots x 2 operands x 64 lanes x 16 bytes (512 KiB)
//     scales  device, 256 slots x 2 operands x 64 lanes x 4 bytes (128 KiB),
//             the scale byte of each lane in byte 0
//     iters   rounds per wave (> 0); each round is 4 MFMAs of 2*32*32*64 flops
//     workgroups, threads: the launch (threads 64 .. 1024, a multiple of 64)
//     sink    device, workgroups * threads floats (the accumulators' sums)
//   Returns 0, or 1 for an argument outside these bounds, or 2 when the
//   launch fails.  Does not synchronize.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(1024) mfma_rate_kernel(const uint4* frags, const uint32_t* scales, int64_t iters,
                                                         float* sink) {
  const int lane = threadIdx.x & 63;
  const int slot = (int)((blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) & 255u);
  const uint4 a = frags[(2 * slot) * 64 + lane];
  const uint4 b = frags[(2 * slot + 1) * 64 + lane];
  const int sa = (int)scales[(2 * slot) * 64 + lane];
  const int sb = (int)scales[(2 * slot + 1) * 64 + lane];
  const v8i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c0, 4, 4, 0, sa, 0, sb);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B, A, c1, 4, 4, 0, sb, 0, sa);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, A, c2, 4, 4, 0, sa, 0, sa);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B, B, c3, 4, 4, 0, sb, 0, sb);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

extern "C" int mxp_mfma_rate(const void* frags, const void* scales, long long iters, int workgroups, int threads,
                             float* sink, hipStream_t stream) {
  if (!frags || !scales || !sink || iters <= 0 || workgroups <= 0 || threads < 64 || threads > 1024 ||
      threads % 64 != 0)
    return 1;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)workgroups), dim3((unsigned)threads), 0, stream,
                     (const uint4*)frags, (const uint32_t*)scales, (int64_t)iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
