// Issue cost of single vector instructions that the quantizer's cast leans
// on, against v_fma_f32: every lane runs 8 independent chains of one
// instruction for 2048 rounds (no memory traffic inside the loop), so the
// launch time per instruction and SIMD gives each one's cost in issue slots.
// A measurement aid, not part of the quantize/GEMM path.
//
//   mxp_valu_rate(op, workgroups, sink, stream)
//     op 0 v_fma_f32; 1 v_cvt_scalef32_pk_fp4_f32; 2 v_cvt_scalef32_sr_pk_fp4_f32;
//        3 v_mad_u64_u32 with an XOR of its halves (two instructions per round);
//        4 v_pk_max_u16; 5 v_mov_b32 with DPP plus an add (two);
//        6 v_permlane32_swap_b32 plus a move and an add (three per swap);
//        7 v_mul_lo_u32 plus an add (two)
//     workgroups: the launch (256 lanes each); sink: device, workgroups * 256 uint32
//   Returns 0, 1 for an argument outside these bounds, or 2 when the launch
//   fails.  Does not synchronize.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

template <int OP>
__global__ void __launch_bounds__(256) valu_rate_kernel(uint32_t* sink, uint32_t seed) {
  uint32_t a[8];
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = seed * (threadIdx.x + 17u * i) + i;
    f[i] = (float)(a[i] & 1023u) * 0.001f;
  }
  for (int it = 0; it < 2048; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (OP == 0) {
        f[i] = __builtin_fmaf(f[i], 1.0001f, 0.5f);
      } else if constexpr (OP == 1) {
        a[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a[i], f[i], f[(i + 1) & 7], 1.0f, 0);
      } else if constexpr (OP == 2) {
        a[i] = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(a[i], (v2f){f[i], 0.0f}, a[i], 1.0f, 0);
      } else if constexpr (OP == 3) {
        const uint64_t p = (uint64_t)a[i] * 0xD2511F53u;
        a[i] = (uint32_t)(p >> 32) ^ (uint32_t)p;
      } else if constexpr (OP == 4) {
        a[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a[i]),
                                                                      __builtin_bit_cast(us2, a[(i + 1) & 7])));
      } else if constexpr (OP == 5) {
        a[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)a[i], 0xB1, 0xF, 0xF, false) + 1u;
      } else if constexpr (OP == 6) {
        const auto s = __builtin_amdgcn_permlane32_swap(a[i], a[(i + 1) & 7], false, false);
        a[i] = s[0] + s[1];
      } else {
        a[i] = a[i] * a[(i + 3) & 7] + 1u;
      }
    }
  }
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += a[i] + __float_as_uint(f[i]);
  sink[blockIdx.x * 256u + threadIdx.x] = s;
}

extern "C" int mxp_valu_rate(int op, int workgroups, uint32_t* sink, hipStream_t stream) {
  if (!sink || workgroups <= 0 || op < 0 || op > 7) return 1;
  const dim3 g((unsigned)workgroups), b(256);
  const uint32_t seed = 7u;
  switch (op) {
    case 0: hipLaunchKernelGGL(valu_rate_kernel<0>, g, b, 0, stream, sink, seed); break;
    case 1: hipLaunchKernelGGL(valu_rate_kernel<1>, g, b, 0, stream, sink, seed); break;
    case 2: hipLaunchKernelGGL(valu_rate_kernel<2>, g, b, 0, stream, sink, seed); break;
    case 3: hipLaunchKernelGGL(valu_rate_kernel<3>, g, b, 0, stream, sink, seed); break;
    case 4: hipLaunchKernelGGL(valu_rate_kernel<4>, g, b, 0, stream, sink, seed); break;
    case 5: hipLaunchKernelGGL(valu_rate_kernel<5>, g, b, 0, stream, sink, seed); break;
    case 6: hipLaunchKernelGGL(valu_rate_kernel<6>, g, b, 0, stream, sink, seed); break;
    default: hipLaunchKernelGGL(valu_rate_kernel<7>, g, b, 0, stream, sink, seed); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
