// Block-scaled MXFP4 x MXFP4 GEMM with fp32 accumulation on gfx950's scaled
// MFMA (V_MFMA_SCALE_F32_32X32X64_F8F6F4), the one dense contraction of the
// path ("Pre-addestramento ... con MXFP4", Metodologia: the Fprop, Dgrad and
// Wgrad GEMMs on native FP4 matrix units).
//
// C[m][n] = sum_k A[m][k] * B[n][k]; both operands K-contiguous: codes
// [rows][K/2] (element 2j in the low nibble), one E8M0 byte per 32 elements.
//
// Operand layout the MFMA expects (32x32x64, 4-bit elements): lane l holds row
// (l % 32) and the 32 consecutive k of block (l / 32) as 16 bytes, low nibble
// first, plus that block's E8M0 scale in one byte of a 32-bit operand chosen
// by op_sel; the 32x32 fp32 result sits in 16 registers, register r of lane l
// being row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
//
// The uniform E1M2 grid runs on the same instruction with 6-bit E2M3
// operands: code (s, k) maps exactly to (s << 5) | (k << 1), value k/4.
//
// Tiling: a 256-lane workgroup owns a 256x256 block of C (four waves of
// 128x128 = 4x4 MFMA tiles), K advances 128 elements (64 bytes per row) per
// step through LDS; the next step's global loads are issued before the MFMAs.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_kernels.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256;
constexpr int kBKBytes = 64;            // 128 fp4 elements per row per K step
constexpr int kGemmThreads = 256;

__device__ __forceinline__ int swz(int row, int piece) {  // 16-byte piece position within a 64-byte row
  return (piece ^ ((row >> 1) & 3)) * 16;
}

// E1M2 code nibbles (8 per dword) -> 6-bit E2M3 codes packed LSB first.
__device__ __forceinline__ void e1m2_to_e2m3(const uint32_t (&in)[4], uint32_t (&out)[6]) {
  uint64_t acc = 0;
  int nbits = 0, o = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t n = (in[d] >> (4 * q)) & 0xFu;
      const uint64_t f6 = ((n & 8u) << 2) | ((n & 7u) << 1);
      acc |= f6 << nbits;
      nbits += 6;
      if (nbits >= 32) {
        out[o++] = (uint32_t)acc;
        acc >>= 32;
        nbits -= 32;
      }
    }
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int GRID, int OUT>
__global__ void __launch_bounds__(kGemmThreads, 1)
gemm_kernel(const GemmParams p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[kBM * kBKBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kBN * kBKBytes];
  __shared__ uint32_t sSA[kBM], sSB[kBN];

  // tile order: consecutive workgroups walk down M within a column band of N
  const int tile = blockIdx.x;
  const int bm = tile % tiles_m, bn = tile / tiles_m;
  const int64_t m0 = (int64_t)bm * kBM, n0 = (int64_t)bn * kBN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t kbytes = p.K / 2, kblocks = p.K / 32;
  const int nk = (int)((p.K + 127) / 128);

  // global -> register staging: 4 x 16 B of A and of B, one scale dword each
  uint4 ra[4], rb[4];
  uint32_t rsa, rsb;
  auto gload = [&](int kt) {
    const int64_t kb0 = (int64_t)kt * kBKBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (t >> 2) + 64 * i, pc = t & 3;
      const int64_t kb = kb0 + pc * 16;
      const int64_t ga = m0 + r, gb = n0 + r;
      ra[i] = (ga < p.M && kb < kbytes) ? *(const uint4*)(p.a_codes + ga * p.lda_codes + kb) : uint4{0u, 0u, 0u, 0u};
      rb[i] = (gb < p.N && kb < kbytes) ? *(const uint4*)(p.b_codes + gb * p.ldb_codes + kb) : uint4{0u, 0u, 0u, 0u};
    }
    rsa = 0u;
    rsb = 0u;
    const int64_t ga = m0 + t, gb = n0 + t;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t kblk = (int64_t)kt * 4 + b;
      if (kblk < kblocks) {
        if (ga < p.M) rsa |= (uint32_t)p.a_scales[ga * p.lda_scales + kblk] << (8 * b);
        if (gb < p.N) rsb |= (uint32_t)p.b_scales[gb * p.ldb_scales + kblk] << (8 * b);
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (t >> 2) + 64 * i, pc = t & 3;
      *(uint4*)(sA + r * kBKBytes + swz(r, pc)) = ra[i];
      *(uint4*)(sB + r * kBKBytes + swz(r, pc)) = rb[i];
    }
    sSA[t] = rsa;
    sSB[t] = rsb;
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  gload(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8i fa[4], fb[4];
      int sa[4], sb[4];
      const int pc = 2 * h + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra_row = wm * 128 + i * 32 + (lane & 31);
        const int rb_row = wn * 128 + i * 32 + (lane & 31);
        const uint4 va = *(const uint4*)(sA + ra_row * kBKBytes + swz(ra_row, pc));
        const uint4 vb = *(const uint4*)(sB + rb_row * kBKBytes + swz(rb_row, pc));
        if constexpr (GRID == MX_GRID_E2M1) {
          fa[i] = v8i{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
          fb[i] = v8i{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
        } else {
          uint32_t o6[6];
          e1m2_to_e2m3({va.x, va.y, va.z, va.w}, o6);
          fa[i] = v8i{(int)o6[0], (int)o6[1], (int)o6[2], (int)o6[3], (int)o6[4], (int)o6[5], 0, 0};
          e1m2_to_e2m3({vb.x, vb.y, vb.z, vb.w}, o6);
          fb[i] = v8i{(int)o6[0], (int)o6[1], (int)o6[2], (int)o6[3], (int)o6[4], (int)o6[5], 0, 0};
        }
        sa[i] = (int)(sSA[ra_row] >> (8 * (lane >> 5)));
        sb[i] = (int)(sSB[rb_row] >> (8 * (lane >> 5)));
      }
      constexpr int kFmt = GRID == MX_GRID_E2M1 ? 4 : 2;   // 4: fp4 E2M1, 2: fp6 E2M3
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (h == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], kFmt, kFmt, 0, sa[i], 0, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], kFmt, kFmt, 2, sa[i], 2, sb[j]);
        }
    }
  }

  // epilogue
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        if (row < p.M && col < p.N) {
          if constexpr (OUT == MX_OUT_F32)
            ((float*)p.c)[row * p.ldc + col] = acc[i][j][r];
          else
            ((uint16_t*)p.c)[row * p.ldc + col] = f32_to_bf16_rne(acc[i][j][r]);
        }
      }
    }
}

hipError_t launch_gemm(const GemmParams& p, int grid_kind, int out_kind, hipStream_t s) {
  const int tiles_m = (int)((p.M + kBM - 1) / kBM), tiles_n = (int)((p.N + kBN - 1) / kBN);
  const dim3 g((unsigned)(tiles_m * tiles_n));
  if (grid_kind == MX_GRID_E2M1) {
    if (out_kind == MX_OUT_F32)
      hipLaunchKernelGGL((gemm_kernel<MX_GRID_E2M1, MX_OUT_F32>), g, dim3(kGemmThreads), 0, s, p, tiles_m, tiles_n);
    else
      hipLaunchKernelGGL((gemm_kernel<MX_GRID_E2M1, MX_OUT_BF16>), g, dim3(kGemmThreads), 0, s, p, tiles_m, tiles_n);
  } else {
    if (out_kind == MX_OUT_F32)
      hipLaunchKernelGGL((gemm_kernel<MX_GRID_E1M2, MX_OUT_F32>), g, dim3(kGemmThreads), 0, s, p, tiles_m, tiles_n);
    else
      hipLaunchKernelGGL((gemm_kernel<MX_GRID_E1M2, MX_OUT_BF16>), g, dim3(kGemmThreads), 0, s, p, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace mx
