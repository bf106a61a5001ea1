// 16-value block quantization: MX scales per 16 values, and NVFP4-style
// double-block scaling ("Résumé Technique : TetraJet-v2", section 2.A:
// 16-value groups under an 8-bit scale inside 128-value outer blocks that
// carry a scale of their own, no tensor-wide absmax).
//
// MX16:   per 16 values, e = clamp(floor(log2 amax) - emax, -127, 127) as an
//         E8M0 byte, then the MX cast (the 32-value kernel's rules).
// Double: per 128 values s_o = RN32(amax128 / 2688) (float32); per 16 values
//         s_i = E4M3 nearest to amax16 / (6 s_o) (ties to even, saturating
//         at 448; the float64 quotient lands on the same side of every E4M3
//         midpoint as the exact one); y = RN32(RN64(x * RN64(1 / (s_i s_o))))
//         cast to E2M1 at unit scale.  s_i = 0 leaves only the sign; an outer
//         block with Inf/NaN gets s_o = NaN, inner 0x7F, codes 0.
//
// These scales are not what gfx950's scaled MFMA consumes (32-value blocks,
// E8M0), so this is a quantizer only.  One thread per 128 values along the
// quantization axis: row-wise it reads 256 contiguous bytes; column-wise the
// threads of a wave take adjacent columns, so each of its 128 row reads is
// contiguous across the wave.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

constexpr int kB16Threads = 256;

// nearest E4M3 code of q >= 0 (float64), ties to the even code, saturating at 448
__device__ __forceinline__ uint32_t e4m3_code(double q) {
  if (!(q < 448.0)) return 0x7Eu;
  int e2;
  const double m = frexp(q, &e2);                 // q = m * 2^e2, m in [0.5, 1)
  int E = e2 - 1;                                 // q in [2^E, 2^(E+1))
  if (q == 0.0) return 0u;
  if (E < -6) return (uint32_t)rint(ldexp(q, 9));   // subnormal: k * 2^-9; k = 8 is the code of 2^-6
  uint32_t mant = (uint32_t)rint((ldexp(m, 1) - 1.0) * 8.0);
  if (mant == 8u) {
    mant = 0u;
    ++E;
  }
  const uint32_t code = ((uint32_t)(E + 7) << 3) | mant;
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ double e4m3_value(uint32_t code) {
  const uint32_t e = code >> 3, m = code & 7u;
  return e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + 0.125 * (double)m, (int)e - 7);
}

template <bool COL>
__device__ __forceinline__ uint32_t load_x(const Block16Params& p, int64_t line, int64_t pos) {
  return COL ? (uint32_t)p.x[pos * p.ld_x + line] : (uint32_t)p.x[line * p.ld_x + pos];
}

// MODE 0: MX16 (E8M0 per 16); MODE 1: double block (float32 per 128, E4M3 per 16)
template <int MODE, int GRID, int ROUND, bool COL>
__global__ void __launch_bounds__(kB16Threads) block16_kernel(const Block16Params p) {
  const int64_t len = COL ? p.rows : p.cols;       // along the quantization axis
  const int64_t lines = COL ? p.cols : p.rows;
  const int64_t groups = (len + 127) / 128;
  const int64_t id = (int64_t)blockIdx.x * kB16Threads + threadIdx.x;
  if (id >= lines * groups) return;
  int64_t line, g;
  if (COL) {
    g = id / lines;
    line = id % lines;
  } else {
    line = id / groups;
    g = id % groups;
  }
  const int64_t base = 128 * g;
  const int nb = (int)min((int64_t)8, (len - base) / 16);   // inner blocks present (len % 16 == 0)
  const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
  const uint32_t stream = COL ? 1u : 0u;

  // the 128 values as bf16 pairs
  uint32_t v[64];
  if (!COL && nb == 8) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 q = *(const uint4*)(p.x + line * p.ld_x + base + 8 * i);
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int64_t pos = base + 2 * i;
      v[i] = pos < len ? (load_x<COL>(p, line, pos) | (load_x<COL>(p, line, pos + 1) << 16)) : 0u;
    }
  }

  // outer scale (double block)
  double so = 0.0;
  bool outer_bad = false;
  if constexpr (MODE == 1) {
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 64; ++i) mx = max(mx, max(v[i] & 0x7FFFu, (v[i] >> 16) & 0x7FFFu));
    outer_bad = mx >= 0x7F80u;
    const float sof = outer_bad ? __uint_as_float(0x7FC00000u)
                                : (float)((double)__uint_as_float(mx << 16) / 2688.0);
    so = (double)sof;
    p.outer[line * p.ld_outer + g] = sof;
  }

#pragma unroll
  for (int b = 0; b < 8; ++b) {
    if (b < nb) {
      uint32_t mx = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = max(mx, max(v[8 * b + i] & 0x7FFFu, (v[8 * b + i] >> 16) & 0x7FFFu));
      const int64_t pos0 = base + 16 * b;
      // Philox words of the 16 elements (element index line * len + pos)
      uint32_t u[16] = {};
      if constexpr (ROUND == MX_ROUND_SR) {
        const uint64_t i0 = ((uint64_t)line * (uint64_t)len + (uint64_t)pos0) >> 2;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const U4 r = philox4x32_10((uint32_t)(i0 + h), (uint32_t)((i0 + h) >> 32), stream, 0u, k0, k1);
          u[4 * h] = r.x;
          u[4 * h + 1] = r.y;
          u[4 * h + 2] = r.z;
          u[4 * h + 3] = r.w;
        }
      }
      uint32_t w0 = 0, w1 = 0;
      uint32_t scale_byte_out;
      if constexpr (MODE == 0) {
        const bool bad = mx >= 0x7F80u;
        const uint32_t byte = bad ? 0xFFu : scale_byte<GRID>((__float_as_uint(__uint_as_float(mx << 16)) >> 23) & 0xFFu);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t bits = (i & 1) ? (v[8 * b + i / 2] & 0xFFFF0000u) : (v[8 * b + i / 2] << 16);
          const uint32_t c = cast_one<GRID, ROUND>(__uint_as_float(bits), byte, u[i]);
          if (i < 8) w0 |= c << (4 * i);
          else w1 |= c << (4 * (i - 8));
        }
        if (bad) w0 = w1 = 0u;
        scale_byte_out = byte;
      } else {
        uint32_t code = 0x7Fu;
        double r = 0.0;
        if (!outer_bad) {
          const double amax = (double)__uint_as_float(mx << 16);
          code = (so > 0.0 && amax > 0.0) ? e4m3_code(amax / (6.0 * so)) : 0u;
          const double d = e4m3_value(code) * so;             // exact: 4 x 24 significant bits
          r = d > 0.0 ? 1.0 / d : 0.0;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t bits = (i & 1) ? (v[8 * b + i / 2] & 0xFFFF0000u) : (v[8 * b + i / 2] << 16);
          const float x = __uint_as_float(bits);
          // s_i = 0: a signed zero keeps the sign
          const float y = r > 0.0 ? (float)((double)x * r) : __uint_as_float(bits & 0x80000000u);
          const uint32_t c = cast_one<MX_GRID_E2M1, ROUND>(y, 127u, u[i]);
          if (i < 8) w0 |= c << (4 * i);
          else w1 |= c << (4 * (i - 8));
        }
        if (outer_bad) w0 = w1 = 0u;
        scale_byte_out = code;
      }
      *(uint2*)(p.codes + line * p.ld_codes + pos0 / 2) = uint2{w0, w1};
      p.scales[line * p.ld_scales + pos0 / 16] = (uint8_t)scale_byte_out;
    }
  }
}

template <int MODE, int GRID, int ROUND>
static void launch_axis(const Block16Params& p, bool col, hipStream_t s) {
  const int64_t len = col ? p.rows : p.cols, lines = col ? p.cols : p.rows;
  const int64_t n = lines * ((len + 127) / 128);
  const dim3 g((unsigned)((n + kB16Threads - 1) / kB16Threads));
  if (col) hipLaunchKernelGGL((block16_kernel<MODE, GRID, ROUND, true>), g, dim3(kB16Threads), 0, s, p);
  else hipLaunchKernelGGL((block16_kernel<MODE, GRID, ROUND, false>), g, dim3(kB16Threads), 0, s, p);
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
