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
// The uniform E1M2 grid runs on the same instruction with FP8 E4M3 operands
// (every value k/4 is exact in E4M3), converted after the LDS read; the
// FP6 E2M3 form (s << 5) | (k << 1) is kept as the alternative carrier.
//
// Tiling: every kernel gives a workgroup 256x256 blocks of C.  The whole-tile
// kernel (the hot path) is persistent, one 512-lane workgroup per CU: eight
// waves of 128x64 (4x2 MFMA tiles), K advancing 256 elements (128 bytes per
// row) per step, the next step copied global -> LDS by DMA while the MFMAs
// consume the current one.  The general kernel (any shape) uses four waves of
// 128x128, K advancing 128 elements per step through bounds-checked loads.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_kernels.h"
#include "gemm_path.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256;
constexpr int kBKBytes = 64;            // 128 fp4 elements per row per K step
constexpr int kGemmThreads = 256;

__device__ __forceinline__ int swz(int row, int piece) {  // 16-byte piece position within a 64-byte row
  return (piece ^ ((row >> 1) & 3)) * 16;
}

// E1M2 code nibbles (8 per dword) -> 6-bit E2M3 codes packed LSB first:
// nibble (s, k) becomes (s << 5) | (k << 1).  The 8 nibbles of a dword are
// spread from a 4-bit to a 6-bit pitch in three steps (halves 8 bits apart,
// then quarters 4 bits, then odd nibbles 2 bits), each a shift and two masks
// on a 64-bit value, and the fields are then formed in place.  The 48-bit
// chunks of the four dwords concatenate into the six output dwords.
__device__ __forceinline__ uint64_t e1m2_chunk(uint32_t d) {
  uint64_t x = d;
  x = (x & 0x000000000000FFFFull) | ((x << 8) & 0x000000FFFF000000ull);
  x = (x & 0x00000000FF0000FFull) | ((x << 4) & 0x00000FF0000FF000ull);
  x = (x & 0x000000F00F00F00Full) | ((x << 2) & 0x00003C03C03C03C0ull);
  return ((x & 0x0000208208208208ull) << 2) | ((x & 0x00001C71C71C71C7ull) << 1);
}
__device__ __forceinline__ void e1m2_to_e2m3(const uint32_t (&in)[4], uint32_t (&out)[6]) {
  const uint64_t c0 = e1m2_chunk(in[0]), c1 = e1m2_chunk(in[1]), c2 = e1m2_chunk(in[2]), c3 = e1m2_chunk(in[3]);
  out[0] = (uint32_t)c0;
  out[1] = (uint32_t)(c0 >> 32) | ((uint32_t)c1 << 16);
  out[2] = (uint32_t)(c1 >> 16);
  out[3] = (uint32_t)c2;
  out[4] = (uint32_t)(c2 >> 32) | ((uint32_t)c3 << 16);
  out[5] = (uint32_t)(c3 >> 16);
}

// E1M2 code nibbles (8 per dword) -> FP8 E4M3 bytes with the same values
// (k/4 for magnitude code k, sign from bit 3): a byte-permute table lookup of
// the magnitude codes and the sign bit moved to bit 7.  The even nibbles of a
// dword land in the low output dword and the odd ones in the high one, so a
// block's values are reordered; both operands are reordered alike and the
// block's scale is shared, so the dot product is the same sum.
//
// The 8-bit operand layout differs from the 4- and 6-bit one: in every lane,
// bytes 0-15 belong to the first 32-wide block of the 64 k (scaled by lane
// l % 32's scale) and bytes 16-31 to the second (lane l % 32 + 32's scale).
// Lane l < 32 converts block 0 and lane l + 32 block 1, so the upper 16 bytes
// of the low lanes trade places with the lower 16 bytes of the high lanes.
constexpr uint32_t kE4M3QuarterLo = 0x34302800u;   // 0, 0.25, 0.5, 0.75
constexpr uint32_t kE4M3QuarterHi = 0x3E3C3A38u;   // 1, 1.25, 1.5, 1.75
__device__ __forceinline__ void e1m2_to_e4m3(const uint32_t (&in)[4], uint32_t (&out)[8]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = in[d];
    const uint32_t lo = __builtin_amdgcn_perm(kE4M3QuarterHi, kE4M3QuarterLo, w & 0x07070707u);
    const uint32_t hi = __builtin_amdgcn_perm(kE4M3QuarterHi, kE4M3QuarterLo, (w >> 4) & 0x07070707u);
    out[2 * d] = lo | ((w << 4) & 0x80808080u);
    out[2 * d + 1] = hi | (w & 0x80808080u);
  }
}

// the FP8 or the FP6 carrier of the uniform grid on the matrix cores
constexpr bool kE1M2AsFp8 = true;

// One lane's MFMA operand from its 16 code bytes (32 values of a block): E2M1
// as is (fp4), E1M2 as FP8 E4M3 (exchanged across the wave's halves, so the
// whole wave must call it together) or FP6 E2M3 of the same values.
template <int GRID>
__device__ __forceinline__ v8i operand(const uint4& x) {
  if constexpr (GRID == MX_GRID_E2M1) {
    return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  } else if constexpr (kE1M2AsFp8) {
    uint32_t o8[8];
    e1m2_to_e4m3({x.x, x.y, x.z, x.w}, o8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // lanes 32-63 of o8[i] <-> lanes 0-31 of o8[4 + i]
      const auto sw = __builtin_amdgcn_permlane32_swap(o8[i], o8[4 + i], false, false);
      o8[i] = sw[0];
      o8[4 + i] = sw[1];
    }
    return v8i{(int)o8[0], (int)o8[1], (int)o8[2], (int)o8[3], (int)o8[4], (int)o8[5], (int)o8[6], (int)o8[7]};
  } else {
    uint32_t o6[6];
    e1m2_to_e2m3({x.x, x.y, x.z, x.w}, o6);
    return v8i{(int)o6[0], (int)o6[1], (int)o6[2], (int)o6[3], (int)o6[4], (int)o6[5], 0, 0};
  }
}

// The whole-tile kernel's operand: its E1M2 fragments already hold half of each block (load_quarter), so
// the FP8 bytes need no exchange across the wave's halves.
template <int GRID>
__device__ __forceinline__ v8i operand_tile(const uint4& x) {
  if constexpr (GRID == MX_GRID_E1M2 && kE1M2AsFp8) {
    uint32_t o8[8];
    e1m2_to_e4m3({x.x, x.y, x.z, x.w}, o8);
    return v8i{(int)o8[0], (int)o8[1], (int)o8[2], (int)o8[3], (int)o8[4], (int)o8[5], (int)o8[6], (int)o8[7]};
  } else {
    return operand<GRID>(x);
  }
}

// MFMA format code of a grid's operands: 4 fp4 E2M1; 0 fp8 E4M3 or 2 fp6 E2M3 for E1M2
template <int GRID>
constexpr int mfma_fmt() { return GRID == MX_GRID_E2M1 ? 4 : (kE1M2AsFp8 ? 0 : 2); }

// Two floats to packed bf16 (a in the low half) by gfx950's packed conversion:
// round to nearest even, a NaN quieted with its payload kept.  Over all 2^32
// float inputs it gives the same bits as the plain definition, that is
// (u + 0x7FFF + bit 16 of u) >> 16 for non-NaN u, and (u >> 16) | 0x40 for NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Tile order: workgroup ids are dealt round-robin to the 8 XCDs.  Groups of
// 4 (M) x 8 (N) tiles are dealt to XCDs group by group, so the 32 workgroups
// an XCD runs at once share 4 A strips and 8 B strips in that XCD's L2.
constexpr int kGroupM = 4, kGroupN = 8, kXcds = 8;



struct TileMap {
  int tiles_m, tiles_n, groups_m, groups;
};

__device__ __forceinline__ bool map_tile(const TileMap& tm, int& bm, int& bn) {
  const int id = blockIdx.x;
  const int xcd = id % kXcds, j = id / kXcds;
  const int g = (j / (kGroupM * kGroupN)) * kXcds + xcd, m = j % (kGroupM * kGroupN);
  if (g >= tm.groups) return false;
  bm = (g % tm.groups_m) * kGroupM + m % kGroupM;
  bn = (g / tm.groups_m) * kGroupN + m / kGroupM;
  return bm < tm.tiles_m && bn < tm.tiles_n;
}

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))


// Fragments of one K step from an LDS stage and its MFMAs: the wave owns
// MT x NT 32x32 tiles at rows r0 + 32i, columns c0 + 32j of the block.
template <int GRID, int MT, int NT>
__device__ __forceinline__ void mma_step(const uint8_t* a, const uint8_t* b, const uint32_t* sa_w,
                                         const uint32_t* sb_w, int r0, int c0, int lane, v16f (&acc)[MT][NT]) {
  const int half = lane >> 5, lrow = lane & 31;
  v8i fa[2][MT], fb[2][NT];
  int sa[MT], sb[NT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int ar = r0 + i * 32 + lrow;
    sa[i] = (int)(sa_w[ar] >> (8 * half));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 x = *(const uint4*)(a + ar * kBKBytes + swz(ar, 2 * h + half));
      fa[h][i] = operand<GRID>(x);
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int br = c0 + j * 32 + lrow;
    sb[j] = (int)(sb_w[br] >> (8 * half));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 y = *(const uint4*)(b + br * kBKBytes + swz(br, 2 * h + half));
      fb[h][j] = operand<GRID>(y);
    }
  }
  constexpr int kFmt = mfma_fmt<GRID>();
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[0][i], fb[0][j], acc[i][j], kFmt, kFmt, 0,
                                                                  sa[i], 0, sb[j]);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[1][i], fb[1][j], acc[i][j], kFmt, kFmt, 2,
                                                                  sa[i], 2, sb[j]);
}

// register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32 of a 32x32 tile;
// for each r the 64 lanes write two 32-element row segments
template <int OUT, bool CHECK, int MT, int NT>
__device__ __forceinline__ void store_tile(const GemmParams& p, int64_t row0, int64_t col0, int lane,
                                           const v16f (&acc)[MT][NT]) {
  const int half = lane >> 5, lrow = lane & 31;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t col = col0 + j * 32 + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
        if (!CHECK || (row < p.M && col < p.N)) {
          if constexpr (OUT == MX_OUT_F32)
            ((float*)p.c)[row * p.ldc + col] = acc[i][j][r];
          else
            ((uint16_t*)p.c)[row * p.ldc + col] = (uint16_t)pack_bf16(acc[i][j][r], 0.0f);
        }
      }
    }
}

// Whole-tile epilogue with wide stores.  For each group of four accumulator
// registers (four consecutive rows) and each quad of lanes (four consecutive
// columns) the 4x4 block is transposed with two DPP exchanges (lane pairs
// l ^ 1, then l ^ 2), after which lane 4a + k holds row k of the block,
// columns 4a .. 4a + 3 in order: one 16-byte fp32 store per lane and register
// group, every row segment a whole 128-byte run.  bf16 goes further (below):
// neighbouring quads pair up so that each lane stores eight columns, 16
// bytes, since the store instruction count bounds the epilogue.  Values are
// moved, never combined, so the stored numbers are the accumulators' (or
// their bf16 roundings) bit for bit.
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
}

__device__ __forceinline__ void transpose4(float (&v)[4], int lane) {
  const bool odd = (lane & 1) != 0, hi = (lane & 2) != 0;
  // pairs (0,1), (2,3) across lanes l, l ^ 1
#pragma unroll
  for (int r = 0; r < 4; r += 2) {
    const float got = dpp_xor1(odd ? v[r] : v[r + 1]);
    if (odd) v[r] = got;
    else v[r + 1] = got;
  }
  // pairs (0,2), (1,3) across lanes l, l ^ 2
  const float g0 = dpp_xor2(hi ? v[0] : v[2]);
  const float g1 = dpp_xor2(hi ? v[1] : v[3]);
  if (hi) {
    v[0] = g0;
    v[1] = g1;
  } else {
    v[2] = g0;
    v[3] = g1;
  }
}

__device__ __forceinline__ const uint8_t* wave_uniform(const uint8_t* p);
__device__ __forceinline__ uint32_t dpp_xor1_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_xor2_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}

// An accumulator element read out of its AGPR where it is used (the 4 x 4
// accumulators stay in AGPRs; letting the compiler copy them all into VGPRs
// ahead of the stores spills).
__device__ __forceinline__ float agpr_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

template <int OUT, int MT, int NT, bool W16>
__device__ __forceinline__ void store_tile_wide(const GemmParams& p, int64_t row0, int64_t col0, int lane,
                                                const v16f (&acc)[MT][NT]) {
  const int half = lane >> 5, quad = (lane & 31) >> 2, k = lane & 3;
  if constexpr (OUT == MX_OUT_F32 || !W16) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = NT > 2 ? agpr_read(acc[i][j][4 * g + e]) : acc[i][j][4 * g + e];
          transpose4(v, lane);
          const int64_t row = row0 + i * 32 + 8 * g + 4 * half + k;
          const int64_t col = col0 + j * 32 + 4 * quad;
          // non-temporal: the output streams past the L2, which keeps the operand panels the next tiles read
          if constexpr (OUT == MX_OUT_F32) {
            typedef float f4v __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(f4v{v[0], v[1], v[2], v[3]}, (f4v*)((float*)p.c + row * p.ldc + col));
          } else {
            typedef unsigned int u2v __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(u2v{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])},
                                        (u2v*)((uint16_t*)p.c + row * p.ldc + col));
          }
          // with the accumulators in AGPRs, keep each group's reads next to its store instead of letting all
          // of them be hoisted into VGPRs at once
          if constexpr (NT > 2) __builtin_amdgcn_sched_barrier(0);
        }
  } else {
    // bf16, 16 bytes per lane.  Each 4x4 block is rounded first (P0 = rows 0-1, P1 = rows 2-3 of the
    // lane's column) and transposed as 16-bit values.  Exchange 1 (lanes l ^ 2): lanes k < 2 keep
    // rows 0-1 of their own column and get rows 0-1 of column k + 2; lanes k >= 2 keep rows 2-3 and
    // get those of column k - 2, so that A holds column k & 1 and B column (k & 1) + 2, both for rows
    // (k & 2) .. +1.  Exchange 2 (lanes l ^ 1) swaps 16-bit halves: an even lane sends the high
    // halves of A and B, an odd lane the low ones; byte permutes give lane k row k, columns 0-3.
    // Then the quads of a pair (lanes l ^ 4) trade four columns: the even quad ends with eight columns
    // of the wave's left 32-column half, the odd quad with eight of the right half, for the same row.
    // One store then writes eight whole 128-byte rows.  Values are moved, never combined.
    const bool low = k < 2, odd = (k & 1) != 0, qodd = (quad & 1) != 0;
    const uint32_t sel_s = odd ? 0x05040100u : 0x07060302u;    // (A, B) -> what goes to the partner
    const uint32_t sel_q0 = odd ? 0x03020504u : 0x05040100u;   // (R, A) -> columns 0-1
    const uint32_t sel_q1 = odd ? 0x03020706u : 0x07060100u;   // (R, B) -> columns 2-3
    // the lane's byte offset from its row group's first element; the group's base is wave-uniform
    const uint32_t loff = (uint32_t)(((4 * half + k) * p.ldc + 4 * (quad & ~1) + 32 * (quad & 1)) * 2);
    auto rows4 = [&](const v16f& a4, int g, uint32_t& q0, uint32_t& q1) {
      const uint32_t p0 = pack_bf16(a4[4 * g], a4[4 * g + 1]), p1 = pack_bf16(a4[4 * g + 2], a4[4 * g + 3]);
      const uint32_t recv = dpp_xor2_u(low ? p1 : p0);
      const uint32_t a = low ? p0 : recv, b = low ? recv : p1;
      const uint32_t r = dpp_xor1_u(__builtin_amdgcn_perm(b, a, sel_s));
      q0 = __builtin_amdgcn_perm(r, a, sel_q0);
      q1 = __builtin_amdgcn_perm(r, b, sel_q1);
    };
    static_assert(NT % 2 == 0, "the wave's tile rows pair 32-column halves");
#pragma unroll
    for (int jp = 0; jp < NT; jp += 2)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int g = 0; g < 4; g += 2) {
        // rows R = 8g + 4h + k and R + 8, each in the left (j = jp) and right (j = jp + 1) half
        uint32_t a0[2], a1[2], b0[2], b1[2];
        rows4(acc[i][jp], g, a0[0], a0[1]);
        rows4(acc[i][jp + 1], g, a1[0], a1[1]);
        rows4(acc[i][jp], g + 1, b0[0], b0[1]);
        rows4(acc[i][jp + 1], g + 1, b1[0], b1[1]);
        // an even quad keeps the left half and gets its partner's left columns; an odd quad keeps the
        // right half (lanes l ^ 4; bit mode: and 0x1F, xor 4)
        uint32_t ra[2], rb[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          ra[d] = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(qodd ? a0[d] : a1[d]), 0x101F);
          rb[d] = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(qodd ? b0[d] : b1[d]), 0x101F);
        }
        typedef unsigned int u4v __attribute__((ext_vector_type(4)));
        const u4v da = qodd ? u4v{ra[0], ra[1], a1[0], a1[1]} : u4v{a0[0], a0[1], ra[0], ra[1]};
        const u4v db = qodd ? u4v{rb[0], rb[1], b1[0], b1[1]} : u4v{b0[0], b0[1], rb[0], rb[1]};
        const uint8_t* base = wave_uniform((const uint8_t*)p.c + ((row0 + i * 32 + 8 * g) * p.ldc + col0 + 32 * jp) * 2);
        __builtin_nontemporal_store(da, (__attribute__((address_space(1))) u4v*)(base + loff));
        __builtin_nontemporal_store(db, (__attribute__((address_space(1))) u4v*)(base + loff + 16 * p.ldc));
        if constexpr (NT > 2) __builtin_amdgcn_sched_barrier(0);
      }
  }
}

// Global -> LDS DMA of 16 (or 4) bytes per lane: LDS address = M0 + size*lane.
// Issued as inline asm so the compiler does not place its own conservative
// vmcnt waits for them; the kernel waits explicitly.  The instruction writes
// no VGPR and its address operand is read at issue.  An SALU write of M0
// needs one wait state before an LDS-DMA instruction reads it: the s_nop.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma16_off(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4_off(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}
// a pointer that is the same in every lane, moved to SGPRs
__device__ __forceinline__ const uint8_t* wave_uniform(const uint8_t* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ---------------------------------------------------------------------------
// Whole-tile path.  A workgroup owns a 256 x 256 block of C, as 8 waves (2
// along M x 4 along N, each 128 x 64 = 4 x 2 MFMA tiles, two waves per SIMD;
// NT = 2) or as 4 waves (2 x 2, each 128 x 128 = 4 x 4 MFMA tiles with the
// accumulators in AGPRs, one wave per SIMD; NT = 4), which reads a third
// fewer fragment bytes from LDS per MFMA.
// K advances 256 per step: every row contributes one whole 128-byte line per
// step, moved global -> LDS by DMA (global_load_lds_dwordx4) into one of two
// 68 KB stages while the MFMAs consume the other.  Within a step the four
// 64-deep K quarters are software pipelined: the fragments of quarter q+1 are
// read from LDS while the MFMAs of quarter q run (two fragment register sets),
// and the barrier of the next step sits behind the last quarter's MFMAs.
template <int NT>
constexpr int full_threads() { return NT == 2 ? 512 : 256; }
constexpr int kRowBytes = 128;            // 256 fp4 elements per row per K step
constexpr int kFullStageBytes = kBM * kRowBytes;

__device__ __forceinline__ int swz8(int row, int piece) {  // 16-byte slot within a 128-byte row
  return (piece ^ ((row >> 1) & 7)) * 16;
}

template <int NT>
struct Frags {
  uint4 a[4], b[NT];         // raw 16-byte code pieces (32 elements each)
  uint32_t sa[4], sb[NT];    // raw scale dwords (4 blocks); the lane's byte is picked at the MFMA
};

// fragments of K quarter q (64 deep) for the wave's 4 x 2 tiles.  Tile rows
// start at multiples of 32, so a lane's swizzled slot depends only on its row
// within the tile: one per-lane offset per quarter, the tiles are immediates.
// vb: whole 32-value blocks of this K step inside K (8 but in a ragged last
// step).  A lane's block in quarter q is 2q + half; past the edge its codes
// are zeros in LDS and its scale dwords may be stale or never copied, so it
// takes a stand-in scale (all bytes 127): the products stay exact zeros.
//
// E1M2 (the 8-bit operand layout): lane l takes half of each of the quarter's two blocks instead of one
// whole block, the 8 bytes at 8 * (l / 32) in both blocks' pieces, so that its converted bytes 0-15
// belong to the first block and 16-31 to the second with no exchange across the wave's halves.
template <int NT, int GRID>
__device__ __forceinline__ void load_quarter(Frags<NT>& f, const uint8_t* a, const uint8_t* b, const uint32_t* sa,
                                             const uint32_t* sb, int q, int r0, int c0, int lane, int vb,
                                             const Frags<NT>& prev) {
  const int half = lane >> 5, lrow = lane & 31;
  const int off = lrow * kRowBytes + swz8(lrow, 2 * q + half);
  const int off0 = lrow * kRowBytes + swz8(lrow, 2 * q) + 8 * half;
  const int off1 = lrow * kRowBytes + swz8(lrow, 2 * q + 1) + 8 * half;
  auto piece = [&](const uint8_t* base) {
    if constexpr (GRID == MX_GRID_E1M2 && kE1M2AsFp8) {
      const uint2 p0 = *(const uint2*)(base + off0), p1 = *(const uint2*)(base + off1);
      return uint4{p0.x, p0.y, p1.x, p1.y};
    } else {
      return *(const uint4*)(base + off);
    }
  };
  // quarters 1 and 3 use the same scale dword as 0 and 2: taken from the previous quarter's fragments
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.a[i] = piece(a + (r0 + 32 * i) * kRowBytes);
    f.sa[i] = (q & 1) ? prev.sa[i] : sa[(q >> 1) * kBM + r0 + 32 * i + lrow];
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    f.b[j] = piece(b + (c0 + 32 * j) * kRowBytes);
    f.sb[j] = (q & 1) ? prev.sb[j] : sb[(q >> 1) * kBN + c0 + 32 * j + lrow];
  }
  if (vb < 8) {
    if (2 * q + half >= vb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) f.sa[i] = 0x7F7F7F7Fu;
#pragma unroll
      for (int j = 0; j < NT; ++j) f.sb[j] = 0x7F7F7F7Fu;
    }
  }
}


// the 8 MFMAs of one quarter; OPSEL picks the scale byte pair (quarters 0,2 -> 0; 1,3 -> 2)
// Lanes 32-63 hold the odd 32-block of each 64-deep quarter: their scale is
// one byte above the even block's, so their dwords are shifted by 8.
template <int GRID, int OPSEL, int NT>
__device__ __forceinline__ void mfma_quarter(const Frags<NT>& f, v16f (&acc)[4][NT], int shift) {
  constexpr int kFmt = mfma_fmt<GRID>();
  v8i bj[NT];
  int sbj[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    bj[j] = operand_tile<GRID>(f.b[j]);
    sbj[j] = (int)(f.sb[j] >> shift);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v8i ai = operand_tile<GRID>(f.a[i]);
    const int sai = (int)(f.sa[i] >> shift);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ai, bj[j], acc[i][j], kFmt, kFmt, OPSEL, sai, OPSEL,
                                                                  sbj[j]);
  }
  // the MFMAs are side-effect free; an empty volatile asm on their results keeps
  // them at this point of the pipeline instead of being sunk past later phases
  // (the 4 x 4 accumulators live in AGPRs)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (NT == 2) asm volatile("" : "+v"(acc[i][j]));
      else asm volatile("" : "+a"(acc[i][j]));
    }
}

// First row (or column) of tile t of a dimension of size n >= 256: the last
// tile of a ragged dimension is moved back to end at n, so every copy reads
// rows inside the operand and every store lands inside C.  The rows it shares
// with the tile before are computed twice by the same MFMA sequence, and
// both writes carry the same bits.
__device__ __forceinline__ int64_t tile_origin(int t, int tile, int64_t n) {
  const int64_t o = (int64_t)t * tile;
  return o + tile <= n ? o : n - tile;
}

// Persistent: one workgroup per CU walks its tiles (round r of the XCD-grouped
// order: group r*8 + xcd, member = this workgroup's index on its XCD) as one
// continuous stream of K steps, so the DMA lookahead runs across tile
// boundaries and a tile's stores drain while the next tile computes.
struct Walk {
  int xcd, member, rounds;
};

// The problems one launch walks: one GEMM, or several that share K, the
// operand pitches, the grid and the output kind (a grouped launch).  Their
// tile groups are numbered one after the other, problem i holding groups
// gend[i-1] .. gend[i]-1 (gend[-1] = 0; entries past the last problem repeat
// its end), so a round deals groups of different problems to different XCDs
// and a problem whose tiles end part-way through a round leaves no CU idle
// while another problem has tiles left.
template <int NP>
struct GemmSet {
  GemmParams p[NP];
  TileMap tm[NP];
  int gend[NP];
};

// element i of a per-problem array, i wave-uniform (a chain of scalar selects, no indexed load)
template <typename T, int NP>
__device__ __forceinline__ T pick(const T (&v)[NP], int i) {
  T x = v[0];
#pragma unroll
  for (int j = 1; j < NP; ++j)
    if (i == j) x = v[j];
  return x;
}

template <int NP>
__device__ __forceinline__ bool round_tile(const GemmSet<NP>& s, const Walk& w, int r, int& pi, int& bm, int& bn) {
  int g = r * kXcds + w.xcd;
  pi = 0;
  if constexpr (NP == 1) {
    if (g >= s.tm[0].groups) return false;
  } else {
    if (g >= s.gend[NP - 1]) return false;
    int base = 0;
#pragma unroll
    for (int i = 0; i < NP - 1; ++i)
      if (g >= s.gend[i]) {
        pi = i + 1;
        base = s.gend[i];
      }
    g -= base;
  }
  const TileMap tm = NP == 1 ? s.tm[0] : pick(s.tm, pi);
  bm = (g % tm.groups_m) * kGroupM + w.member % kGroupM;
  bn = (g / tm.groups_m) * kGroupN + w.member / kGroupM;
  return bm < tm.tiles_m && bn < tm.tiles_n;
}

// first round >= r holding a tile for this workgroup, or w.rounds
template <int NP>
__device__ __forceinline__ int next_round(const GemmSet<NP>& s, const Walk& w, int r, int& pi, int& bm, int& bn) {
  for (; r < w.rounds; ++r)
    if (round_tile(s, w, r, pi, bm, bn)) return r;
  return w.rounds;
}

// RK: K is not a multiple of 256 (a ragged last step); a separate instance, so
// that the whole-step kernel carries none of its register cost.  NP: problems
// in the launch (1, or a grouped launch's slots); K and the operand pitches are
// the first problem's, which every problem of a grouped launch shares.
template <int GRID, int OUT, bool RK, int NT, bool W16, int NP>
__global__ void __launch_bounds__(full_threads<NT>(), 1)
gemm_full_kernel(const GemmSet<NP> s, int rounds) {
  const GemmParams& p = s.p[0];
  __shared__ __attribute__((aligned(1024))) uint8_t sA[2][kFullStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[2][kFullStageBytes];
  __shared__ __attribute__((aligned(1024))) uint32_t sSA[2][2 * kBM];    // [dword d][row]: blocks 4d..4d+3
  __shared__ __attribute__((aligned(1024))) uint32_t sSB[2][2 * kBN];

  Walk w;
  w.xcd = blockIdx.x % kXcds;
  w.member = blockIdx.x / kXcds;
  w.rounds = rounds;
  int pi, bm, bn;
  int r = next_round(s, w, 0, pi, bm, bn);
  if (r >= w.rounds) return;

  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r0 = wm * 128, c0 = wn * 32 * NT;
  const int nk = (int)((p.K + 255) / 256);
  const int vb_last = RK ? (int)((p.K % 256) / 32) : 8;   // blocks in the last step
  auto blocks_in = [&](int kt) { return RK && kt == nk - 1 ? vb_last : 8; };

  // DMA: one instruction moves 64 lanes x 16 B = 1 KB = 8 rows of 128 B; lane
  // i -> row +i/8, LDS slot i%8, which must hold global piece (i%8) ^
  // ((row>>1)&7).  Half the waves move a whole K step: waves w and w ^ 4
  // (placed on one SIMD by the round-robin wave dispatch) take alternate
  // steps, so that while one issues the step's 20 copies the other keeps that
  // SIMD's matrix core busy; all eight issuing at once after the barrier
  // stalled every SIMD behind the copies.  The
  // wave covers rows 32(w & 3) + 128h .. +31 of A and of B (h = 0, 1), and
  // the scale dwords of rows 64(w & 3) + lane of both.  Offsets are from the
  // tile's first row (operands are < 4 GiB).  Copy e = 4h + c covers rows
  // 32(w & 3) + 128h + 8c + lane/8; the slot swizzle of such a row depends on
  // c only through c & 1, so each lane keeps two offsets per operand and adds
  // the copy's wave-uniform row base.
  uint32_t la[2], lb[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = 8 * c + (lane >> 3);
    const int piece = (lane & 7) ^ ((row >> 1) & 7);
    la[c] = (uint32_t)(row * p.lda_codes + piece * 16);
    lb[c] = (uint32_t)(row * p.ldb_codes + piece * 16);
  }
  auto copy_rows = [&](int e) { return 32 * (wave & 3) + 128 * (e >> 2) + 8 * (e & 2); };
  auto offa = [&](int e) { return la[e & 1] + (uint32_t)(copy_rows(e) * p.lda_codes); };
  auto offb = [&](int e) { return lb[e & 1] + (uint32_t)(copy_rows(e) * p.ldb_codes); };
  const int srow = 64 * (wave & 3) + lane;
  const uint32_t osa = (uint32_t)(srow * p.lda_scales), osb = (uint32_t)(srow * p.ldb_scales);
  const uint32_t lA = lds_addr(&sA[0][32 * (wave & 3) * kRowBytes]), lB = lds_addr(&sB[0][32 * (wave & 3) * kRowBytes]);
  const uint32_t lSA = lds_addr(&sSA[0][64 * (wave & 3)]), lSB = lds_addr(&sSB[0][64 * (wave & 3)]);

  // DMA of K step kt of tile (tbm, tbn) of problem tpi into stage st, by the waves of parity kt % 2
  auto issue = [&](int tpi, int tbm, int tbn, int kt, int st) {
    if (NT == 2 && (wave >> 2) != (kt & 1)) return;
    const GemmParams& q = NP == 1 ? p : pick(s.p, tpi);
    const int64_t m0 = tile_origin(tbm, kBM, q.M), n0 = tile_origin(tbn, kBN, q.N);
    const uint8_t* abase = wave_uniform(q.a_codes + m0 * p.lda_codes);
    const uint8_t* bbase = wave_uniform(q.b_codes + n0 * p.ldb_codes);
    const uint8_t* sabase = wave_uniform(q.a_scales + m0 * p.lda_scales);
    const uint8_t* sbbase = wave_uniform(q.b_scales + n0 * p.ldb_scales);
    const uint32_t kb = (uint32_t)kt * kRowBytes;
    const int vb = blocks_in(kt);
    if (vb == 8) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // the copy's row base and K offset go into the wave-uniform base; the lane keeps only la / lb
          const int e = 4 * h + c;
          dma16_off(abase + copy_rows(e) * p.lda_codes + kb, la[e & 1],
                    lA + st * kFullStageBytes + (128 * h + 8 * c) * kRowBytes);
          dma16_off(bbase + copy_rows(e) * p.ldb_codes + kb, lb[e & 1],
                    lB + st * kFullStageBytes + (128 * h + 8 * c) * kRowBytes);
        }
      dma4_off(sabase, osa + 8 * kt, lSA + st * (2 * kBM * 4));
      dma4_off(sabase, osa + 8 * kt + 4, lSA + st * (2 * kBM * 4) + kBM * 4);
      dma4_off(sbbase, osb + 8 * kt, lSB + st * (2 * kBN * 4));
      dma4_off(sbbase, osb + 8 * kt + 4, lSB + st * (2 * kBN * 4) + kBN * 4);
    } else {
      // ragged last step: a lane copies its piece (block (lane % 8) ^ swizzle of its row) only if the block
      // lies inside K, and writes zeros in its place otherwise, so nothing past the row's K edge is read.  A
      // scale dword is copied if it holds a block inside K: it then ends within the scale row, whose stride
      // is a multiple of 4 bytes.  Blocks past the edge take a stand-in scale when read (load_quarter).
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int gp = (lane & 7) ^ (4 * (c & 1) + (lane >> 4));
          const int rowoff = (32 * (wave & 3) + 128 * h + 8 * c) * kRowBytes + 16 * lane;
          if (gp < vb) {
            dma16_off(abase, offa(4 * h + c) + kb, lA + st * kFullStageBytes + (128 * h + 8 * c) * kRowBytes);
            dma16_off(bbase, offb(4 * h + c) + kb, lB + st * kFullStageBytes + (128 * h + 8 * c) * kRowBytes);
          } else {
            *(uint4*)(&sA[st][rowoff]) = uint4{0u, 0u, 0u, 0u};
            *(uint4*)(&sB[st][rowoff]) = uint4{0u, 0u, 0u, 0u};
          }
        }
      dma4_off(sabase, osa + 8 * kt, lSA + st * (2 * kBM * 4));
      dma4_off(sbbase, osb + 8 * kt, lSB + st * (2 * kBN * 4));
      if (vb > 4) {
        dma4_off(sabase, osa + 8 * kt + 4, lSA + st * (2 * kBM * 4) + kBM * 4);
        dma4_off(sbbase, osb + 8 * kt + 4, lSB + st * (2 * kBN * 4) + kBN * 4);
      }
    }
  };

  v16f acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // the tile after the current one, and the DMA cursor two K steps ahead
  int npi = 0, nbm = 0, nbn = 0;
  int rn = next_round(s, w, r + 1, npi, nbm, nbn);
  Frags<NT> f0, f1;
  const int shift = 8 * (lane >> 5);
  issue(pi, bm, bn, 0, 0);
  // the waits and the barrier in one asm statement: its memory clobber keeps the compiler's LDS
  // accesses on their side of the barrier (the barrier builtin alone is not a memory operation)
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  if (nk > 1) issue(pi, bm, bn, 1, 1);
  else if (rn < w.rounds) issue(npi, nbm, nbn, 0, 1);
  load_quarter<NT, GRID>(f0, sA[0], sB[0], sSA[0], sSB[0], 0, r0, c0, lane, blocks_in(0), f1);
  int st = 0;
  for (;;) {
    for (int kt = 0; kt < nk; ++kt) {
      const uint8_t* a = sA[st];
      const uint8_t* b = sB[st];
      const uint32_t* sa = sSA[st];
      const uint32_t* sb = sSB[st];
      // sched_barrier keeps each phase where it is written: without it the
      // scheduler hoists every quarter's reads to the top and runs out of VGPRs
      const int vb = blocks_in(kt);
      load_quarter<NT, GRID>(f1, a, b, sa, sb, 1, r0, c0, lane, vb, f0);
      __builtin_amdgcn_sched_barrier(0);
      mfma_quarter<GRID, 0, NT>(f0, acc, shift);
      __builtin_amdgcn_sched_barrier(0);
      load_quarter<NT, GRID>(f0, a, b, sa, sb, 2, r0, c0, lane, vb, f1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_quarter<GRID, 2, NT>(f1, acc, shift);
      __builtin_amdgcn_sched_barrier(0);
      load_quarter<NT, GRID>(f1, a, b, sa, sb, 3, r0, c0, lane, vb, f0);
      __builtin_amdgcn_sched_barrier(0);
      mfma_quarter<GRID, 0, NT>(f0, acc, shift);
      __builtin_amdgcn_sched_barrier(0);
      const bool more = kt + 1 < nk || rn < w.rounds;
      if (more) {
        // the next step's stage has landed for this wave; every wave has read
        // its last fragments of this stage; then refill it two steps ahead
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (kt + 2 < nk) issue(pi, bm, bn, kt + 2, st);
        else if (rn < w.rounds && kt + 2 - nk < nk) issue(npi, nbm, nbn, kt + 2 - nk, st);
        st ^= 1;
        load_quarter<NT, GRID>(f0, sA[st], sB[st], sSA[st], sSB[st], 0, r0, c0, lane, blocks_in(kt + 1 < nk ? kt + 1 : 0), f1);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma_quarter<GRID, 2, NT>(f1, acc, shift);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NP == 1) {
      store_tile_wide<OUT, 4, NT, W16>(p, tile_origin(bm, kBM, p.M) + r0, tile_origin(bn, kBN, p.N) + c0, lane, acc);
    } else {
      const GemmParams q = pick(s.p, pi);
      store_tile_wide<OUT, 4, NT, W16>(q, tile_origin(bm, kBM, q.M) + r0, tile_origin(bn, kBN, q.N) + c0, lane, acc);
    }
    if (rn >= w.rounds) break;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    r = rn;
    pi = npi;
    bm = nbm;
    bn = nbn;
    rn = next_round(s, w, r + 1, npi, nbm, nbn);
  }
}

// Any shape (ragged M, N; K % 32 == 0): bounds-checked loads through registers.
template <int GRID, int OUT>
__global__ void __launch_bounds__(kGemmThreads, 1)
gemm_general_kernel(const GemmParams p, const TileMap tm) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[kBM * kBKBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kBN * kBKBytes];
  __shared__ uint32_t sSA[kBM], sSB[kBN];

  int bm, bn;
  if (!map_tile(tm, bm, bn)) return;
  const int64_t m0 = (int64_t)bm * kBM, n0 = (int64_t)bn * kBN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t kbytes = p.K / 2, kblocks = p.K / 32;
  const int nk = (int)((p.K + 127) / 128);
  const int pc = t & 3;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int kt = 0; kt < nk; ++kt) {
    const int64_t kb = (int64_t)kt * kBKBytes + pc * 16;
    uint4 ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (t >> 2) + 64 * i;
      ra[i] = (m0 + r < p.M && kb < kbytes) ? *(const uint4*)(p.a_codes + (m0 + r) * p.lda_codes + kb)
                                             : uint4{0u, 0u, 0u, 0u};
      rb[i] = (n0 + r < p.N && kb < kbytes) ? *(const uint4*)(p.b_codes + (n0 + r) * p.ldb_codes + kb)
                                             : uint4{0u, 0u, 0u, 0u};
    }
    uint32_t xa = 0u, xb = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t kblk = (int64_t)kt * 4 + b;
      if (kblk < kblocks) {
        if (m0 + t < p.M) xa |= (uint32_t)p.a_scales[(m0 + t) * p.lda_scales + kblk] << (8 * b);
        if (n0 + t < p.N) xb |= (uint32_t)p.b_scales[(n0 + t) * p.ldb_scales + kblk] << (8 * b);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (t >> 2) + 64 * i;
      *(uint4*)(&sA[r * kBKBytes + swz(r, pc)]) = ra[i];
      *(uint4*)(&sB[r * kBKBytes + swz(r, pc)]) = rb[i];
    }
    sSA[t] = xa;
    sSB[t] = xb;
    __syncthreads();
    mma_step<GRID, 4, 4>(sA, sB, sSA, sSB, wm * 128, wn * 128, lane, acc);
  }
  store_tile<OUT, true, 4, 4>(p, m0 + wm * 128, n0 + wn * 128, lane, acc);
}

// MFMA tiles per wave along N on the whole-tile path: 2 (eight waves of 128 x 64) or 4 (four waves of
// 128 x 128).  Four waves read a third fewer fragment bytes but leave one wave per SIMD to hide every
// barrier and copy issue; on the Llama shapes they ran 5-18% slower, with the same output bits.
constexpr int kWaveTileN = 2;

// whole-tile kernel instance for a grid, output kind, K and output row form
template <int GRID, int OUT, int NP>
static void launch_full(const GemmSet<NP>& set, int groups, bool wide16, hipStream_t s) {
  // one workgroup per CU: 8 XCDs x 32 members; round r deals group r*8+xcd
  const int rounds = (groups + kXcds - 1) / kXcds;
  constexpr int NT = kWaveTileN;
  const dim3 g(kXcds * kGroupM * kGroupN), b(full_threads<NT>());
  const bool rk = set.p[0].K % 256 != 0;
  // fp32 rows are always written 16 bytes per lane, bf16 rows when wide16 holds (a grouped launch is
  // made only then)
  constexpr bool kNarrow = OUT == MX_OUT_BF16 && NP == 1;
  if (!kNarrow || wide16) {
    if (!rk) hipLaunchKernelGGL((gemm_full_kernel<GRID, OUT, false, NT, true, NP>), g, b, 0, s, set, rounds);
    else hipLaunchKernelGGL((gemm_full_kernel<GRID, OUT, true, NT, true, NP>), g, b, 0, s, set, rounds);
  } else if constexpr (kNarrow) {
    if (!rk) hipLaunchKernelGGL((gemm_full_kernel<GRID, OUT, false, NT, false, NP>), g, b, 0, s, set, rounds);
    else hipLaunchKernelGGL((gemm_full_kernel<GRID, OUT, true, NT, false, NP>), g, b, 0, s, set, rounds);
  }
}

static TileMap tile_map(const GemmParams& p) {
  TileMap tm;
  tm.tiles_m = (int)((p.M + kBM - 1) / kBM);
  tm.tiles_n = (int)((p.N + kBN - 1) / kBN);
  tm.groups_m = (tm.tiles_m + kGroupM - 1) / kGroupM;
  const int groups_n = (tm.tiles_n + kGroupN - 1) / kGroupN;
  tm.groups = tm.groups_m * groups_n;
  return tm;
}

static bool full_path(const GemmParams& p, int out_kind) {
  return gemm_full_path(p.M, p.N, p.K, (uintptr_t)p.a_scales, (uintptr_t)p.b_scales, p.lda_codes, p.ldb_codes,
                        p.lda_scales, p.ldb_scales, (uintptr_t)p.c, p.ldc, out_kind == MX_OUT_F32);
}

// bf16 rows written 16 bytes per lane need 16-byte aligned rows and tile origins
static bool wide16_rows(const GemmParams& p) {
  return p.ldc % 8 == 0 && p.N % 8 == 0 && (uintptr_t)p.c % 16 == 0;
}

hipError_t launch_gemm(const GemmParams& p, int grid_kind, int out_kind, hipStream_t s) {
  GemmSet<1> set;
  set.p[0] = p;
  set.tm[0] = tile_map(p);
  set.gend[0] = set.tm[0].groups;
  const TileMap& tm = set.tm[0];
  if (full_path(p, out_kind)) {
    const bool w16 = wide16_rows(p);
    if (grid_kind == MX_GRID_E2M1) {
      if (out_kind == MX_OUT_F32) launch_full<MX_GRID_E2M1, MX_OUT_F32>(set, tm.groups, w16, s);
      else launch_full<MX_GRID_E2M1, MX_OUT_BF16>(set, tm.groups, w16, s);
    } else {
      if (out_kind == MX_OUT_F32) launch_full<MX_GRID_E1M2, MX_OUT_F32>(set, tm.groups, w16, s);
      else launch_full<MX_GRID_E1M2, MX_OUT_BF16>(set, tm.groups, w16, s);
    }
  } else {
    const int wgs = ((tm.groups + kXcds - 1) / kXcds) * kXcds * kGroupM * kGroupN;
    const dim3 g((unsigned)wgs), b(kGemmThreads);
    if (grid_kind == MX_GRID_E2M1) {
      if (out_kind == MX_OUT_F32) hipLaunchKernelGGL((gemm_general_kernel<MX_GRID_E2M1, MX_OUT_F32>), g, b, 0, s, p, tm);
      else hipLaunchKernelGGL((gemm_general_kernel<MX_GRID_E2M1, MX_OUT_BF16>), g, b, 0, s, p, tm);
    } else {
      if (out_kind == MX_OUT_F32) hipLaunchKernelGGL((gemm_general_kernel<MX_GRID_E1M2, MX_OUT_F32>), g, b, 0, s, p, tm);
      else hipLaunchKernelGGL((gemm_general_kernel<MX_GRID_E1M2, MX_OUT_BF16>), g, b, 0, s, p, tm);
    }
  }
  return hipGetLastError();
}

// Several GEMMs in one persistent launch when they all take the whole-tile path with one K, one set of
// operand pitches and (bf16) 16-byte rows; otherwise each runs as its own launch, with the same results.
hipError_t launch_gemm_grouped(const GemmParams* ps, int count, int grid_kind, int out_kind, hipStream_t s) {
  bool together = count > 1 && count <= kMaxGroup;
  for (int i = 0; together && i < count; ++i) {
    const GemmParams& p = ps[i];
    together = full_path(p, out_kind) && (out_kind == MX_OUT_F32 || wide16_rows(p)) && p.K == ps[0].K &&
               p.lda_codes == ps[0].lda_codes && p.ldb_codes == ps[0].ldb_codes &&
               p.lda_scales == ps[0].lda_scales && p.ldb_scales == ps[0].ldb_scales;
  }
  if (!together) {
    for (int i = 0; i < count; ++i) {
      const hipError_t e = launch_gemm(ps[i], grid_kind, out_kind, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  GemmSet<kMaxGroup> set;
  int groups = 0;
  for (int i = 0; i < kMaxGroup; ++i) {
    set.p[i] = ps[i < count ? i : count - 1];
    set.tm[i] = tile_map(set.p[i]);
    if (i < count) groups += set.tm[i].groups;
    set.gend[i] = groups;
  }
  if (grid_kind == MX_GRID_E2M1) {
    if (out_kind == MX_OUT_F32) launch_full<MX_GRID_E2M1, MX_OUT_F32>(set, groups, true, s);
    else launch_full<MX_GRID_E2M1, MX_OUT_BF16>(set, groups, true, s);
  } else {
    if (out_kind == MX_OUT_F32) launch_full<MX_GRID_E1M2, MX_OUT_F32>(set, groups, true, s);
    else launch_full<MX_GRID_E1M2, MX_OUT_BF16>(set, groups, true, s);
  }
  return hipGetLastError();
}

}  // namespace mx
