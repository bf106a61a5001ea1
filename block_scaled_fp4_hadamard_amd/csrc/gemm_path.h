// Which GEMM kernel a shape takes: host-only logic, no HIP types, so that it
// can be compiled and checked on a machine without a GPU.
#pragma once
#include <stdint.h>

namespace mx {

constexpr int64_t kFullTile = 256;   // rows and columns of C per workgroup on the whole-tile path

// The whole-tile (LDS-copy) kernel needs:
//  - at least one whole 256 x 256 tile along M and N (a ragged last tile is
//    moved back to end at the edge) and at least two 256-deep K steps (a
//    ragged last step is zero-filled);
//  - N % 4 == 0, 4-byte aligned scale rows with a pitch that is a multiple of
//    4, ldc % 4 == 0, and C aligned for its 16-byte (fp32) or 8-byte (bf16)
//    stores;
//  - every copy offset within 32 bits: a copy addresses a tile's operand
//    bytes as a 32-bit offset from the tile's first row, at most
//    255 * ld_codes + K / 2 for codes and 255 * ld_scales + K / 32 for scales.
// Every other shape runs the bounds-checked kernel, whose addresses are 64-bit.
inline bool gemm_full_path(int64_t M, int64_t N, int64_t K, uintptr_t a_scales, uintptr_t b_scales,
                           int64_t lda_codes, int64_t ldb_codes, int64_t lda_scales, int64_t ldb_scales,
                           uintptr_t c, int64_t ldc, bool out_f32) {
  const int64_t lim = int64_t(1) << 32;
  const bool offsets32 = (kFullTile - 1) * lda_codes + K / 2 < lim && (kFullTile - 1) * ldb_codes + K / 2 < lim &&
                         (kFullTile - 1) * lda_scales + K / 32 < lim && (kFullTile - 1) * ldb_scales + K / 32 < lim;
  return M >= kFullTile && N >= kFullTile && N % 4 == 0 && K >= 2 * kFullTile && a_scales % 4 == 0 &&
         b_scales % 4 == 0 && lda_scales % 4 == 0 && ldb_scales % 4 == 0 && ldc % 4 == 0 &&
         c % (out_f32 ? 16u : 8u) == 0 && offsets32;
}

}  // namespace mx
