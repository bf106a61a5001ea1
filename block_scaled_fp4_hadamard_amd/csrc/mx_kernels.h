// Internal interface between the C ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/mxfp4.h"

namespace mx {

struct QuantParams {
  const uint16_t* x;
  int64_t rows, cols, ld_x;
  uint8_t* row_codes;
  int64_t ld_row_codes;
  uint8_t* row_scales;
  int64_t ld_row_scales;
  uint8_t* col_codes;
  int64_t ld_col_codes;
  uint8_t* col_scales;
  int64_t ld_col_scales;
  uint64_t seed;
  uint32_t sign_mask;   // bit j set: input j of every Hadamard chunk is negated
  int32_t n_row_tiles, n_col_tiles, n_row_groups;   // filled by launch_quant
  bool fast_ok;         // output pitches allow 32-bit offsets within a tile (filled by launch_quant)
};

hipError_t launch_quant(QuantParams p, int had_n, bool rht, int grid_kind, int round, bool do_row, bool do_col,
                        hipStream_t s);

// The rotation alone: float32 y of every 32-value block along one axis
// (column axis: y holds the transpose, y[c][r]).
struct RotateParams {
  const uint16_t* x;
  int64_t rows, cols, ld_x;
  float* y;
  int64_t ld_y;         // floats between lines of y
  bool col;
  uint32_t sign_mask;   // bit j set: input j of every Hadamard chunk is negated
};

hipError_t launch_rotate(RotateParams p, int had_n, bool rht, hipStream_t s);

// The MX cast of float32 lines (block 32), stochastic-rounding stream `stream`.
struct QuantF32Params {
  const float* y;
  int64_t lines, len, ld_y;
  uint8_t* codes;
  int64_t ld_codes;
  uint8_t* scales;
  int64_t ld_scales;
  uint64_t seed;
  uint32_t stream;
};

hipError_t launch_quant_f32(const QuantF32Params& p, int grid_kind, int round, hipStream_t s);

// OsciReset on float32 master weights and their row-wise MX quantization.
struct OsciParams {
  float* w;
  int64_t rows, cols, ld_w;
  const uint8_t* codes;
  int64_t ld_codes;
  const uint8_t* scales;
  int64_t ld_scales;
  float* w_prev;
  float* q_prev;
  float* dist_m;
  float* dist_q;
  int64_t ld_s;          // floats between rows of the four state arrays
  int mode;              // mx_osci_mode
  float threshold;
  unsigned long long* resets;   // optional count of the elements reset (added to)
};

hipError_t launch_osci(const OsciParams& p, int grid_kind, hipStream_t s);

struct GemmParams {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int64_t lda_codes, lda_scales, ldb_codes, ldb_scales;
  int64_t M, N, K;
  void* c;
  int64_t ldc;
};

hipError_t launch_gemm(const GemmParams& p, int grid_kind, int out_kind, hipStream_t s);
// up to kMaxGroup GEMMs of one K: one launch when they can share it, else one launch each
constexpr int kMaxGroup = MX_GEMM_GROUP_MAX;
hipError_t launch_gemm_grouped(const GemmParams* ps, int count, int grid_kind, int out_kind, hipStream_t s);

struct MxNormParams {
  const uint16_t* x;
  int64_t rows, cols, ld_x;
  uint8_t* codes;
  int64_t ld_codes;
  uint8_t* scales;
  int64_t ld_scales;
  float* rho;
  float c;
  uint64_t seed;
};

hipError_t launch_mxnorm(const MxNormParams& p, int power, int grid_kind, int round, hipStream_t s);

struct QuantStatsParams {
  const uint16_t* x;
  int64_t rows, cols, ld_x;
  const uint8_t* codes;
  int64_t ld_codes;
  const uint8_t* scales;
  int64_t ld_scales;
  int axis_col;         // 0: row-wise output (blocks along rows), 1: column-wise
  int grid;
  uint32_t sign_mask;   // bit j set: input j of every Hadamard chunk is negated
  mx_quant_stats_t* out;
};

hipError_t launch_quant_stats(const QuantStatsParams& p, int had_n, hipStream_t s);

// 16-value blocks along one axis: MX E8M0 scales, or the double-block layout
// (E4M3 per 16 values in `scales`, float32 per 128 values in `outer`)
struct Block16Params {
  const uint16_t* x;
  int64_t rows, cols, ld_x;
  uint8_t* codes;
  int64_t ld_codes;
  uint8_t* scales;
  int64_t ld_scales;
  float* outer;
  int64_t ld_outer;
  uint64_t seed;
};

hipError_t launch_block16(const Block16Params& p, bool double_block, int grid_kind, int round, bool col,
                          hipStream_t s);

}  // namespace mx
