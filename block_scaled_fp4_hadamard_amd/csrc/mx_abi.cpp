// C ABI of the MX quantizer and GEMM: argument validation, the random sign
// vector of the randomized Hadamard rotation, and the kernel launches.
// Validation happens before any HIP call, so argument errors never touch the
// device.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mx_kernels.h"

namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u, kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;

// Host Philox4x32-10, word 0 only: the sign vector of the randomized rotation
// is word 0 of the draw with counter (0, 0, 2, 0) under key had_seed.
uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c0 * kM0, p1 = (uint64_t)c2 * kM1;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += kW0;
    k1 += kW1;
  }
  return c0;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

mx_status check_qtensor(const mx_qtensor* q, int64_t lines, int64_t k, int32_t block) {
  if (q == nullptr || q->codes == nullptr || q->scales == nullptr) return MX_ERR_INVALID;
  // the 32-value kernels store 16 code bytes at a time, the 16-value kernel 8
  const int64_t step = block == 16 ? 8 : 16;
  if (((uintptr_t)q->codes % (uintptr_t)step) != 0 || q->ld_codes % step != 0) return MX_ERR_INVALID;
  if (q->ld_codes < k / 2 || q->ld_scales < k / block) return MX_ERR_INVALID;
  if (lines > 1 && (q->ld_codes <= 0 || q->ld_scales <= 0)) return MX_ERR_INVALID;
  return MX_OK;
}

mx_status quantize_impl(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t block, int grid,
                        int round, int axis, uint64_t seed, int had_n, int had_kind, uint64_t had_seed,
                        const mx_qtensor* row_out, const mx_qtensor* col_out, void* stream) {
  if (rows < 0 || cols < 0) return MX_ERR_INVALID;
  if (grid != MX_GRID_E2M1 && grid != MX_GRID_E1M2) return MX_ERR_INVALID;
  if (round != MX_ROUND_RTNE && round != MX_ROUND_SR) return MX_ERR_INVALID;
  if (axis != MX_AXIS_ROW && axis != MX_AXIS_COL && axis != MX_AXIS_BOTH) return MX_ERR_INVALID;
  if (had_kind != MX_HAD_NONE && had_kind != MX_HAD_DET && had_kind != MX_HAD_RAND) return MX_ERR_INVALID;
  if (had_kind == MX_HAD_NONE) had_n = 0;
  else if (had_n != 16 && had_n != 32) return MX_ERR_INVALID;
  if (block != 16 && block != 32) return MX_ERR_INVALID;
  if (had_n > block) return MX_ERR_INVALID;
  const bool do_row = (axis & MX_AXIS_ROW) != 0, do_col = (axis & MX_AXIS_COL) != 0;
  if (rows == 0 || cols == 0) return MX_OK;
  if (x == nullptr || !aligned16(x)) return MX_ERR_INVALID;
  if (ld_x < cols || ld_x % 8 != 0 || cols % 8 != 0 || ld_x >= (int64_t(1) << 25)) return MX_ERR_INVALID;
  if (do_row) {
    if (cols % block != 0) return MX_ERR_INVALID;
    mx_status s = check_qtensor(row_out, rows, cols, block);
    if (s != MX_OK) return s;
  }
  if (do_col) {
    if (rows % block != 0) return MX_ERR_INVALID;
    mx_status s = check_qtensor(col_out, cols, rows, block);
    if (s != MX_OK) return s;
  }
  if (block == 16) {
    // 16-value MX blocks: a separate kernel, no rotation
    if (had_n != 0) return MX_ERR_UNSUPPORTED;
    for (int a = 0; a < 2; ++a) {
      const bool col = a == 1;
      if (col ? !do_col : !do_row) continue;
      const mx_qtensor* q = col ? col_out : row_out;
      mx::Block16Params b{};
      b.x = x;
      b.rows = rows;
      b.cols = cols;
      b.ld_x = ld_x;
      b.codes = q->codes;
      b.ld_codes = q->ld_codes;
      b.scales = q->scales;
      b.ld_scales = q->ld_scales;
      b.seed = seed;
      if (mx::launch_block16(b, false, grid, round, col, (hipStream_t)stream) != hipSuccess) return MX_ERR_DEVICE;
    }
    return MX_OK;
  }
  if (block != 32) return MX_ERR_UNSUPPORTED;
  mx::QuantParams p{};
  p.x = x;
  p.rows = rows;
  p.cols = cols;
  p.ld_x = ld_x;
  if (do_row) {
    p.row_codes = row_out->codes;
    p.ld_row_codes = row_out->ld_codes;
    p.row_scales = row_out->scales;
    p.ld_row_scales = row_out->ld_scales;
  }
  if (do_col) {
    p.col_codes = col_out->codes;
    p.ld_col_codes = col_out->ld_codes;
    p.col_scales = col_out->scales;
    p.ld_col_scales = col_out->ld_scales;
  }
  p.seed = seed;
  p.sign_mask = 0u;
  const bool rht = had_kind == MX_HAD_RAND;
  if (rht) {
    const uint32_t w0 = philox_word0(0u, 0u, 2u, 0u, (uint32_t)had_seed, (uint32_t)(had_seed >> 32));
    p.sign_mask = had_n == 32 ? w0 : (w0 & 0xFFFFu);
  }
  hipError_t e = mx::launch_quant(p, had_n, rht, grid, round, do_row, do_col, (hipStream_t)stream);
  return e == hipSuccess ? MX_OK : MX_ERR_DEVICE;
}

// mx_gemm's argument checks; on MX_OK with M, N > 0, p holds the problem
mx_status gemm_args(const mx_qtensor* a, const mx_qtensor* b, int64_t M, int64_t N, int64_t K, int grid,
                    int32_t block, void* c, int64_t ldc, int out, mx::GemmParams& p) {
  if (M < 0 || N < 0 || K <= 0) return MX_ERR_INVALID;
  if (grid != MX_GRID_E2M1 && grid != MX_GRID_E1M2) return MX_ERR_INVALID;
  if (out != MX_OUT_F32 && out != MX_OUT_BF16) return MX_ERR_INVALID;
  if (block != 16 && block != 32) return MX_ERR_INVALID;
  if (K % block != 0) return MX_ERR_INVALID;
  if (M == 0 || N == 0) return MX_OK;
  mx_status s = check_qtensor(a, M, K, block);
  if (s != MX_OK) return s;
  s = check_qtensor(b, N, K, block);
  if (s != MX_OK) return s;
  const uintptr_t esize = out == MX_OUT_F32 ? 4u : 2u;
  if (c == nullptr || ((uintptr_t)c % esize) != 0 || ldc < N) return MX_ERR_INVALID;
  if (block != 32) return MX_ERR_UNSUPPORTED;
  p = mx::GemmParams{};
  p.a_codes = a->codes;
  p.a_scales = a->scales;
  p.b_codes = b->codes;
  p.b_scales = b->scales;
  p.lda_codes = a->ld_codes;
  p.lda_scales = a->ld_scales;
  p.ldb_codes = b->ld_codes;
  p.ldb_scales = b->ld_scales;
  p.M = M;
  p.N = N;
  p.K = K;
  p.c = c;
  p.ldc = ldc;
  return MX_OK;
}

}  // namespace

extern "C" {

mx_status mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t block, mx_grid grid,
                      mx_round round, mx_axis axis, uint64_t seed, const mx_qtensor* row_out,
                      const mx_qtensor* col_out, void* hip_stream) {
  return quantize_impl(x, rows, cols, ld_x, block, grid, round, axis, seed, 0, MX_HAD_NONE, 0, row_out, col_out,
                       hip_stream);
}

mx_status mx_hadamard_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t block,
                               mx_grid grid, mx_round round, mx_axis axis, uint64_t seed, int32_t had_n,
                               mx_had had_kind, uint64_t had_seed, const mx_qtensor* row_out,
                               const mx_qtensor* col_out, void* hip_stream) {
  if (had_kind == MX_HAD_NONE) return MX_ERR_INVALID;
  return quantize_impl(x, rows, cols, ld_x, block, grid, round, axis, seed, had_n, had_kind, had_seed, row_out,
                       col_out, hip_stream);
}

mx_status mx_gemm(const mx_qtensor* a, const mx_qtensor* b, int64_t M, int64_t N, int64_t K, mx_grid grid,
                  int32_t block, void* c, int64_t ldc, mx_out out, void* hip_stream) {
  mx::GemmParams p{};
  const mx_status s = gemm_args(a, b, M, N, K, grid, block, c, ldc, out, p);
  if (s != MX_OK || M == 0 || N == 0) return s;
  hipError_t e = mx::launch_gemm(p, grid, out, (hipStream_t)hip_stream);
  return e == hipSuccess ? MX_OK : MX_ERR_DEVICE;
}

mx_status mx_gemm_grouped(const mx_gemm_problem* problems, int32_t count, int64_t K, mx_grid grid, int32_t block,
                          mx_out out, void* hip_stream) {
  if (problems == nullptr || count < 1 || count > MX_GEMM_GROUP_MAX) return MX_ERR_INVALID;
  mx::GemmParams ps[MX_GEMM_GROUP_MAX];
  int n = 0;
  for (int i = 0; i < count; ++i) {
    const mx_gemm_problem& q = problems[i];
    const mx_status s = gemm_args(q.a, q.b, q.M, q.N, K, grid, block, q.c, q.ldc, out, ps[n]);
    if (s != MX_OK) return s;
    if (q.M > 0 && q.N > 0) ++n;
  }
  if (n == 0) return MX_OK;
  hipError_t e = mx::launch_gemm_grouped(ps, n, grid, out, (hipStream_t)hip_stream);
  return e == hipSuccess ? MX_OK : MX_ERR_DEVICE;
}

mx_status mx_mxnorm_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t power, float c,
                             mx_grid grid, mx_round round, uint64_t seed, const mx_qtensor* out, float* rho,
                             void* hip_stream) {
  if (rows < 0 || cols < 0) return MX_ERR_INVALID;
  if (power != 1 && power != 2) return MX_ERR_INVALID;
  if (!(c > 0.0f) || c > 3.0e38f) return MX_ERR_INVALID;          // rejects NaN, non-positive and infinite c
  if (grid != MX_GRID_E2M1 && grid != MX_GRID_E1M2) return MX_ERR_INVALID;
  if (round != MX_ROUND_RTNE && round != MX_ROUND_SR) return MX_ERR_INVALID;
  if (rows == 0 || cols == 0) return MX_OK;
  if (cols % 32 != 0 || cols > 65536) return MX_ERR_INVALID;
  if (x == nullptr || !aligned16(x)) return MX_ERR_INVALID;
  if (ld_x < cols || ld_x % 8 != 0) return MX_ERR_INVALID;
  mx_status s = check_qtensor(out, rows, cols, 32);
  if (s != MX_OK) return s;
  if (rho == nullptr || ((uintptr_t)rho & 3u) != 0) return MX_ERR_INVALID;
  mx::MxNormParams p{};
  p.x = x;
  p.rows = rows;
  p.cols = cols;
  p.ld_x = ld_x;
  p.codes = out->codes;
  p.ld_codes = out->ld_codes;
  p.scales = out->scales;
  p.ld_scales = out->ld_scales;
  p.rho = rho;
  p.c = c;
  p.seed = seed;
  hipError_t e = mx::launch_mxnorm(p, power, grid, round, (hipStream_t)hip_stream);
  return e == hipSuccess ? MX_OK : MX_ERR_DEVICE;
}

mx_status mx_quant_stats(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, mx_axis axis, mx_grid grid,
                         int32_t had_n, mx_had had_kind, uint64_t had_seed, const mx_qtensor* q,
                         mx_quant_stats_t* stats, void* hip_stream) {
  if (rows < 0 || cols < 0) return MX_ERR_INVALID;
  if (axis != MX_AXIS_ROW && axis != MX_AXIS_COL) return MX_ERR_INVALID;
  if (grid != MX_GRID_E2M1 && grid != MX_GRID_E1M2) return MX_ERR_INVALID;
  if (had_kind != MX_HAD_NONE && had_kind != MX_HAD_DET && had_kind != MX_HAD_RAND) return MX_ERR_INVALID;
  if (had_kind == MX_HAD_NONE) had_n = 0;
  else if (had_n != 16 && had_n != 32) return MX_ERR_INVALID;
  if (stats == nullptr || ((uintptr_t)stats & 7u) != 0) return MX_ERR_INVALID;
  if (rows == 0 || cols == 0) return MX_OK;
  if (x == nullptr || ((uintptr_t)x & 1u) != 0 || ld_x < cols) return MX_ERR_INVALID;
  const bool col = axis == MX_AXIS_COL;
  const int64_t lines = col ? cols : rows, len = col ? rows : cols;
  if (len % 32 != 0) return MX_ERR_INVALID;
  mx_status s = check_qtensor(q, lines, len, 32);
  if (s != MX_OK) return s;
  mx::QuantStatsParams p{};
  p.x = x;
  p.rows = rows;
  p.cols = cols;
  p.ld_x = ld_x;
  p.codes = q->codes;
  p.ld_codes = q->ld_codes;
  p.scales = q->scales;
  p.ld_scales = q->ld_scales;
  p.axis_col = col ? 1 : 0;
  p.grid = grid;
  p.sign_mask = 0u;
  if (had_kind == MX_HAD_RAND) {
    const uint32_t w0 = philox_word0(0u, 0u, 2u, 0u, (uint32_t)had_seed, (uint32_t)(had_seed >> 32));
    p.sign_mask = had_n == 32 ? w0 : (w0 & 0xFFFFu);
  }
  p.out = stats;
  hipError_t e = mx::launch_quant_stats(p, had_n, (hipStream_t)hip_stream);
  return e == hipSuccess ? MX_OK : MX_ERR_DEVICE;
}

mx_status mx_nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, mx_round round,
                            mx_axis axis, uint64_t seed, const mx_nvfp4_tensor* row_out,
                            const mx_nvfp4_tensor* col_out, void* hip_stream) {
  if (rows < 0 || cols < 0) return MX_ERR_INVALID;
  if (round != MX_ROUND_RTNE && round != MX_ROUND_SR) return MX_ERR_INVALID;
  if (axis != MX_AXIS_ROW && axis != MX_AXIS_COL && axis != MX_AXIS_BOTH) return MX_ERR_INVALID;
  if (rows == 0 || cols == 0) return MX_OK;
  if (x == nullptr || !aligned16(x)) return MX_ERR_INVALID;
  if (ld_x < cols || ld_x % 8 != 0 || cols % 8 != 0) return MX_ERR_INVALID;
  const bool do_row = (axis & MX_AXIS_ROW) != 0, do_col = (axis & MX_AXIS_COL) != 0;
  for (int a = 0; a < 2; ++a) {
    const bool col = a == 1;
    if (col ? !do_col : !do_row) continue;
    const mx_nvfp4_tensor* q = col ? col_out : row_out;
    const int64_t lines = col ? cols : rows, len = col ? rows : cols;
    if (len % 128 != 0) return MX_ERR_INVALID;
    if (q == nullptr || q->codes == nullptr || q->inner == nullptr || q->outer == nullptr) return MX_ERR_INVALID;
    if (!aligned16(q->codes) || q->ld_codes % 16 != 0 || q->ld_codes < len / 2) return MX_ERR_INVALID;
    if (q->ld_inner < len / 16 || q->ld_outer < len / 128 || ((uintptr_t)q->outer & 3u) != 0) return MX_ERR_INVALID;
    if (lines > 1 && (q->ld_inner <= 0 || q->ld_outer <= 0)) return MX_ERR_INVALID;
  }
  for (int a = 0; a < 2; ++a) {
    const bool col = a == 1;
    if (col ? !do_col : !do_row) continue;
    const mx_nvfp4_tensor* q = col ? col_out : row_out;
    mx::Block16Params b{};
    b.x = x;
    b.rows = rows;
    b.cols = cols;
    b.ld_x = ld_x;
    b.codes = q->codes;
    b.ld_codes = q->ld_codes;
    b.scales = q->inner;
    b.ld_scales = q->ld_inner;
    b.outer = q->outer;
    b.ld_outer = q->ld_outer;
    b.seed = seed;
    if (mx::launch_block16(b, true, MX_GRID_E2M1, round, col, (hipStream_t)hip_stream) != hipSuccess)
      return MX_ERR_DEVICE;
  }
  return MX_OK;
}

mx_status mx_hadamard_rotate(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t had_n,
                             mx_had had_kind, uint64_t had_seed, mx_axis axis, float* y, int64_t ld_y,
                             void* hip_stream) {
  if (rows < 0 || cols < 0) return MX_ERR_INVALID;
  if (had_kind != MX_HAD_DET && had_kind != MX_HAD_RAND) return MX_ERR_INVALID;
  if (had_n != 16 && had_n != 32) return MX_ERR_INVALID;
  if (axis != MX_AXIS_ROW && axis != MX_AXIS_COL) return MX_ERR_INVALID;
  if (rows == 0 || cols == 0) return MX_OK;
  const bool col = axis == MX_AXIS_COL;
  const int64_t len = col ? rows : cols;
  if (len % 32 != 0) return MX_ERR_INVALID;
  if (x == nullptr || !aligned16(x) || ld_x < cols || ld_x % 8 != 0 || cols % 8 != 0) return MX_ERR_INVALID;
  if (y == nullptr || !aligned16(y) || ld_y < len || ld_y % 4 != 0) return MX_ERR_INVALID;
  mx::RotateParams p{};
  p.x = x;
  p.rows = rows;
  p.cols = cols;
  p.ld_x = ld_x;
  p.y = y;
  p.ld_y = ld_y;
  p.col = col;
  p.sign_mask = 0u;
  const bool rht = had_kind == MX_HAD_RAND;
  if (rht) {
    const uint32_t w0 = philox_word0(0u, 0u, 2u, 0u, (uint32_t)had_seed, (uint32_t)(had_seed >> 32));
    p.sign_mask = had_n == 32 ? w0 : (w0 & 0xFFFFu);
  }
  hipError_t e = mx::launch_rotate(p, had_n, rht, (hipStream_t)hip_stream);
  return e == hipSuccess ? MX_OK : MX_ERR_DEVICE;
}

mx_status mx_quantize_f32(const float* y, int64_t lines, int64_t len, int64_t ld_y, mx_grid grid, mx_round round,
                          mx_axis axis, uint64_t seed, const mx_qtensor* out, void* hip_stream) {
  if (lines < 0 || len < 0) return MX_ERR_INVALID;
  if (grid != MX_GRID_E2M1 && grid != MX_GRID_E1M2) return MX_ERR_INVALID;
  if (round != MX_ROUND_RTNE && round != MX_ROUND_SR) return MX_ERR_INVALID;
  if (axis != MX_AXIS_ROW && axis != MX_AXIS_COL) return MX_ERR_INVALID;
  if (lines == 0 || len == 0) return MX_OK;
  if (len % 32 != 0) return MX_ERR_INVALID;
  if (y == nullptr || !aligned16(y) || ld_y < len || ld_y % 4 != 0) return MX_ERR_INVALID;
  mx_status s = check_qtensor(out, lines, len, 32);
  if (s != MX_OK) return s;
  mx::QuantF32Params p{};
  p.y = y;
  p.lines = lines;
  p.len = len;
  p.ld_y = ld_y;
  p.codes = out->codes;
  p.ld_codes = out->ld_codes;
  p.scales = out->scales;
  p.ld_scales = out->ld_scales;
  p.seed = seed;
  p.stream = axis == MX_AXIS_COL ? 1u : 0u;
  hipError_t e = mx::launch_quant_f32(p, grid, round, (hipStream_t)hip_stream);
  return e == hipSuccess ? MX_OK : MX_ERR_DEVICE;
}

mx_status mx_osci_reset(float* w, int64_t rows, int64_t cols, int64_t ld_w, const mx_qtensor* q, mx_grid grid,
                        float* w_prev, float* q_prev, float* dist_m, float* dist_q, int64_t ld_state,
                        mx_osci_mode mode, float threshold, uint64_t* resets, void* hip_stream) {
  if (rows < 0 || cols < 0) return MX_ERR_INVALID;
  if (grid != MX_GRID_E2M1 && grid != MX_GRID_E1M2) return MX_ERR_INVALID;
  if (mode != MX_OSCI_INIT && mode != MX_OSCI_TRACK && mode != MX_OSCI_CHECK) return MX_ERR_INVALID;
  if (mode == MX_OSCI_CHECK && !(threshold >= 0.0f && threshold <= 3.0e38f)) return MX_ERR_INVALID;
  if (rows == 0 || cols == 0) return MX_OK;
  if (cols % 32 != 0) return MX_ERR_INVALID;
  const float* arrays[5] = {w, w_prev, q_prev, dist_m, dist_q};
  for (const float* a : arrays)
    if (a == nullptr || !aligned16(a)) return MX_ERR_INVALID;
  if (ld_w < cols || ld_w % 4 != 0 || ld_state < cols || ld_state % 4 != 0) return MX_ERR_INVALID;
  if (resets != nullptr && ((uintptr_t)resets & 7u) != 0) return MX_ERR_INVALID;
  mx_status s = check_qtensor(q, rows, cols, 32);
  if (s != MX_OK) return s;
  mx::OsciParams p{};
  p.w = w;
  p.rows = rows;
  p.cols = cols;
  p.ld_w = ld_w;
  p.codes = q->codes;
  p.ld_codes = q->ld_codes;
  p.scales = q->scales;
  p.ld_scales = q->ld_scales;
  p.w_prev = w_prev;
  p.q_prev = q_prev;
  p.dist_m = dist_m;
  p.dist_q = dist_q;
  p.ld_s = ld_state;
  p.mode = mode;
  p.threshold = threshold;
  p.resets = (unsigned long long*)resets;
  hipError_t e = mx::launch_osci(p, grid, (hipStream_t)hip_stream);
  return e == hipSuccess ? MX_OK : MX_ERR_DEVICE;
}

const char* mx_status_str(mx_status status) {
  switch (status) {
    case MX_OK: return "MX_OK";
    case MX_ERR_INVALID: return "MX_ERR_INVALID: invalid argument";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED: valid request not implemented";
    case MX_ERR_DEVICE: return "MX_ERR_DEVICE: HIP runtime error";
  }
  return "unknown mx_status";
}

int32_t mx_version(void) { return 100; }

}  // extern "C"
