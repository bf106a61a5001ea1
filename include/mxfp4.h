/*
 * mxfp4.h - C ABI of the MI355X (gfx950) block-scaled 4-bit quantizer and GEMM.
 *
 * What is computed (by page title and section):
 *  - "Pre-addestramento di Modelli Linguistici di Grandi Dimensioni con MXFP4",
 *    Metodologia: the three GEMMs of a linear layer's training step (Fprop,
 *    Dgrad, Wgrad) in MXFP4, optionally after a deterministic H16/H32 or a
 *    randomized Hadamard rotation; stochastic rounding as an alternative.
 *  - "Ripensare il Bias di Shrinkage nel Pretraining di LLM in FP4",
 *    Problematica and Metodologia 2: E2M1 under round-to-nearest-even, and the
 *    uniform E1M2/INT4 grid of the UFP4 recipe.
 *  - "MXNorm: Reusing MXFP block scales ...", Sommario tecnico 2: one shared
 *    scale per block derived from the block's absolute maximum.
 *  - "Résumé Technique : TetraJet-v2", section 2.A: stochastic rounding with
 *    E[round(x)] = x.
 *  - "MXNorm: Reusing MXFP block scales ...", Sommario tecnico 2: row
 *    normalization by an inverse-RMS estimate built from the block maxima,
 *    fused with the cast (mx_mxnorm_quantize).
 *
 * Data layout (all row-major, strides in the units named):
 *  - Input x: bf16 bit patterns, x[r * ld_x + c], 0 <= r < rows, 0 <= c < cols.
 *  - A quantized operand (mx_qtensor) of L lines of length K:
 *      codes [L][K/2] bytes, line stride ld_codes bytes; element 2j of a line in
 *      the low nibble of byte j; nibble bit 3 = sign, bits 2..0 = magnitude code
 *      (E2M1: 0,0.5,1,1.5,2,3,4,6; E1M2: k/4);
 *      scales [L][K/block] bytes (E8M0: value 2^(byte-127), 0xFF = NaN block),
 *      line stride ld_scales bytes.
 *  - Row-wise output: lines = rows, K = cols (blocks run along a row).
 *    Column-wise output: lines = cols, K = rows: the quantized transpose, so
 *    every GEMM operand is K-contiguous.
 *
 * The cast: e = clamp(floor(log2 amax) - emax, -127, 127) per block of 32
 * (emax 2 for E2M1, 0 for E1M2; amax 0 gives -127); v = |y| / 2^e goes to the
 * grid by round-to-nearest-even (ties to the even code, saturating at the top
 * level) or by stochastic rounding: with lo <= v < hi adjacent levels and
 * f = (v - lo) / (hi - lo), round up iff floor(f * 2^16) + r >= 2^16
 * (add-and-truncate on 16 random bits: unbiased up to 2^-16 of a step), where
 * r is the 16-bit half (i mod 2, low half first) of word (i mod 8) / 2 of
 * Philox4x32-10(key = seed, counter = (i div 8, stream, 0)) for the element at
 * index i of the output's logical row-major order (row-wise: r*cols + c,
 * stream 0; column-wise: c*rows + r, stream 1).  A block holding a non-finite
 * value gets scale 0xFF and codes 0.
 *
 * The rotation (mx_hadamard_quantize): y = RN32(RN32(S) * RN32(1/sqrt(n)))
 * per aligned chunk of n = 16 or 32 along the quantization axis, where S is
 * the EXACT value of sum_j H[i][j] s_j x_j, H the Sylvester matrix
 * (H[i][j] = (-1)^popcount(i & j)), s_j = +1 (MX_HAD_DET) or, for
 * MX_HAD_RAND, s_j = -1 iff bit j of word 0 of
 * Philox4x32-10(key = had_seed, counter = (0, 0, 2, 0)).  An exact zero sum
 * gives +0; a chunk holding a non-finite input gives NaN outputs.
 *
 * Conventions:
 *  - All pointers are caller-owned DEVICE pointers (the mx_qtensor structs
 *    themselves are host memory, read before the call returns).  The library
 *    allocates no memory and keeps no mutable global state; calls are
 *    thread-safe.
 *  - Every call is asynchronous on hip_stream (a hipStream_t; NULL = the
 *    default stream).  Argument errors are reported synchronously, before
 *    anything is launched.  A launch failure returns MX_ERR_DEVICE; faults
 *    surface at the caller's next synchronization.
 *  - Nothing throws across the ABI.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_OK = 0,
  MX_ERR_INVALID = 1,      /* a null/misaligned pointer, a bad size or stride, an enum out of range */
  MX_ERR_UNSUPPORTED = 2,  /* a valid request this library does not implement (e.g. block 16 GEMM) */
  MX_ERR_DEVICE = 3        /* the HIP runtime refused a launch or query */
} mx_status;

typedef enum { MX_GRID_E2M1 = 0, MX_GRID_E1M2 = 1 } mx_grid;
typedef enum { MX_ROUND_RTNE = 0, MX_ROUND_SR = 1 } mx_round;
typedef enum { MX_AXIS_ROW = 1, MX_AXIS_COL = 2, MX_AXIS_BOTH = 3 } mx_axis;   /* bit mask */
typedef enum { MX_HAD_NONE = 0, MX_HAD_DET = 1, MX_HAD_RAND = 2 } mx_had;
typedef enum { MX_OUT_F32 = 0, MX_OUT_BF16 = 1 } mx_out;
typedef enum { MX_OSCI_INIT = 0, MX_OSCI_TRACK = 1, MX_OSCI_CHECK = 2 } mx_osci_mode;

/* An NVFP4-style double-block operand (mx_nvfp4_quantize): L lines of length K. */
typedef struct {
  uint8_t *codes;     /* device: [L][K/2] packed E2M1 codes, as mx_qtensor */
  int64_t ld_codes;   /* bytes between lines; >= K/2, multiple of 16 */
  uint8_t *inner;     /* device: [L][K/16] E4M3 scale bytes */
  int64_t ld_inner;   /* bytes between lines; >= K/16 */
  float *outer;       /* device: [L][K/128] float32 scales, 4-byte aligned */
  int64_t ld_outer;   /* floats between lines; >= K/128 */
} mx_nvfp4_tensor;

/* Totals of mx_quant_stats (see there); 8-byte aligned device memory. */
typedef struct {
  double sum_sq;       /* sum of y^2 over the counted blocks */
  double sum_err_sq;   /* sum of (y - y_hat)^2 */
  uint64_t hist[8];    /* count of every magnitude code 0..7 */
  uint64_t blocks;     /* 32-value blocks counted */
} mx_quant_stats_t;

typedef struct {
  uint8_t *codes;     /* device: [lines][K/2] packed 4-bit codes; 16-byte aligned (8 with block 16) */
  int64_t ld_codes;   /* bytes between lines; >= K/2, multiple of 16 (of 8 with block 16) */
  uint8_t *scales;    /* device: [lines][K/block] E8M0 bytes */
  int64_t ld_scales;  /* bytes between lines; >= K/block */
} mx_qtensor;

/*
 * mx_quantize: block-scaled 4-bit quantization of a bf16 matrix, no rotation.
 *   x          device, 16-byte aligned, bf16 bit patterns
 *   rows, cols >= 0 (either 0: nothing to do, MX_OK); cols % 8 == 0;
 *              cols % block == 0 if the row-wise output is requested,
 *              rows % block == 0 if the column-wise output is requested
 *   ld_x       elements between rows; >= cols, multiple of 8, below 2^25
 *   block      32 (the MX block) or 16 (16-value MX blocks, E8M0 scales
 *              [L][K/16]; not with a rotation: mx_hadamard_quantize with
 *              block 16 returns MX_ERR_UNSUPPORTED)
 *   grid       MX_GRID_E2M1 or MX_GRID_E1M2
 *   round      MX_ROUND_RTNE or MX_ROUND_SR (seed keys the Philox draws)
 *   axis       which outputs to write; row_out / col_out must be non-null for
 *              the requested ones (codes 16-byte aligned, 8 with block 16) and are ignored
 *              otherwise
 * Both outputs of MX_AXIS_BOTH come from one pass over x.
 */
mx_status mx_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                      int32_t block, mx_grid grid, mx_round round, mx_axis axis,
                      uint64_t seed, const mx_qtensor *row_out, const mx_qtensor *col_out,
                      void *hip_stream);

/*
 * mx_hadamard_quantize: as mx_quantize, after a block Hadamard rotation of
 * order had_n (16 or 32, dividing block) along each output's quantization
 * axis (row-wise: along a row; column-wise: along a column).  had_kind
 * MX_HAD_DET or MX_HAD_RAND (had_seed draws the sign vector; the same vector
 * serves both outputs, so the rotation cancels in a GEMM whose two operands
 * were rotated with the same had_n, had_kind and had_seed).
 */
mx_status mx_hadamard_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                               int32_t block, mx_grid grid, mx_round round, mx_axis axis,
                               uint64_t seed, int32_t had_n, mx_had had_kind, uint64_t had_seed,
                               const mx_qtensor *row_out, const mx_qtensor *col_out,
                               void *hip_stream);

/*
 * mx_gemm: C[m][n] = sum_k A[m][k] * B[n][k] on the decoded values, with fp32
 * accumulation ("Pre-addestramento ... con MXFP4", Metodologia: MXFP4 GEMMs on
 * native FP4 matrix units).
 *   a          M lines of length K (codes [M][K/2], scales [M][K/32])
 *   b          N lines of length K (codes [N][K/2], scales [N][K/32])
 *   M, N, K    >= 0 (any 0: nothing to do; K == 0 is rejected); K % 32 == 0
 *   grid       the grid both operands were quantized to (E1M2 runs as exact
 *              FP8 E4M3 on the matrix units: every value k/4 is exact there)
 *   block      32
 *   c          device, row-major [M][ldc] fp32 or bf16 (round to nearest even
 *              of the fp32 result); aligned to its element size, ldc >= N
 * Any accepted shape gives the same numbers.  The fast path (256 x 256 tiles
 * fed by LDS copies) takes M, N >= 256, N % 4 == 0, K >= 512, 4-byte aligned
 * scale rows with ld_scales % 4 == 0, ldc % 4 == 0, c 16-byte (fp32) or
 * 8-byte (bf16) aligned, and an operand span per 256-row tile below 4 GiB
 * (255 * ld_codes + K/2 < 2^32 and 255 * ld_scales + K/32 < 2^32, for both
 * operands); bf16 output is fastest with ldc % 8 == 0, N % 8 == 0 and c
 * 16-byte aligned.  Other shapes run a slower bounds-checked kernel.
 */
mx_status mx_gemm(const mx_qtensor *a, const mx_qtensor *b, int64_t M, int64_t N, int64_t K,
                  mx_grid grid, int32_t block, void *c, int64_t ldc, mx_out out,
                  void *hip_stream);

/*
 * mx_gemm_grouped: count independent mx_gemm problems of one K, grid and
 * output kind in one launch ("Pre-addestramento ... con MXFP4", Metodologia:
 * the Wgrad GEMMs of a block's linear layers, which nothing in the backward
 * pass reads before the optimizer step, so they can run as a group).  Problem
 * i computes C_i[m][n] = sum_k A_i[m][k] * B_i[n][k] exactly as mx_gemm(a_i,
 * b_i, M_i, N_i, K, grid, block, c_i, ldc_i, out) does, to the bit.  One
 * persistent launch walks the tiles of all problems when every problem takes
 * mx_gemm's fast path, the problems share the operand pitches (ld_codes and
 * ld_scales of every a_i, and of every b_i), and bf16 outputs have
 * ldc_i % 8 == 0, N_i % 8 == 0 and 16-byte aligned c_i; a problem whose tiles
 * end part-way through a round of the chip then leaves no CU idle while the
 * next problem has tiles.  Otherwise the problems run one launch each, in
 * order.  The outputs must not overlap one another or any operand.
 *   problems   host array of count entries (read before the call returns)
 *   count      1 .. MX_GEMM_GROUP_MAX
 *   K, grid, block, out   as mx_gemm, for every problem
 * Every problem is validated as mx_gemm validates its arguments before
 * anything is launched; problems with M_i or N_i of 0 are skipped.
 */
#define MX_GEMM_GROUP_MAX 8
typedef struct {
    const mx_qtensor *a;   /* M lines of length K */
    const mx_qtensor *b;   /* N lines of length K */
    int64_t M, N;
    void *c;               /* device, row-major [M][ldc] */
    int64_t ldc;
} mx_gemm_problem;

mx_status mx_gemm_grouped(const mx_gemm_problem *problems, int32_t count, int64_t K, mx_grid grid,
                          int32_t block, mx_out out, void *hip_stream);

/*
 * mx_mxnorm_quantize: MXNorm fused with the row-wise MX cast ("MXNorm: Reusing
 * MXFP block scales for efficient tensor normalisation", Sommario tecnico 2).
 * Row t is scaled by rho_t = c * ((1/K) sum_k m_tk^p)^(-1/p), the inverse-RMS
 * estimate from its K = cols/32 block maxima, and the scaled row is quantized
 * row-wise (block 32) as by mx_quantize with axis MX_AXIS_ROW.  The gain of
 * the normalization is not applied (it belongs in the next layer's weights).
 * Exactly:
 *   m_tk  = max |x| over block k of row t (bf16 values; NaN counts as +inf);
 *   S_t   = sum of m_tk^p in float64 as a balanced binary tree over the
 *           blocks in order (neighbours first), missing blocks of a
 *           power-of-two count being zeros;
 *   q_t   = RN64(S_t / K);
 *   rho_t = RN32 of the exact real number c * q_t^(-1/p) (ties to even;
 *           +inf on overflow), or 0 when q_t is 0 or +inf;
 *   y     = RN32(x * rho_t), cast with stochastic-rounding stream 0.
 *   x          device, 16-byte aligned, bf16 bit patterns
 *   rows, cols >= 0 (either 0: nothing to do, MX_OK); cols % 32 == 0,
 *              cols <= 65536
 *   ld_x       elements between rows; >= cols, multiple of 8
 *   power      p: 1 or 2 (the pages favour 2)
 *   c          the correction constant c(p, 32) > 0, finite (for rows of
 *              i.i.d. normal values E[M^p]^(1/p), M the largest |value| of
 *              32: about 2.3471 for p = 1 and 2.3895 for p = 2)
 *   grid, round, seed   as mx_quantize
 *   out        rows lines of length cols (codes 16-byte aligned)
 *   rho        device, float[rows], 4-byte aligned: rho_t for the backward pass
 */
mx_status mx_mxnorm_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                             int32_t power, float c, mx_grid grid, mx_round round, uint64_t seed,
                             const mx_qtensor *out, float *rho, void *hip_stream);

/*
 * mx_quant_stats: diagnostics of a quantized tensor ("Ripensare il Bias di
 * Shrinkage nel Pretraining di LLM in FP4", Risultati Sperimentali,
 * Diagnostica di Quantizzazione: SQNR and bucket usage with and without the
 * rotation, E2M1 against E1M2).  Adds to *stats, over every block whose scale
 * byte is not 0xFF: sum of y^2, sum of (y - y_hat)^2, the counts of the 8
 * magnitude codes and the number of blocks.  y are the values the cast
 * received (x, or its rotation as defined for mx_hadamard_quantize, formed
 * with float64 butterflies: exact for chunks spanning at most 40 binades,
 * within float64 rounding otherwise); y_hat is the decoded code times
 * 2^(scale byte - 127).  SQNR = 10 log10(sum_sq / sum_err_sq).
 *   x, rows, cols, ld_x   the tensor that was quantized (ld_x >= cols)
 *   axis       MX_AXIS_ROW or MX_AXIS_COL: which output q is
 *   grid, had_n, had_kind, had_seed   as passed to the quantizer (had_kind
 *              MX_HAD_NONE: no rotation)
 *   q          the quantized output (lines and length as for that axis;
 *              the quantized axis a multiple of 32)
 *   stats      device, 8-byte aligned; the caller zeroes it before the first
 *              call; several calls may accumulate into one total.  The
 *              float64 sums are added with atomics, so their last bits may
 *              vary from run to run; the counts are exact.
 */
mx_status mx_quant_stats(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x, mx_axis axis,
                         mx_grid grid, int32_t had_n, mx_had had_kind, uint64_t had_seed,
                         const mx_qtensor *q, mx_quant_stats_t *stats, void *hip_stream);

/*
 * mx_nvfp4_quantize: NVFP4-style double-block quantization ("Résumé
 * Technique : TetraJet-v2", section 2.A: 16-value groups under an 8-bit scale,
 * inside 128-value outer blocks scaled as a whole, with no tensor-wide absmax).
 * Along each requested axis (row-wise: along a row; column-wise: the
 * transpose's rows, i.e. along the token axis):
 *   s_o = RN32(amax128 / 2688)                 float32 per 128 values
 *   s_i = E4M3 nearest to amax16 / (6 * s_o)   (ties to even, saturating at
 *         448; exact quotient), one byte per 16 values
 *   y   = RN32(RN64(x * RN64(1 / (s_i * s_o)))), cast to E2M1 at unit scale
 *         by RTNE or the stochastic rule of mx_quantize (stream 0 row-wise,
 *         1 column-wise), saturating at 6; decoded value = code * s_i * s_o.
 * s_i = 0 (a zero or underflowing inner block) leaves only the sign bit; an
 * outer block holding Inf or NaN gets s_o = NaN, inner 0x7F and codes 0.
 * gfx950's matrix cores take 32-value E8M0 blocks, so mx_gemm does not take
 * these operands.
 *   x, rows, cols, ld_x   as mx_quantize (16-byte aligned, ld_x % 8 == 0,
 *              cols % 8 == 0); the quantized axis a multiple of 128
 *   round      MX_ROUND_RTNE or MX_ROUND_SR (seed keys the Philox draws)
 *   axis       which outputs; row_out / col_out non-null for those
 */
mx_status mx_nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x, mx_round round,
                            mx_axis axis, uint64_t seed, const mx_nvfp4_tensor *row_out,
                            const mx_nvfp4_tensor *col_out, void *hip_stream);

/*
 * mx_hadamard_rotate: the block Hadamard rotation alone, as float32 ("Ripensare
 * il Bias di Shrinkage nel Pretraining di LLM in FP4", Efficienza: the random
 * Hadamard transform fused with the FP4 quantization against the two run as
 * separate kernels; this and mx_quantize_f32 are the separate kernels).
 * y = RN32(RN32(S) * RN32(1/sqrt(n))) of the exact sum, as for
 * mx_hadamard_quantize, for every aligned chunk of had_n values along the axis.
 *   x, rows, cols, ld_x  device bf16 bit patterns, 16-byte aligned; ld_x >= cols,
 *              ld_x % 8 == 0, cols % 8 == 0
 *   had_n, had_kind, had_seed  as mx_hadamard_quantize (MX_HAD_DET or MX_HAD_RAND)
 *   axis       MX_AXIS_ROW: rotate along each row; y is [rows][ld_y], cols % 32 == 0
 *              MX_AXIS_COL: rotate along each column; y holds the transpose,
 *              [cols][ld_y] with y[c][r], rows % 32 == 0
 *   y, ld_y    device float32, 16-byte aligned; ld_y (floats) >= the rotated
 *              axis' length and a multiple of 4
 */
mx_status mx_hadamard_rotate(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x, int32_t had_n,
                             mx_had had_kind, uint64_t had_seed, mx_axis axis, float *y, int64_t ld_y,
                             void *hip_stream);

/*
 * mx_quantize_f32: the MX cast (block 32) of float32 lines, as mx_quantize
 * casts the values it computes: block absmax, E8M0 scale, RTNE or stochastic
 * rounding, a block holding a non-finite value getting scale 0xFF and codes 0.
 * With y from mx_hadamard_rotate the codes and scales equal those of
 * mx_hadamard_quantize for the same axis.
 *   y          device float32 [lines][ld_y], 16-byte aligned, ld_y >= len and a
 *              multiple of 4; len % 32 == 0
 *   axis       which output of the original tensor the lines are, for the
 *              stochastic-rounding draws: MX_AXIS_ROW (its rows, stream 0) or
 *              MX_AXIS_COL (its columns, y holding the transpose, stream 1);
 *              element j of line l has index l * len + j
 *   grid, round, seed   as mx_quantize
 *   out        lines lines of length len (codes 16-byte aligned)
 */
mx_status mx_quantize_f32(const float *y, int64_t lines, int64_t len, int64_t ld_y, mx_grid grid, mx_round round,
                          mx_axis axis, uint64_t seed, const mx_qtensor *out, void *hip_stream);

/*
 * mx_osci_reset: OsciReset on float32 master weights ("Résumé Technique :
 * TetraJet-v2", 2. Méthodologie, B: the oscillation risk is the distance the
 * quantized weight travels over the distance the master weight travels; when
 * the learning rate is small and the risk exceeds a threshold, the master
 * weight is reset to the centre of its current quantization bin).  Per
 * element, in float32 with one rounding per operation:
 *   q      = the decoded value of w's code in q (level times 2^(scale - 127));
 *   MX_OSCI_INIT:  w_prev = w, q_prev = q, dist_m = dist_q = 0;
 *   MX_OSCI_TRACK: dist_m += |w - w_prev|, dist_q += |q - q_prev|;
 *   MX_OSCI_CHECK: as TRACK, then w = q where dist_q > threshold * dist_m
 *                  (the caller checks when its learning rate is small), and
 *                  dist_m = dist_q = 0 everywhere (a new window);
 *   then w_prev = w, q_prev = q.
 *   w          device float32 [rows][ld_w], 16-byte aligned, ld_w % 4 == 0;
 *              written only where reset
 *   q          w's row-wise quantization (block 32: e.g. mx_quantize_f32 of w
 *              with MX_AXIS_ROW), rows lines of length cols; cols % 32 == 0
 *   grid       the grid q was cast to
 *   w_prev, q_prev, dist_m, dist_q   device float32 state [rows][ld_state],
 *              16-byte aligned, ld_state % 4 == 0; written by every mode
 *   threshold  finite, >= 0 (read by MX_OSCI_CHECK only)
 *   resets     optional device counter (8-byte aligned, or NULL): the number
 *              of elements reset is added to it
 */
mx_status mx_osci_reset(float *w, int64_t rows, int64_t cols, int64_t ld_w, const mx_qtensor *q, mx_grid grid,
                        float *w_prev, float *q_prev, float *dist_m, float *dist_q, int64_t ld_state,
                        mx_osci_mode mode, float threshold, uint64_t *resets, void *hip_stream);

/* A static, human-readable name for a status code. */
const char *mx_status_str(mx_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t mx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
