"""The block-scaled GEMM on decoded values (oracle side).

Test infrastructure only: see the package docstring.

"Pre-addestramento ... con MXFP4", Metodologia: the three GEMMs of a linear
layer's training step (forward Fprop, activation gradient Dgrad, weight
gradient Wgrad) run with both operands in MXFP4 on native FP4 matrix units.
The product is defined on decoded values: every element is its grid level
times 2^(scale byte - 127) of its block, and
    C[m, n] = sum_k A[m, k] * B[n, k]
with both operands stored K-contiguous (an "NT" product).  The oracle forms
C in float64; products of two decoded values are exact there (at most four
significant bits), so C is exact whenever the partial sums stay within 53 bits.
G = |A| |B|^T is the scale of the tolerance |C_gpu - C| <= 1e-5 * G.
"""
import numpy as np

from .formats import E8M0_BIAS, E8M0_NAN, levels


def decode(codes, scales, grid, k, block=32):
    """Decoded float64 values (rows, k) of packed codes (rows, k/2) and scales (rows, k/block)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    nib = np.empty((rows, codes.shape[1] * 2), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    nib = nib[:, :k]
    lv = levels(grid)
    mag = lv[nib & 7]
    val = np.where(nib & 8, -mag, mag)
    sb = np.repeat(scales.astype(np.int64), block, axis=1)[:, :k]
    scale = np.where(sb == E8M0_NAN, np.nan, np.ldexp(1.0, sb - E8M0_BIAS))
    return val * scale


def gemm_ref(a_codes, a_scales, b_codes, b_scales, k, grid, rows=None, cols=None, block=32):
    """(C, G) in float64 for the rows/cols subsets requested (all when None)."""
    a = decode(a_codes if rows is None else np.asarray(a_codes)[rows],
               a_scales if rows is None else np.asarray(a_scales)[rows], grid, k, block)
    b = decode(b_codes if cols is None else np.asarray(b_codes)[cols],
               b_scales if cols is None else np.asarray(b_scales)[cols], grid, k, block)
    c = a @ b.T
    g = np.abs(a) @ np.abs(b).T
    return c, g


def bf16_round_f64(x):
    """float64 -> nearest bf16 value (ties to even), through float32 with one rounding each.

    Used only to form the bf16 tolerance; the GEMM's bf16 output is checked
    against C with a bound that covers both roundings.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)
