"""Quantization diagnostics: SQNR and bucket usage of an MX-quantized tensor (oracle side).

Test infrastructure only: see the package docstring.

"Ripensare il Bias di Shrinkage nel Pretraining di LLM in FP4", Risultati
Sperimentali (Diagnostica di Quantizzazione e GEMM): the quality of a 4-bit
cast is read from its signal-to-quantization-noise ratio and from how evenly
it uses the grid's buckets, with and without the random Hadamard rotation, for
E2M1 and for the uniform E1M2 grid.

Readings (the pages name the quantities without formulas):
* the signal is y, the values the cast receives (the rotated values when a
  rotation is applied, y = RN32(RN32(S) * RN32(1/sqrt(n))) as oracle.hadamard
  defines it; the bf16 inputs otherwise); the noise is y - y_hat with y_hat the
  decoded code times 2^(scale byte - 127).  SQNR = 10 log10(sum y^2 / sum
  (y - y_hat)^2) over the tensor, in float64;
* blocks with scale byte 0xFF (non-finite) are left out of every sum;
* bucket usage is the histogram of the 8 magnitude codes; the effective bucket
  ratio is exp(H) / 8, H the Shannon entropy (nats) of that histogram, i.e.
  the effective number of buckets in use over the number available.
"""
import math

import numpy as np

from .formats import E8M0_NAN, bf16_bits_to_f64
from .gemm import decode
from .hadamard import rotate_lines, rht_signs

AXES = ("row", "col")


def cast_input(x_bits, axis="row", had_n=0, had_kind="det", had_seed=0):
    """The values the cast sees, as float64 lines along the quantization axis (lines, length)."""
    bits = np.asarray(x_bits, dtype=np.uint16)
    lines = bits if axis == "row" else np.ascontiguousarray(bits.T)
    if had_n:
        signs = rht_signs(had_n, had_seed) if had_kind == "rand" else None
        return rotate_lines(lines, had_n, signs).astype(np.float64)
    return bf16_bits_to_f64(lines)


def quant_stats_ref(x_bits, codes, scales, axis="row", grid="e2m1", had_n=0, had_kind="det", had_seed=0,
                    block=32):
    """(sum y^2, sum (y - y_hat)^2, histogram of magnitude codes (8,), blocks counted) over finite blocks."""
    y = cast_input(x_bits, axis, had_n, had_kind, had_seed)
    lines, length = y.shape
    yhat = decode(codes, scales, grid, length, block)
    nib = np.empty((lines, codes.shape[1] * 2), dtype=np.uint8)
    nib[:, 0::2] = np.asarray(codes) & 0xF
    nib[:, 1::2] = np.asarray(codes) >> 4
    keep_blk = np.asarray(scales)[:, :length // block] != E8M0_NAN
    keep = np.repeat(keep_blk, block, axis=1)
    yk = np.where(keep, y, 0.0)
    ek = np.where(keep, y - np.where(keep, yhat, 0.0), 0.0)
    hist = np.bincount((nib[:, :length] & 7)[keep], minlength=8).astype(np.int64)
    return float(np.sum(yk * yk)), float(np.sum(ek * ek)), hist, int(keep_blk.sum())


def sqnr_db(sum_sq, sum_err_sq):
    return math.inf if sum_err_sq == 0 else 10.0 * math.log10(sum_sq / sum_err_sq)


def effective_bucket_ratio(hist):
    p = np.asarray(hist, dtype=np.float64)
    p = p[p > 0] / p.sum()
    return float(math.exp(-np.sum(p * np.log(p))) / 8.0)
