"""Block-scaled 4-bit quantization of a bf16 tensor (oracle side).

Test infrastructure only: see the package docstring.

The steps follow the pages' description of an MX cast, in order:
 1. optional block Hadamard rotation along the quantization axis
    ("Pre-addestramento ... con MXFP4", Metodologia; oracle.hadamard);
 2. the absolute maximum of every block of 32 consecutive values
    ("MXNorm: Reusing MXFP block scales ...", Sommario tecnico 2);
 3. one shared power-of-two scale per block, e = floor(log2 amax) - emax
    (oracle.formats.scale_exponent), stored as an E8M0 byte e + 127;
 4. the cast of v = |y| / 2^e onto the 4-bit grid, by round-to-nearest-even
    ("Ripensare il Bias di Shrinkage ...", Problematica) or by stochastic
    rounding that is unbiased in expectation ("Résumé Technique : TetraJet-v2",
    section 2.A), saturating at the largest level, keeping the sign of y;
 5. packing two 4-bit codes per byte.
Row-wise quantization blocks each row along its columns (the Fprop and Dgrad
operands); column-wise quantization blocks each column along the rows, i.e.
along the token axis for the Wgrad operands ("Pre-addestramento ... con MXFP4",
Metodologia: the three GEMMs Fprop, Dgrad and Wgrad).

Readings where the pages are silent (all listed with their reasons in the
design notes):
* code nibble: bit 3 = sign of y (so -0 gives 0x8), bits 2..0 = magnitude code;
  element 2j in the low nibble of byte j; scales row-major, one byte per block;
* the column-wise output is the row-wise quantization of the transpose;
* a block holding a non-finite y gets scale byte 0xFF and all codes 0;
* RTNE: nearest level, a tie goes to the even code, anything above the top
  level saturates to it;
* SR: with lo <= v < hi adjacent levels, frac = (v - lo) / (hi - lo) and
  P = floor(frac * 2^16), the magnitude rounds up iff P + r >= 2^16 for the
  element's 16-bit draw r, i.e. floor(frac + r / 2^16) on a 16-bit truncated
  frac; v at or above the top level saturates.  The probability of rounding
  up is P / 2^16, so E[SR(v)] = v up to less than 2^-16 of a step;
* the 16-bit draw of the element at index i of the output's logical row-major
  order (row r, column c of a row-wise output: i = r*cols + c; a column-wise
  output is indexed in the transposed tensor: i = c*rows + r) is half i mod 2
  (low half first) of word (i mod 8) div 2 of Philox4x32-10(key = seed,
  counter = (i div 8, stream)), stream 0 for the row-wise output and 1 for the
  column-wise one: one call serves eight elements;
* a tail block shorter than 32 (oracle only) takes its absmax over the values
  present; a missing high nibble is 0.
"""
from fractions import Fraction

import numpy as np

from .formats import (E2M1, E1M2, EMAX, E8M0_BIAS, E8M0_NAN, SCALE_EXP_MIN, SCALE_EXP_MAX,
                      bf16_bits_to_f64, levels)
from .hadamard import rotate_lines, rht_signs, HADAMARD_SIZES
from .philox import uniform_halfwords, STREAM_ROW_SR, STREAM_COL_SR

RTNE = "rtne"
SR = "sr"
BLOCK_SIZES = (16, 32)


def rtne_magnitude_codes(v, grid):
    """RTNE of v >= 0 (float64 array, exact) onto the grid's 8 magnitudes."""
    lv = levels(grid)
    mids = (lv[:-1] + lv[1:]) / 2.0                 # exact in float64
    idx = np.searchsorted(mids, v, side="left")     # number of midpoints strictly below v
    at = np.minimum(idx, len(mids) - 1)
    tie = (idx < len(mids)) & (v == mids[at])
    return np.where(tie & (idx % 2 == 1), idx + 1, idx).astype(np.uint8)


def sr_magnitude_codes(v, r, grid):
    """Stochastic rounding of v >= 0 onto the grid, given 16-bit draws r (same shape).

    Round up from the largest level lo <= v iff floor(frac * 2^16) + r >= 2^16:
    frac = (v - lo) / (hi - lo) truncated to 16 bits, plus a 16-bit uniform
    fraction, carried into the integer part.  The probability of rounding up
    is floor(frac * 2^16) / 2^16, so E[SR(v)] = v up to less than 2^-16 of a
    step ("Résumé Technique : TetraJet-v2", section 2: unbiased stochastic
    rounding).

    v - lo is exact in float64: either lo = 0, or lo >= v/2 (Sterbenz), since
    adjacent levels of both grids are at most a factor 2 apart.
    """
    lv = levels(grid)
    lo = np.searchsorted(lv, v, side="right") - 1   # largest level <= v
    top = lo >= len(lv) - 1
    lo_c = np.minimum(lo, len(lv) - 2)
    width = lv[lo_c + 1] - lv[lo_c]
    frac = (v - lv[lo_c]) / width                   # width is a power of two: exact
    p16 = np.floor(frac * 2.0 ** 16)                # 16-bit fixed-point probability
    up = p16 + np.asarray(r, dtype=np.float64) >= 2.0 ** 16
    code = np.where(top, len(lv) - 1, lo + up.astype(np.int64))
    return code.astype(np.uint8)


def block_scale_exponents(amax, grid):
    """e = clamp(floor(log2 amax) - emax, -127, 127) per block; amax = 0 gives -127."""
    mant, ex = np.frexp(amax)                       # amax = mant * 2^ex, mant in [0.5, 1): exact
    e = np.clip(ex.astype(np.int64) - 1 - EMAX[grid], SCALE_EXP_MIN, SCALE_EXP_MAX)
    return np.where(amax == 0.0, SCALE_EXP_MIN, e)


def quantize_lines(bits, grid=E2M1, rounding=RTNE, seed=0, stream=STREAM_ROW_SR,
                   had_n=0, signs=None, block=32, line_ids=None):
    """Quantize every line (row) of a 2-D bf16 array along its last axis.

    bits: (lines, length) uint16 bf16 patterns.  line_ids: the index of each
    given line in the whole output (default 0, 1, ...), which only enters the
    stochastic-rounding element index.
    Returns (codes, scales): codes (lines, ceil(length/2)) uint8 with element
    2j in the low nibble of byte j; scales (lines, ceil(length/block)) uint8.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    assert bits.ndim == 2 and grid in (E2M1, E1M2) and rounding in (RTNE, SR)
    assert block in BLOCK_SIZES
    lines, length = bits.shape

    # 1. optional rotation along the line
    if had_n:
        assert had_n in HADAMARD_SIZES and length % had_n == 0 and block % had_n == 0
        y = rotate_lines(bits, had_n, signs)
    else:
        y = bf16_bits_to_f64(bits).astype(np.float32)
    return quantize_values(y, grid, rounding, seed, stream, block, line_ids)


def quantize_values(y, grid=E2M1, rounding=RTNE, seed=0, stream=STREAM_ROW_SR, block=32, line_ids=None):
    """Steps 2-5 on float32 values y (lines, length): absmax, scale, cast, pack.

    Same outputs and element indexing as quantize_lines.
    """
    y = np.asarray(y, dtype=np.float32)
    assert y.ndim == 2 and grid in (E2M1, E1M2) and rounding in (RTNE, SR) and block in BLOCK_SIZES
    lines, length = y.shape

    # pad to whole blocks (oracle-only tails: zeros do not change the absmax)
    nblk = -(-length // block)
    ypad = np.zeros((lines, nblk * block), dtype=np.float32)
    ypad[:, :length] = y
    yb = ypad.reshape(lines, nblk, block).astype(np.float64)

    # 2. block absmax, and which blocks hold a non-finite value
    finite_blk = np.isfinite(yb).all(axis=2)
    amax = np.where(finite_blk, np.abs(np.where(np.isfinite(yb), yb, 0.0)).max(axis=2), 0.0)

    # 3. shared exponent and E8M0 byte
    e = block_scale_exponents(amax, grid)
    scales = np.where(finite_blk, e + E8M0_BIAS, E8M0_NAN).astype(np.uint8)

    # 4. cast v = |y| / 2^e (exact: a power-of-two rescale of a float32 in float64)
    v = np.ldexp(np.abs(np.where(np.isfinite(yb), yb, 0.0)), -e[:, :, None])
    if rounding == RTNE:
        mag = rtne_magnitude_codes(v, grid)
    else:
        ids = np.arange(lines) if line_ids is None else np.asarray(line_ids)
        idx = (ids.astype(np.uint64)[:, None] * np.uint64(length)
               + np.arange(nblk * block, dtype=np.uint64)[None, :])
        r = uniform_halfwords(seed, stream, idx).reshape(lines, nblk, block)
        mag = sr_magnitude_codes(v, r, grid)
    sign = np.signbit(yb).astype(np.uint8)
    codes4 = (sign << 3) | mag
    codes4 = np.where(finite_blk[:, :, None], codes4, 0).astype(np.uint8)
    codes4 = codes4.reshape(lines, nblk * block)[:, :length]

    # 5. pack: element 2j -> low nibble, 2j+1 -> high nibble
    if length % 2:
        codes4 = np.concatenate([codes4, np.zeros((lines, 1), dtype=np.uint8)], axis=1)
    packed = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def quantize_ref(x_bits, axis="row", grid=E2M1, rounding=RTNE, seed=0,
                 had_n=0, had_kind="det", had_seed=0, block=32, lines=None):
    """Quantize a (rows, cols) bf16 tensor row-wise, column-wise or both.

    Returns {"row": (codes, scales), "col": (codes, scales)} with the requested
    keys.  Row-wise blocks run along columns (codes (rows, cols/2)); column-wise
    blocks run along rows and are stored transposed (codes (cols, rows/2)).
    With had_kind "rand" every rotation uses the same sign vector from had_seed.
    lines (one axis only): quantize just these output lines (rows for "row",
    columns for "col"), in that order; the result equals those lines of the
    whole output.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    assert axis in ("row", "col", "both")
    assert lines is None or axis != "both"
    signs = rht_signs(had_n, had_seed) if (had_n and had_kind == "rand") else None
    out = {}
    if axis in ("row", "both"):
        src = x_bits if lines is None else x_bits[np.asarray(lines)]
        out["row"] = quantize_lines(src, grid, rounding, seed, STREAM_ROW_SR, had_n, signs, block, lines)
    if axis in ("col", "both"):
        src = x_bits.T if lines is None else x_bits[:, np.asarray(lines)].T
        out["col"] = quantize_lines(np.ascontiguousarray(src), grid, rounding, seed,
                                    STREAM_COL_SR, had_n, signs, block, lines)
    return out


# ---------------------------------------------------------------------------
# Scalar, exact-arithmetic forms of the cast, for pinning the array code.

def cast_scalar(v, grid, rounding, r=0):
    """Magnitude code of one exact value v >= 0 (a Fraction), by exhaustive search.

    RTNE: the level nearest to v; on a tie the even code.  SR: round up from
    the largest level <= v iff floor(frac * 2^16) + r >= 2^16 for the 16-bit
    draw r.  Above the top level both saturate.
    """
    lv = [Fraction(x) for x in levels(grid)]
    v = Fraction(v)
    if v >= lv[-1]:
        return len(lv) - 1
    if rounding == RTNE:
        best = min(range(len(lv)), key=lambda k: (abs(v - lv[k]), k % 2))
        return best
    lo = max(k for k in range(len(lv)) if lv[k] <= v)
    frac = (v - lv[lo]) / (lv[lo + 1] - lv[lo])
    p16 = (frac * 2 ** 16).numerator // (frac * 2 ** 16).denominator
    return lo + (1 if p16 + int(r) >= 2 ** 16 else 0)
