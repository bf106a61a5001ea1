"""NVFP4-style double-block quantization (oracle side).

Test infrastructure only: see the package docstring.

"Résumé Technique : TetraJet-v2", section 2.A (Quantification Double Bloc Non
Biaisée): NVFP4 groups 16 values under an 8-bit scale; an outer block of 128
values is scaled as a whole and its 16-value inner blocks are scaled locally,
which avoids a tensor-wide absmax.  Values are E2M1 (the NVFP4 element);
stochastic rounding keeps E[round(x)] = x in the backward pass.

Readings (the page gives the structure, not the arithmetic):
* inner scale: FP8 E4M3 (bias 7, largest 448, subnormals 2^-9 apart, code
  0x7F NaN), one byte per 16 values; outer scale: float32 per 128 values;
* s_o = RN32(amax_128 / 2688), 2688 = 6 * 448, so that the outer block's
  largest value reaches the top of the E4M3 x E2M1 range;
* s_i = the E4M3 value nearest to amax_16 / (6 * s_o) (ties to the even
  code; above 448 saturates to 448; the quotient taken exactly);
* y = RN32(RN64(x * RN64(1 / (s_i * s_o)))), then the MX cast of y at unit
  scale: E2M1 by RTNE or by the 16-bit stochastic rule of oracle.quantize,
  saturating at 6, sign in bit 3, element 2j in the low nibble, the 16-bit
  Philox draw of element i of the output's logical row-major order (stream 0
  row-wise, 1 column-wise);
* s_i = 0 (all-zero inner block, or underflow) gives codes that keep only the
  sign; s_o = 0 (an all-zero outer block) gives s_i = 0;
* an outer block holding Inf or NaN gets s_o = NaN, inner scales 0x7F and zero
  codes.
"""
from fractions import Fraction

import numpy as np

from .formats import E2M1, bf16_bits_to_f64
from .quantize import quantize_values, RTNE
from .philox import STREAM_ROW_SR, STREAM_COL_SR

INNER = 16
OUTER = 128
E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_value(code):
    """Value of a positive E4M3 code 0x00..0x7E from its bit fields (bias 7)."""
    e, m = code >> 3, code & 7
    return m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(0x7F)])


def e4m3_nearest(q):
    """E4M3 code of the value nearest to q >= 0 (exact Fraction or float): ties to the even code, saturating."""
    q = Fraction(q)
    if q >= Fraction(E4M3_MAX):
        return 0x7E
    best = None
    for c in range(0x7F):
        d = abs(Fraction(float(E4M3_TABLE[c])) - q)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def e4m3_nearest_array(q):
    """Vectorized e4m3_nearest on float64 quotients q = amax / (6 s_o).

    The decision equals the exact one: the midpoints between E4M3 values have
    at most 5 significant bits and the exact quotient of an 8-bit amax by
    6 s_o (26 bits) differs from such a midpoint, when it is not equal, by more
    than 2^-31 of it, far above float64's rounding, so the float64 quotient
    falls on the same side of every midpoint and equals one only when the
    exact quotient does.
    """
    q = np.asarray(q, dtype=np.float64)
    mids = (E4M3_TABLE[:-1] + E4M3_TABLE[1:]) / 2.0            # exact
    idx = np.searchsorted(mids, q, side="left")                 # midpoints strictly below q
    at = np.minimum(idx, len(mids) - 1)
    tie = (idx < len(mids)) & (q == mids[at])
    code = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    return np.where(q >= E4M3_MAX, 0x7E, np.minimum(code, 0x7E)).astype(np.uint8)


def _lines(x_bits, axis):
    b = np.asarray(x_bits, dtype=np.uint16)
    return b if axis == "row" else np.ascontiguousarray(b.T)


def nvfp4_quantize_ref(x_bits, axis="row", rounding=RTNE, seed=0, lines=None):
    """Double-block quantization along one axis.

    Returns (codes (L, K/2) uint8, inner scales (L, K/16) uint8 E4M3, outer scales (L, K/128) float32).
    lines: only these output lines (their stochastic-rounding indices keep their place).
    """
    src = _lines(x_bits, axis)
    n_lines, k = src.shape
    assert k % OUTER == 0
    ids = np.arange(n_lines) if lines is None else np.asarray(lines)
    x = bf16_bits_to_f64(src[ids])                         # exact
    nl = len(ids)
    xo = x.reshape(nl, k // OUTER, OUTER)
    finite_o = np.isfinite(xo).all(axis=2)
    amax_o = np.where(finite_o, np.abs(np.where(np.isfinite(xo), xo, 0)).max(axis=2), 0.0)
    s_o = np.where(finite_o, (amax_o / 2688.0).astype(np.float32), np.float32(np.nan)).astype(np.float32)

    xi = x.reshape(nl, k // INNER, INNER)
    amax_i = np.abs(np.where(np.isfinite(xi), xi, 0)).max(axis=2)
    so_i = np.repeat(s_o, OUTER // INNER, axis=1).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where((so_i > 0) & (amax_i > 0), amax_i / (6.0 * np.where(so_i > 0, so_i, 1.0)), 0.0)
    inner = np.where(np.isnan(so_i), E4M3_NAN, e4m3_nearest_array(q)).astype(np.uint8)
    si = np.where(inner == E4M3_NAN, np.nan, E4M3_TABLE[np.minimum(inner, 0x7E)])
    d = si * so_i                                          # exact in float64 (4 x 24 significant bits)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = np.where(d > 0, 1.0 / np.where(d > 0, d, 1.0), 0.0)
        y = (xi * r[:, :, None]).astype(np.float32)       # RN64 product, then RN32
    # s_i = 0 keeps only the sign: a signed zero carries it through the cast
    y = np.where((d == 0)[:, :, None], np.copysign(0.0, xi), y).astype(np.float32)
    bad = ~np.repeat(finite_o, OUTER // INNER, axis=1)
    y = np.where(bad[:, :, None], np.float32(np.nan), y).reshape(nl, k).astype(np.float32)
    # the MX cast of y at unit scale: 16-value blocks whose absmax is forced to give scale byte 127
    stream = STREAM_ROW_SR if axis == "row" else STREAM_COL_SR
    codes = _cast_unit_scale(y, rounding, seed, stream, ids, k)
    codes = np.where(np.repeat(bad, INNER // 2, axis=1), 0, codes).astype(np.uint8)
    return codes, inner, s_o


def _cast_unit_scale(y, rounding, seed, stream, ids, k):
    """E2M1 codes of y at scale 2^0 (RTNE or SR), packed; element indices as in oracle.quantize."""
    from .quantize import rtne_magnitude_codes, sr_magnitude_codes
    from .philox import uniform_halfwords
    yy = np.where(np.isfinite(y), y, 0).astype(np.float64)
    v = np.abs(yy)
    if rounding == RTNE:
        mag = rtne_magnitude_codes(v, E2M1)
    else:
        idx = ids.astype(np.uint64)[:, None] * np.uint64(k) + np.arange(k, dtype=np.uint64)[None, :]
        r = uniform_halfwords(seed, stream, idx).reshape(v.shape)
        mag = sr_magnitude_codes(v, r, E2M1)
    codes4 = ((np.signbit(y).astype(np.uint8) << 3) | mag).astype(np.uint8)
    return (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)


def nvfp4_decode(codes, inner, outer):
    """Decoded float64 values (L, K) of a double-block operand."""
    from .gemm import decode
    L, half = codes.shape
    k = half * 2
    ones = np.full((L, k // 32), 127, dtype=np.uint8)      # unit E8M0 scale: the bare E2M1 values
    v = decode(codes, ones, E2M1, k, 32)
    si = np.where(inner == E4M3_NAN, np.nan, E4M3_TABLE[np.minimum(inner, 0x7E)])
    return v * np.repeat(si, INNER, axis=1) * np.repeat(np.asarray(outer, np.float64), OUTER, axis=1)
