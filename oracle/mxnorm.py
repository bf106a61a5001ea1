"""MXNorm: row normalization estimated from the MX block maxima, fused with the cast (oracle side).

Test infrastructure only: see the package docstring.

"MXNorm: Reusing MXFP block scales for efficient tensor normalisation",
Sommario tecnico 2 (Metodologia): RMSNorm's inverse RMS of a row is replaced
by an estimate built from the block absolute maxima that the MX cast computes
anyway,

    rho_t = c(p, B) * ( (1/K) * sum_k m_tk^p )^(-1/p),

with m_tk the absmax of block k of row t, K blocks of B = 32 elements,
p = 1 or 2 (Implementazione 2), and c(p, B) a correction constant that the
pages obtain by Monte Carlo.  Normalization and cast are one operation
(Implementazione 1) and the gain is folded into the next layer's weights
(Implementazione 4), so the values cast are x * rho_t.  Section 3 (Teorema 1)
states that the generalized mean of the block maxima of i.i.d. values
converges to the RMS up to a constant; c(p, B) is that constant.

Readings where the pages leave the arithmetic open:
* m_tk is the absmax of the bf16 input block, a NaN counting as +inf;
* S_t = sum_k m_tk^p in float64, added as a balanced binary tree over the
  blocks in order (neighbours, then pairs of pairs, ...), the block count
  padded with zeros to a power of two; every addition rounds to float64;
* q_t = RN64(S_t / K);
* rho_t = RN32 of the exact real number c * q_t^(-1/p), c a float32 (ties to
  even; overflow to +inf); rho_t = 0 when q_t is 0 (an all-zero row) or +inf;
* the cast values are y = RN32(x * rho_t), quantized row-wise exactly as
  oracle.quantize does (block absmax of y, E8M0 scale, RTNE or SR with
  stream 0, pack);
* c(p, B) is (E[M^p])^(1/p) for M the largest |value| of B independent
  standard normal values, which makes rho_t -> 1/RMS for i.i.d. normal rows.
"""
import math
from fractions import Fraction

import numpy as np

from .formats import E2M1, bf16_bits_to_f64
from .quantize import quantize_values, RTNE
from .philox import STREAM_ROW_SR

BLOCK = 32
POWERS = (1, 2)


def block_maxima(bits):
    """(rows, K) float64 absmax of every 32-block of a (rows, cols) bf16 array; NaN counts as +inf."""
    x = bf16_bits_to_f64(np.asarray(bits, dtype=np.uint16))
    rows, cols = x.shape
    assert cols % BLOCK == 0
    a = np.abs(x)
    a = np.where(np.isnan(a), np.inf, a)
    return a.reshape(rows, cols // BLOCK, BLOCK).max(axis=2)


def tree_sum(values):
    """Balanced binary-tree sum in float64 of a 1-D sequence, padded with zeros to a power of two."""
    v = [float(t) for t in values]
    n = 1
    while n < len(v):
        n *= 2
    v += [0.0] * (n - len(v))
    while len(v) > 1:
        v = [v[i] + v[i + 1] for i in range(0, len(v), 2)]   # each sum rounds to float64
    return v[0] if v else 0.0


def _rn32_positive(cmp, guess):
    """RN32 of a positive real z, given cmp(t) = sign(t - z) for dyadic t and a float32 near z."""
    f = np.float32(guess)
    if not np.isfinite(f) or f <= 0:
        f = np.float32(np.finfo(np.float32).max) if not f > 0 else np.float32(np.finfo(np.float32).tiny)
    big = Fraction(2) ** 128 - Fraction(2) ** 103           # the smallest value that rounds to +inf
    if cmp(big) <= 0:
        return np.float32(np.inf)
    for _ in range(64):
        up = np.nextafter(f, np.float32(np.inf))
        dn = np.nextafter(f, np.float32(0))
        hi = (Fraction(float(f)) + Fraction(float(up))) / 2 if np.isfinite(up) else big
        lo = (Fraction(float(f)) + Fraction(float(dn))) / 2
        ch, cl = cmp(hi), cmp(lo)
        if ch < 0:                       # hi < z: move up
            f = up
        elif cl > 0:                     # lo > z: move down
            f = dn
        elif ch == 0:                    # z is the midpoint above f: ties to even
            return f if (f.view(np.uint32) & 1) == 0 else up
        elif cl == 0:
            return f if (f.view(np.uint32) & 1) == 0 else dn
        else:
            return f
    raise AssertionError("RN32 search did not converge")


def inverse_rms_estimate(m_row, p, c):
    """rho_t of one row from its block maxima (float64 array), p in (1, 2), c a float32."""
    assert p in POWERS
    k = len(m_row)
    s = tree_sum(np.asarray(m_row, dtype=np.float64) ** p)    # m^p exact in float64 (m has 8 significant bits)
    q = s / k
    if q == 0.0 or math.isinf(q):
        return np.float32(0.0)
    cf, qf = Fraction(float(np.float32(c))), Fraction(q)
    if p == 1:
        z = cf / qf                                           # the exact value

        def cmp(t):
            return (t > z) - (t < z)
        guess = float(cf) / q
    else:
        z2 = cf * cf / qf                                     # z^2; compare squares (all positive)

        def cmp(t):
            t2 = t * t
            return (t2 > z2) - (t2 < z2)
        guess = float(cf) / math.sqrt(q)
    return _rn32_positive(cmp, guess)


def mxnorm_quantize_ref(x_bits, p=2, c=1.0, grid=E2M1, rounding=RTNE, seed=0, lines=None):
    """Normalize every row by its estimated inverse RMS and quantize it row-wise.

    Returns (codes, scales, rho): codes (rows, cols/2), scales (rows, cols/32),
    rho (rows,) float32.  lines: only these rows (SR indices keep their place).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    ids = np.arange(rows) if lines is None else np.asarray(lines)
    sub = x_bits[ids]
    m = block_maxima(sub)
    rho = np.array([inverse_rms_estimate(m[i], p, c) for i in range(len(ids))], dtype=np.float32)
    x = bf16_bits_to_f64(sub).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        y = (x.astype(np.float64) * rho.astype(np.float64)[:, None]).astype(np.float32)  # product exact, one rounding
    codes, scales = quantize_values(y, grid, rounding, seed, STREAM_ROW_SR, BLOCK, ids)
    return codes, scales, rho


def correction_constant(p, block=BLOCK):
    """c(p, B) = E[M^p]^(1/p), M = max of B independent |N(0,1)| values, by numerical integration.

    P(M > x) = 1 - erf(x / sqrt 2)^B, and E[M^p] = integral over x > 0 of p x^(p-1) P(M > x).
    """
    from scipy.integrate import quad
    f = lambda x: p * x ** (p - 1) * (1.0 - math.erf(x / math.sqrt(2.0)) ** block)
    val, _ = quad(f, 0.0, 40.0, limit=200, epsabs=1e-13, epsrel=1e-12)
    return val ** (1.0 / p)
