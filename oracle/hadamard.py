"""Block Hadamard rotation, deterministic or with random signs (oracle side).

Test infrastructure only: see the package docstring.

Sources, by page title and section:
* "Pre-addestramento ... con MXFP4", Metodologia: deterministic Hadamard
  rotations with 16x16 (H16) and 32x32 (H32) matrices, and randomized
  Hadamard rotations, are the stabilisers tried on the full MXFP4 pipeline;
  Contributi 2: the deterministic H16 variant restores convergence.
* "Ripensare il Bias di Shrinkage ...", Problematica and Metodologia 2, and
  "Résumé Technique : TetraJet-v2", section 2.C: the random Hadamard transform
  (RHT) spreads outliers before 4-bit quantization.

Readings (the pages fix none of these):
* H_n is the Sylvester matrix, H[i][j] = (-1)^popcount(i & j), applied
  block-diagonally in aligned chunks of n along the quantization axis,
  orthonormalised by 1/sqrt(n).
* The randomized variant multiplies by a diagonal of signs first:
  y = H_n (s * x) / sqrt(n), with one sign vector s of length n per call,
  s_j = -1 iff bit j of word 0 of Philox4x32-10(key = seed, counter = (0,0,2,0)).
* The rotated value is y = RN32(RN32(S) * RN32(1/sqrt(n))) where S is the
  EXACT sum  sum_j H[i][j] s_j x_j.  An exact zero sum gives +0.  A chunk
  holding a non-finite input gives NaN for every output of that chunk.
"""
import math

import numpy as np

from .formats import rn32_scaled_int
from .philox import philox4x32_10, split64, STREAM_RHT_SIGNS

HADAMARD_SIZES = (16, 32)


def sylvester(n):
    """Sylvester-ordered Hadamard matrix of order n (a power of two), integer entries."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bits = np.bitwise_and(i, j)
    parity = np.zeros_like(bits)
    while np.any(bits):
        parity ^= bits & 1
        bits >>= 1
    return (1 - 2 * parity).astype(np.int64)


def rht_signs(n, seed):
    """Length-n vector of +-1 for the randomized rotation, drawn from the seed."""
    k0, k1 = split64(np.uint64(seed))
    w0 = int(philox4x32_10(0, 0, STREAM_RHT_SIGNS, 0, k0, k1)[0])
    return np.array([-1 if (w0 >> j) & 1 else 1 for j in range(n)], dtype=np.int64)


def inv_sqrt_f32(n):
    """RN32(1/sqrt(n)) for n a power of two, rounded once from the exact value.

    n = 2^b.  For even b the value 2^(-b/2) is exact.  For odd b it is
    sqrt(2) * 2^(-(b+1)/2), and RN32(sqrt 2) comes from an integer square root:
    with f = floor(sqrt(2) * 2^23), round up iff sqrt(2)*2^23 > f + 1/2, i.e.
    iff 2^48 * 2 > (2f + 1)^2 (sqrt 2 is irrational, so there is no tie).
    """
    b = n.bit_length() - 1
    assert n == 1 << b
    if b % 2 == 0:
        return np.float32(math.ldexp(1.0, -b // 2))
    f = math.isqrt(2 << 46)
    if (2 << 48) > (2 * f + 1) ** 2:
        f += 1
    return np.float32(math.ldexp(f, -23 - (b + 1) // 2))


# A chunk whose nonzero bf16 inputs have biased exponents (subnormals counted
# as 1) spanning at most this many binades has every partial sum of
# +-x_j exactly representable in float64: 8 significant bits per input, at most
# 5 carry bits for 32 terms, 40 + 8 + 5 = 53.
EXACT_F64_SPAN = 40


def _bf16_fields(bits):
    bits = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = (bits >> 15) & 1
    expf = (bits >> 7) & 0xFF
    man = bits & 0x7F
    return sign, expf, man


def _exact_chunk_sums(bits_chunk, hs):
    """Exact S_i = sum_j hs[i][j] x_j for one chunk, as (integer numerator, binary exponent).

    x_j = +-(implicit bit | mantissa) * 2^(max(expf,1) - 134) exactly.
    """
    sign, expf, man = _bf16_fields(bits_chunk)
    eff = np.maximum(expf, 1)
    sig = np.where(expf > 0, man | 0x80, man)
    nz = sig != 0
    if not np.any(nz):
        return [0] * len(bits_chunk), 0
    base = int(eff[nz].min())
    ints = [(-1 if sign[j] else 1) * (int(sig[j]) << int(eff[j] - base)) if nz[j] else 0
            for j in range(len(bits_chunk))]
    sums = [sum(int(hs[i][j]) * ints[j] for j in range(len(ints))) for i in range(len(ints))]
    return sums, base - 134


def rotate_lines(bits, n, signs=None):
    """Rotate every line of a 2-D bf16 array (uint16) along its last axis.

    Returns the rotated values as float32, same shape.  The line length must be
    a multiple of n.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    lines, length = bits.shape
    assert length % n == 0
    h = sylvester(n)
    s = np.ones(n, dtype=np.int64) if signs is None else np.asarray(signs, dtype=np.int64)
    hs = h * s[None, :]                      # H diag(s): column j carries s_j
    chunks = bits.reshape(-1, n)
    x = (chunks.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)

    # S = (H diag(s)) x per chunk, in float64.  Exact where the span test passes.
    sums = x @ hs.T.astype(np.float64)

    _, expf, man = _bf16_fields(chunks)
    finite = expf != 0xFF
    nonzero = (expf != 0) | (man != 0)
    eff = np.maximum(expf, 1)
    big = np.where(nonzero & finite, eff, -1).max(axis=1)
    small = np.where(nonzero & finite, eff, 10 ** 6).min(axis=1)
    chunk_finite = finite.all(axis=1)
    inexact = chunk_finite & (big >= 0) & (big - small > EXACT_F64_SPAN)

    s32 = sums.astype(np.float32)            # RN32 of an exact float64 value: one rounding
    for c in np.nonzero(inexact)[0]:
        ints, q = _exact_chunk_sums(chunks[c], hs)
        s32[c] = np.array([rn32_scaled_int(v, q) for v in ints], dtype=np.float32)

    s32 = np.where(s32 == 0, np.float32(0.0), s32)     # exact zero -> +0
    c = inv_sqrt_f32(n)
    y = (s32.astype(np.float64) * np.float64(c)).astype(np.float32)   # product exact in f64, one rounding
    y[~chunk_finite] = np.float32(np.nan)
    return y.reshape(lines, length)
