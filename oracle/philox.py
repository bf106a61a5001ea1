"""Philox4x32-10 counter-based generator (oracle side).

Test infrastructure only: see the package docstring.

The pages require stochastic rounding that is unbiased in expectation
("Résumé Technique : TetraJet-v2", section 2.A, and "Pre-addestramento ... con
MXFP4", Metodologia), but name no random source.  The draws here come from
Philox4x32 with 10 rounds, as published by Salmon, Moraes, Dror and Shaw
("Parallel random numbers: as easy as 1, 2, 3", SC'11): a 128-bit counter, a
64-bit key, ten rounds of two 32x32->64 multiplies, and a Weyl key schedule.

This module is written from that published definition with plain numpy
uint64 arithmetic; it shares nothing with the device implementation.
"""
import numpy as np

# Round multipliers and Weyl key increments of Philox4x32 (Salmon et al. 2011).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10

_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Return the four 32-bit output words for counters (c0, c1, c2, c3) and key (k0, k1).

    Every argument may be a scalar or a numpy array (broadcast together).  One
    round maps the counter (x0, x1, x2, x3) to
        (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0));
    the key is bumped by (W0, W1) between rounds.
    """
    c = [np.asarray(v, dtype=np.uint64) & _MASK32 for v in (c0, c1, c2, c3)]
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK32
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for r in range(ROUNDS):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = m0 * c[0]          # < 2^64: exact in uint64
        p1 = m1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return tuple(v.astype(np.uint32) for v in c)


def split64(x):
    """(low 32 bits, high 32 bits) of a non-negative integer or uint64 array."""
    x = np.asarray(x, dtype=np.uint64)
    return x & _MASK32, x >> np.uint64(32)


# Counter stream numbers (third counter word).  Stream 0 draws the stochastic
# rounding words of a row-wise output, stream 1 those of a column-wise output,
# stream 2 the random sign vector of a randomized Hadamard rotation.
STREAM_ROW_SR = 0
STREAM_COL_SR = 1
STREAM_RHT_SIGNS = 2


def uniform_halfwords(seed, stream, index):
    """The 16-bit uniform draw of element ``index`` (int array) in ``stream``.

    One Philox4x32-10 call (key (seed lo, seed hi), counter (lo(i div 8),
    hi(i div 8), stream, 0)) yields 128 bits, i.e. eight 16-bit draws: element i
    takes word (i mod 8) div 2 of the call, its low half for even i and its high
    half for odd i.
    """
    index = np.asarray(index, dtype=np.uint64)
    k0, k1 = split64(np.uint64(seed))
    blk = index >> np.uint64(3)
    b0, b1 = split64(blk)
    w = philox4x32_10(b0, b1, np.uint64(stream), np.uint64(0), k0, k1)
    word = ((index & np.uint64(7)) >> np.uint64(1)).astype(np.int64)
    words = np.stack(w, axis=0).astype(np.uint64)  # (4, ...)
    picked = np.take_along_axis(words, word[None, ...], axis=0)[0]
    shift = (index & np.uint64(1)) * np.uint64(16)
    return ((picked >> shift) & np.uint64(0xFFFF)).astype(np.uint32)
