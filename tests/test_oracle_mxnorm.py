"""Pins of the MXNorm oracle (oracle/mxnorm.py) against closed forms, the pages' theorem and invariants.

"MXNorm: Reusing MXFP block scales for efficient tensor normalisation", Sommario tecnico 2 and 3.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle.formats import E2M1, E1M2
from oracle.mxnorm import (block_maxima, tree_sum, inverse_rms_estimate, mxnorm_quantize_ref,
                           correction_constant)
from oracle.quantize import quantize_ref, RTNE, SR
from block_scaled_fp4_hadamard_amd import synth


def bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_correction_constant_closed_forms():
    # one value per block: E[Z^2] = 1 and E|Z| = sqrt(2/pi)
    assert correction_constant(2, 1) == pytest.approx(1.0, abs=1e-12)
    assert correction_constant(1, 1) == pytest.approx(math.sqrt(2.0 / math.pi), abs=1e-12)
    # two values: max(U, V) = (U + V)/2 + |U - V|/2 for U, V chi-square(1); U - V = 2AB with A, B
    # independent N(0,1), so E[max] = 1 + E|A| E|B| = 1 + 2/pi
    assert correction_constant(2, 2) == pytest.approx(math.sqrt(1.0 + 2.0 / math.pi), abs=1e-12)
    # more values per block: a larger maximum
    assert correction_constant(2, 32) > correction_constant(2, 2) > 1.0


def test_tree_sum_order():
    # neighbours first: (2^54 + 1) and (2^54 + 2) both round back to 2^54 (ulp 4, ties to even), while
    # the three pairs of ones reach 4 and add exactly at the top; a left-to-right sum stays at 2^54
    vals = [2.0 ** 54] + [1.0] * 7
    assert tree_sum(vals) == 2.0 ** 54 + 4.0
    seq = 0.0
    for v in vals:
        seq += v
    assert seq == 2.0 ** 54
    # padding with zeros to a power of two changes nothing
    a, b, c, d, e = 0.1, 0.2, 0.3, 0.4, 0.5
    assert tree_sum([a, b, c, d, e]) == ((a + b) + (c + d)) + e


def nearest_f32(z):
    """RN32 of a positive Decimal by comparing distances to neighbouring float32 values (ties to even)."""
    f = np.float32(float(z))
    best = None
    for cand in (np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Decimal(float(cand)) - z)
        key = (d, int(cand.view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


@pytest.mark.parametrize("p", [1, 2])
def test_rho_is_nearest_float32_of_the_exact_value(p):
    getcontext().prec = 60
    rng = np.random.default_rng(3)
    for _ in range(300):
        k = int(rng.integers(1, 200))
        m = bf16(np.abs(rng.standard_normal(k)) * 2.0 ** rng.integers(-20, 20)).astype(np.uint16)
        mv = block_maxima(np.repeat(m[None, :], 32, axis=0).T.reshape(1, -1))[0]   # each block = one value
        c = np.float32(rng.uniform(0.5, 3.0))
        s = tree_sum(mv ** p)
        q = s / k
        z = Decimal(float(c)) / (Decimal(q) if p == 1 else Decimal(q).sqrt())
        assert inverse_rms_estimate(mv, p, c) == nearest_f32(z)


@pytest.mark.parametrize("p", [1, 2])
def test_equal_block_maxima(p):
    # every block has the same absmax m: the mean of m^p is m^p, so rho = RN32(c / m); 96 blocks (not a
    # power of two) also checks the division by K rather than by the padded count
    getcontext().prec = 60
    rng = np.random.default_rng(4)
    m = np.float32(3.25)
    x = rng.uniform(-1, 1, (3, 96 * 32)).astype(np.float32) * m * 0.9
    x[:, ::32] = m
    x[1, 5::32] = -m
    c = np.float32(2.3894571)
    _, _, rho = mxnorm_quantize_ref(bf16(x), p=p, c=c)
    want = nearest_f32(Decimal(float(c)) / Decimal(float(m)))
    assert np.all(rho == want)


@pytest.mark.parametrize("p", [1, 2])
@pytest.mark.parametrize("sigma", [1.0, 3.0e-3, 40.0])
def test_estimate_converges_to_inverse_rms(p, sigma):
    # Teorema 1: for i.i.d. rows the generalized mean of the block maxima tends to the RMS times c(p, B);
    # with c = c(p, 32) the estimate tends to 1/RMS.  K = 2048 blocks: a few tenths of a percent of
    # sampling error.
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 2048 * 32)) * sigma
    c = np.float32(correction_constant(p))
    m = block_maxima(bf16(x))
    rms = np.sqrt(np.mean(f32(bf16(x)).astype(np.float64) ** 2, axis=1))
    for i in range(4):
        rho = inverse_rms_estimate(m[i], p, c)
        assert abs(float(rho) * rms[i] - 1.0) < 0.02


@pytest.mark.parametrize("rounding", [RTNE, SR])
def test_power_of_two_scaling_is_invisible(rounding):
    rng = np.random.default_rng(6)
    x = f32(synth.activation(8, 512, rng))
    c = np.float32(2.39)
    base = mxnorm_quantize_ref(bf16(x), p=2, c=c, rounding=rounding, seed=3)
    for j in (-7, 5, 30):
        got = mxnorm_quantize_ref(bf16(x * 2.0 ** j), p=2, c=c, rounding=rounding, seed=3)
        assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1])
        assert np.array_equal(got[2], (base[2] * np.float32(2.0 ** -j)).astype(np.float32))


@pytest.mark.parametrize("grid", [E2M1, E1M2])
@pytest.mark.parametrize("rounding", [RTNE, SR])
def test_unit_estimate_matches_plain_quantizer(grid, rounding):
    # every block's absmax is 1 and c = 1: rho = 1, so the codes are the plain quantizer's
    rng = np.random.default_rng(7)
    x = rng.uniform(-1, 1, (6, 256)).astype(np.float32)
    x[:, ::32] = 1.0
    x[2, 1::32] = -1.0
    bits = bf16(x)
    for p in (1, 2):
        codes, scales, rho = mxnorm_quantize_ref(bits, p=p, c=1.0, grid=grid, rounding=rounding, seed=11)
        assert np.all(rho == 1.0)
        want = quantize_ref(bits, "row", grid=grid, rounding=rounding, seed=11)["row"]
        assert np.array_equal(codes, want[0]) and np.array_equal(scales, want[1])


def test_output_bound():
    # Sommario tecnico 3 (limits): with p = 2 the largest normalized value is at most c * sqrt(K), as
    # max_k m_k <= sqrt(sum_k m_k^2); with p = 1 at most c * K
    rng = np.random.default_rng(8)
    x = f32(synth.activation(16, 2048, rng, outlier_count=3))
    x[3, 100] = 1e4
    bits = bf16(x)
    k = 2048 // 32
    for p, bound in ((2, math.sqrt(k)), (1, k)):
        c = np.float32(2.35)
        _, _, rho = mxnorm_quantize_ref(bits, p=p, c=c)
        ymax = np.max(np.abs(f32(bits)) * rho[:, None], axis=1)
        assert np.all(ymax <= float(c) * bound * (1 + 2.0 ** -20))


def test_zero_and_nonfinite_rows():
    x = np.zeros((3, 64), dtype=np.float32)
    x[1] = np.linspace(-1, 1, 64)
    bits = bf16(x)
    bits[1, 40] = 0x7F80                      # +inf in block 1 of row 1
    codes, scales, rho = mxnorm_quantize_ref(bits, p=2, c=2.0)
    assert rho[0] == 0.0 and rho[2] == 0.0 and rho[1] == 0.0
    assert np.all(codes[0] == 0) and np.all(scales[0] == 0)
    assert scales[1, 1] == 0xFF and np.all(codes[1, 16:32] == 0)
    assert scales[1, 0] == 0                  # finite values times 0
