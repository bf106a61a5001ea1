"""Pins for the oracle's grids, block scale and cast (CPU only)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle.quantize import (rtne_magnitude_codes, sr_magnitude_codes, block_scale_exponents,
                             cast_scalar, RTNE, SR)


# ---- grids: two derivations must agree --------------------------------------

def test_e2m1_levels_match_bitfield():
    assert [F.e2m1_bitfield_value(k) for k in range(8)] == list(F.E2M1_LEVELS)


def test_e1m2_levels_match_bitfield_and_are_uniform():
    assert [F.e1m2_bitfield_value(k) for k in range(8)] == list(F.E1M2_LEVELS)
    d = np.diff(F.E1M2_LEVELS)
    assert np.all(d == d[0])          # equal left and right bin widths


def test_e2m1_is_non_uniform():
    d = np.diff(F.E2M1_LEVELS)
    assert d[0] == 0.5 and d[3] == 0.5 and d[4] == 1.0 and d[6] == 2.0


# ---- E8M0 decode against torch's float8_e8m0fnu ------------------------------

def test_e8m0_decode_matches_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).float().double().numpy()
    ours = np.array([F.e8m0_value(int(x)) for x in range(256)])
    assert np.isnan(ref[255]) and np.isnan(ours[255])
    assert np.array_equal(ref[:255], ours[:255])


# ---- scale rule over every bf16 value -----------------------------------------

def _all_positive_finite_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)    # +subnormals .. +max finite
    return (bits << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("grid,lo,hi", [(F.E2M1, 4.0, 8.0), (F.E1M2, 1.0, 2.0)])
def test_scale_rule_exhaustive_bf16(grid, lo, hi):
    a = _all_positive_finite_bf16()
    e = block_scale_exponents(a, grid)
    e_scalar = np.array([F.scale_exponent(x, grid) for x in a[::97]])
    assert np.array_equal(e[::97], e_scalar)
    v = np.ldexp(a, -e)
    unclamped = e > F.SCALE_EXP_MIN
    assert np.all((v[unclamped] >= lo) & (v[unclamped] < hi))
    # clamped blocks: floor(log2 amax) - emax fell below -127
    fl = np.array([math.frexp(x)[1] - 1 for x in a[~unclamped]])
    assert np.all(fl - F.EMAX[grid] <= F.SCALE_EXP_MIN)
    assert np.all(v < hi)


def test_scale_of_zero_block_is_smallest():
    assert F.scale_exponent(0.0, F.E2M1) == -127
    assert block_scale_exponents(np.array([0.0]), F.E2M1)[0] == -127
    assert F.e8m0_byte(-127) == 0


def test_scale_examples():
    # 2^(floor(log2 amax) - 2): amax 6 -> e 0, amax 1 -> e -2, amax 8 -> e 1
    assert F.scale_exponent(6.0, F.E2M1) == 0
    assert F.scale_exponent(1.0, F.E2M1) == -2
    assert F.scale_exponent(8.0, F.E2M1) == 1
    assert F.scale_exponent(1.5, F.E1M2) == 0


# ---- RTNE: tie table and exhaustive nearest-level search -----------------------

E2M1_TIES = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}


def test_rtne_tie_table_e2m1():
    v = np.array(list(E2M1_TIES))
    codes = rtne_magnitude_codes(v, F.E2M1)
    assert [F.E2M1_LEVELS[c] for c in codes] == list(E2M1_TIES.values())


def test_rtne_tie_table_e1m2():
    v = np.array([(2 * k + 1) / 8 for k in range(7)])
    codes = rtne_magnitude_codes(v, F.E1M2)
    assert list(codes) == [k if k % 2 == 0 else k + 1 for k in range(7)]


def test_rtne_saturates():
    assert list(rtne_magnitude_codes(np.array([6.0, 6.5, 7.0, 7.999]), F.E2M1)) == [7] * 4
    assert list(rtne_magnitude_codes(np.array([1.75, 1.875, 1.99]), F.E1M2)) == [7] * 3


@pytest.mark.parametrize("grid", [F.E2M1, F.E1M2])
def test_rtne_exhaustive_against_brute_force(grid):
    # every bf16 magnitude in [0, top*4/3) against an exhaustive Fraction search
    bits = np.arange(0, 0x4100, dtype=np.uint32)
    v = (bits << 16).view(np.float32).astype(np.float64)
    v = v[v < (8.0 if grid == F.E2M1 else 2.0)]
    got = rtne_magnitude_codes(v, grid)
    want = np.array([cast_scalar(Fraction(x), grid, RTNE) for x in v])
    assert np.array_equal(got, want)


# ---- shrinkage bias closed form ------------------------------------------------

def _bias_on_bin(grid, i, top_limit):
    lv = np.array(F.E2M1_LEVELS if grid == F.E2M1 else F.E1M2_LEVELS)
    q = lv[i]
    left = (lv[i] - lv[i - 1]) / 2 if i > 0 else 0.0          # magnitude space: bin of 0 starts at 0
    right = (lv[i + 1] - lv[i]) / 2 if i < 7 else (top_limit - lv[i])
    a, b = q - left, q + right
    n = 1 << 20
    v = a + (np.arange(n) + 0.5) * (b - a) / n                  # midpoint lattice: no endpoint ties
    codes = rtne_magnitude_codes(v, grid)
    return np.mean(lv[codes] - v), (left - right) / 2


@pytest.mark.parametrize("grid,top", [(F.E2M1, 8.0), (F.E1M2, 2.0)])
def test_shrinkage_bias_closed_form(grid, top):
    # Expected RTNE error at level q_i under locally uniform density is (l_i - r_i)/2.
    for i in range(8):
        got, closed = _bias_on_bin(grid, i, top)
        assert abs(got - closed) < 1e-12, (grid, i, got, closed)


def test_shrinkage_values_e2m1():
    expect = {0: -0.125, 1: 0.0, 2: 0.0, 3: 0.0, 4: -0.125, 5: 0.0, 6: -0.25, 7: -0.5}
    for i, want in expect.items():
        got, _ = _bias_on_bin(F.E2M1, i, 8.0)
        assert abs(got - want) < 1e-12, (i, got)


def test_uniform_grid_has_no_interior_bias():
    for i in range(1, 7):
        got, _ = _bias_on_bin(F.E1M2, i, 2.0)
        assert abs(got) < 1e-12


# ---- SR: array form against the exact scalar form ----------------------------

@pytest.mark.parametrize("grid", [F.E2M1, F.E1M2])
def test_sr_array_matches_scalar(grid):
    rng = np.random.default_rng(7)
    top = 8.0 if grid == F.E2M1 else 2.0
    v = np.concatenate([rng.uniform(0, top, 4000), np.ldexp(rng.uniform(0.5, 1, 200), -rng.integers(10, 140, 200))])
    v = v.astype(np.float32).astype(np.float64)
    r = rng.integers(0, 2 ** 16, v.size, dtype=np.uint64)
    got = sr_magnitude_codes(v, r, grid)
    want = np.array([cast_scalar(Fraction(float(x)), grid, SR, int(w)) for x, w in zip(v, r)])
    assert np.array_equal(got, want)


def test_sr_threshold_is_floor_of_fixed_point_probability():
    # frac = 1/3 cannot be held in 16 bits: P16 = floor(2^16 / 3) = 21845, and v rounds up iff the 16-bit
    # draw reaches 2^16 - P16 = 43691
    v = np.array([0.5 + 0.5 / 3])      # float64 rounding of 2/3 keeps P16's floor value
    assert int(np.floor((v[0] - 0.5) / 0.5 * 2 ** 16)) == 21845
    assert sr_magnitude_codes(v, np.array([43691]), F.E2M1)[0] == 2
    assert sr_magnitude_codes(v, np.array([65535]), F.E2M1)[0] == 2
    assert sr_magnitude_codes(v, np.array([43690]), F.E2M1)[0] == 1
    assert sr_magnitude_codes(v, np.array([0]), F.E2M1)[0] == 1
    assert sr_magnitude_codes(np.array([1.0]), np.array([65535]), F.E2M1)[0] == 2   # on a level: unchanged
    # the probability is the 16-bit truncated fraction: exactly P16 of the 2^16 draws round up, so the
    # bias is 1/3 - 21845 / 2^16 = 1 / (3 * 2^16), below 2^-16 of the step
    r = np.arange(0, 2 ** 16, dtype=np.uint64)
    ups = sr_magnitude_codes(np.full(r.shape, v[0]), r, F.E2M1) == 2
    assert ups.sum() == 21845
    bias = Fraction(1, 3) - Fraction(int(ups.sum()), 2 ** 16)
    assert 0 < bias < Fraction(1, 2 ** 16)


# ---- exact fp32 rounding of wide sums ------------------------------------------

def test_rn32_scaled_int_matches_numpy_when_f64_exact():
    rng = np.random.default_rng(3)
    for _ in range(3000):
        n = int(rng.integers(-(1 << 52), 1 << 52))
        q = int(rng.integers(-190, 100))
        exact64 = math.ldexp(n, q)                  # n < 2^53: exact in float64
        assert F.rn32_scaled_int(n, q).tobytes() == np.float32(exact64).tobytes() or \
            (np.isinf(np.float32(exact64)) and np.isinf(F.rn32_scaled_int(n, q)))


def test_rn32_scaled_int_needs_more_than_f64():
    # 1 + 2^-24 + 2^-80: above the fp32 midpoint, so it rounds up; float64 would lose 2^-80 and tie to even
    n = (1 << 80) + (1 << 56) + 1
    assert F.rn32_scaled_int(n, -80) == np.float32(1.0 + 2.0 ** -23)
    assert np.float32(math.ldexp(n, -80)) == np.float32(1.0)
    assert F.rn32_scaled_int(-n, -80) == -np.float32(1.0 + 2.0 ** -23)
    assert F.rn32_scaled_int(0, 5).tobytes() == np.float32(0.0).tobytes()
    assert np.isinf(F.rn32_scaled_int(1, 128))
