"""Pins for the oracle's GEMM on decoded values (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle.gemm import decode, gemm_ref


def _random_operand(rng, rows, k, grid_e=(120, 134)):
    codes = rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    scales = rng.integers(grid_e[0], grid_e[1], (rows, k // 32), dtype=np.uint8)
    return codes, scales


def _fraction_value(codes, scales, grid, r, k):
    byte = int(codes[r, k // 2])
    nib = byte & 0xF if k % 2 == 0 else byte >> 4
    lv = F.E2M1_LEVELS if grid == F.E2M1 else F.E1M2_LEVELS
    mag = Fraction(lv[nib & 7])
    e = int(scales[r, k // 32]) - 127
    val = mag * (Fraction(2) ** e)
    return -val if nib & 8 else val


@pytest.mark.parametrize("grid", [F.E2M1, F.E1M2])
def test_gemm_brute_force_fractions(grid):
    rng = np.random.default_rng(21)
    k = 64
    a = _random_operand(rng, 4, k)
    b = _random_operand(rng, 4, k)
    c, g = gemm_ref(*a, *b, k, grid)
    for m in range(4):
        for n in range(4):
            exact = sum(_fraction_value(*a, grid, m, kk) * _fraction_value(*b, grid, n, kk) for kk in range(k))
            absum = sum(abs(_fraction_value(*a, grid, m, kk) * _fraction_value(*b, grid, n, kk)) for kk in range(k))
            assert Fraction(c[m, n]) == exact
            assert Fraction(g[m, n]) == absum


def test_gemm_single_block_identity_and_ones():
    # K = 32, one block: A = code for 1.0 everywhere at scale 2^0 -> C = sum of B's decoded values
    a_codes = np.full((2, 16), 0x22, dtype=np.uint8)           # 1.0, 1.0
    a_scales = np.full((2, 1), 127, dtype=np.uint8)
    rng = np.random.default_rng(1)
    b_codes, b_scales = _random_operand(rng, 3, 32)
    c, g = gemm_ref(a_codes, a_scales, b_codes, b_scales, 32, F.E2M1)
    bd = decode(b_codes, b_scales, F.E2M1, 32)
    assert np.array_equal(c, np.tile(bd.sum(axis=1), (2, 1)))
    assert np.array_equal(g, np.tile(np.abs(bd).sum(axis=1), (2, 1)))


def test_gemm_row_col_subsets():
    rng = np.random.default_rng(5)
    a = _random_operand(rng, 8, 128)
    b = _random_operand(rng, 6, 128)
    c, g = gemm_ref(*a, *b, 128, F.E2M1)
    rows, cols = np.array([1, 5]), np.array([0, 3, 4])
    cs, gs = gemm_ref(*a, *b, 128, F.E2M1, rows=rows, cols=cols)
    assert np.array_equal(cs, c[np.ix_(rows, cols)]) and np.array_equal(gs, g[np.ix_(rows, cols)])


def test_decode_nan_scale():
    codes = np.zeros((1, 16), dtype=np.uint8)
    scales = np.array([[0xFF]], dtype=np.uint8)
    assert np.all(np.isnan(decode(codes, scales, F.E2M1, 32)))
