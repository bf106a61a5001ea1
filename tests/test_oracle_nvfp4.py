"""Pins of the NVFP4-style double-block oracle (oracle/nvfp4.py).

"Résumé Technique : TetraJet-v2", section 2.A (Quantification Double Bloc Non Biaisée).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle.nvfp4 import (E4M3_TABLE, e4m3_value, e4m3_nearest, e4m3_nearest_array, nvfp4_quantize_ref,
                          nvfp4_decode, INNER, OUTER)
from oracle.quantize import RTNE, SR
from block_scaled_fp4_hadamard_amd import synth


def bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_e4m3_table_against_torch():
    torch = pytest.importorskip("torch")
    codes = torch.arange(0x7F, dtype=torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(vals, E4M3_TABLE)
    assert E4M3_TABLE[-1] == 448.0 and E4M3_TABLE[1] == 2.0 ** -9 and E4M3_TABLE[8] == 2.0 ** -6


def test_vectorized_nearest_equals_exhaustive():
    rng = np.random.default_rng(1)
    q = np.concatenate([np.exp2(rng.uniform(-12, 10, 4000)),
                        (E4M3_TABLE[:-1] + E4M3_TABLE[1:]) / 2,             # every tie
                        E4M3_TABLE, [448.0, 460.0, 464.0, 1e6, 0.0]])
    got = e4m3_nearest_array(q)
    for qi, g in zip(q, got):
        assert g == e4m3_nearest(Fraction(float(qi))), qi


def test_ties_go_to_the_even_code():
    # 1.0625 lies halfway between 1 (code 0x38) and 1.125 (0x39): even code 0x38
    assert e4m3_nearest(Fraction(17, 16)) == 0x38
    # 1.1875 between 1.125 (0x39) and 1.25 (0x3A): 0x3A
    assert e4m3_nearest(Fraction(19, 16)) == 0x3A
    assert e4m3_nearest(Fraction(470)) == 0x7E                      # saturates
    assert e4m3_nearest(Fraction(1, 1024)) == 0                     # half the smallest subnormal: even (zero)


def test_outer_scale_puts_the_block_max_at_the_top_code():
    # a block whose largest |x| is the outer maximum gets the largest E4M3 scale (or one step below, from
    # s_o's rounding), and that value decodes to within one E2M1 step of itself
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 512)).astype(np.float32)
    codes, inner, outer = nvfp4_quantize_ref(bf16(x))
    xb = f32(bf16(x)).astype(np.float64)
    for r in range(6):
        for o in range(512 // OUTER):
            blk = xb[r, o * OUTER:(o + 1) * OUTER]
            j = int(np.argmax(np.abs(blk))) // INNER
            assert inner[r, o * 8 + j] in (0x7D, 0x7E)
            assert outer[r, o] == np.float32(np.max(np.abs(blk)) / 2688.0)


def test_decode_error_within_half_a_step():
    # RTNE: |x - decode| <= half the E2M1 step at x's magnitude, times the block's decoded scale
    rng = np.random.default_rng(3)
    bits = synth.activation(16, 1024, rng)
    codes, inner, outer = nvfp4_quantize_ref(bits)
    x = f32(bits).astype(np.float64)
    d = nvfp4_decode(codes, inner, outer)
    sc = np.repeat(E4M3_TABLE[inner], INNER, axis=1) * np.repeat(outer.astype(np.float64), OUTER, axis=1)
    v = np.abs(x) / sc
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    # y itself is x / (s_i s_o) rounded to fp32: allow 2^-23 relative on top of half a step
    assert np.all(np.abs(x - d) <= (step / 2) * sc * (1 + 2.0 ** -20) + np.abs(x) * 2.0 ** -22)


def test_sr_is_unbiased():
    # one value repeated with different element indices: the mean of the decoded SR values is x
    x = np.full((1, 128 * 512), 0.8, dtype=np.float32)
    x[0, ::OUTER] = 3.0                                    # fixes every outer and inner scale
    codes, inner, outer = nvfp4_quantize_ref(bf16(x), rounding=SR, seed=7)
    d = nvfp4_decode(codes, inner, outer)[0]
    sel = np.ones(d.shape, bool)
    sel[::OUTER] = False
    xv = float(f32(bf16(np.array([0.8], dtype=np.float32)))[0])
    assert abs(d[sel].mean() - xv) < 3e-3


def test_zero_and_non_finite_blocks():
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, 128:] = np.linspace(-2, 2, 128)
    bits = bf16(x)
    bits[0, 100] = 0x8000                                   # -0 in an all-zero outer block
    bits[1, 130] = 0x7F80                                   # +inf in the second outer block of row 1
    codes, inner, outer = nvfp4_quantize_ref(bits)
    assert outer[0, 0] == 0 and np.all(inner[0, :8] == 0)
    assert (codes[0, 50] & 0xF) == 0x8                      # the sign of -0 kept
    assert np.isnan(outer[1, 1]) and np.all(inner[1, 8:] == 0x7F) and np.all(codes[1, 64:] == 0)


def test_column_axis_is_the_transpose():
    rng = np.random.default_rng(4)
    bits = synth.gradient(256, 128, rng)
    a = nvfp4_quantize_ref(bits, "col", rounding=SR, seed=3)
    b = nvfp4_quantize_ref(np.ascontiguousarray(bits.T), "row", rounding=SR, seed=3)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    # SR words use stream 1 column-wise: the codes may differ from the transposed row-wise call
    assert np.array_equal(nvfp4_quantize_ref(bits, "col")[0], nvfp4_quantize_ref(np.ascontiguousarray(bits.T))[0])
