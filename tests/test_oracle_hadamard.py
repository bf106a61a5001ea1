"""Pins for the oracle's block Hadamard rotation (CPU only)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard as Hm
from block_scaled_fp4_hadamard_amd.synth import f32_to_bf16_bits


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32])
def test_sylvester_orthogonal_symmetric_and_matches_scipy(n):
    h = Hm.sylvester(n)
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))
    assert np.array_equal(h, h.T)
    assert np.array_equal(h, scipy.linalg.hadamard(n).astype(np.int64))


def test_rht_signs_give_orthogonal_transform():
    for seed in (0, 1, 12345, 2 ** 63 + 5):
        for n in (16, 32):
            s = Hm.rht_signs(n, seed)
            assert set(np.unique(s)) <= {-1, 1}
            hd = Hm.sylvester(n) * s[None, :]
            assert np.array_equal(hd @ hd.T, n * np.eye(n, dtype=np.int64))
    # different seeds give different sign vectors
    assert not np.array_equal(Hm.rht_signs(32, 1), Hm.rht_signs(32, 2))


def _fwht_exact(vals):
    """Independent in-place fast Walsh-Hadamard transform on Fractions (Sylvester order)."""
    a = list(vals)
    h = 1
    while h < len(a):
        for i in range(0, len(a), 2 * h):
            for j in range(i, i + h):
                a[j], a[j + h] = a[j] + a[j + h], a[j] - a[j + h]
        h *= 2
    return a


def _rn32_fraction(x):
    """Nearest fp32 to an exact Fraction, ties to even, by comparing neighbours exactly."""
    if x == 0:
        return np.float32(0.0)
    f = np.float32(float(x))
    if np.isinf(f):
        return f
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        if np.isinf(cand):
            continue
        d = abs(Fraction(float(cand)) - x)
        even = (int(np.float32(cand).view(np.uint32)) & 1) == 0
        key = (d, not even)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def _bf16_to_fraction(b):
    return Fraction(float((np.array([b], dtype=np.uint32) << 16).view(np.float32)[0]))


def _rotation_reference(bits_row, n, signs):
    """y per the definition: RN32(RN32(S) * RN32(1/sqrt n)) with S the exact sum, via FWHT."""
    c = Fraction(float(Hm.inv_sqrt_f32(n)))
    out = []
    for k in range(0, len(bits_row), n):
        x = [_bf16_to_fraction(b) * int(s) for b, s in zip(bits_row[k:k + n], signs)]
        for s_exact in _fwht_exact(x):
            s32 = _rn32_fraction(s_exact)
            out.append(_rn32_fraction(Fraction(float(s32)) * c))
    return np.array(out, dtype=np.float32)


@pytest.mark.parametrize("n,kind", [(16, "det"), (32, "det"), (32, "rand"), (16, "rand")])
def test_rotation_equals_exact_fwht(n, kind):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 64)) * np.exp(rng.uniform(-6, 6, (6, 64)))
    bits = f32_to_bf16_bits(x.astype(np.float32))
    signs = Hm.rht_signs(n, 99) if kind == "rand" else np.ones(n, dtype=np.int64)
    y = Hm.rotate_lines(bits, n, signs if kind == "rand" else None)
    for r in range(bits.shape[0]):
        ref = _rotation_reference(bits[r], n, signs)
        assert y[r].tobytes() == ref.tobytes()


def test_rotation_exact_path_for_wide_exponent_span():
    # chunks whose nonzero inputs span far more than 40 binades: float64 sums would round
    n = 32
    rows = []
    vals = [1.0, 2.0 ** -24, 2.0 ** -60] + [0.0] * 29            # 1 + 2^-24 + 2^-60 > fp32 midpoint
    rows.append(vals)
    rows.append([2.0 ** 100, -2.0 ** 100, 2.0 ** -100] + [3.0 * 2.0 ** -120] * 29)
    rows.append([1e30, -1e30] + list(np.geomspace(1e-30, 1e-3, 30)))
    bits = f32_to_bf16_bits(np.array(rows, dtype=np.float32))
    y = Hm.rotate_lines(bits, n)
    for r in range(len(rows)):
        ref = _rotation_reference(bits[r], n, np.ones(n, dtype=np.int64))
        assert y[r].tobytes() == ref.tobytes()
    # the first output is RN32(S)/sqrt(32) with S rounded up past the midpoint
    s32 = np.float32(1.0 + 2.0 ** -23)
    assert y[0, 0] == np.float32(np.float64(s32) * np.float64(Hm.inv_sqrt_f32(32)))


def test_rotation_preserves_norm_and_cancels():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    w = rng.standard_normal((8, 128)).astype(np.float32)
    xb, wb = f32_to_bf16_bits(x), f32_to_bf16_bits(w)
    xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wv = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for n in (16, 32):
        s = Hm.rht_signs(n, 3)
        xr = Hm.rotate_lines(xb, n, s).astype(np.float64)
        wr = Hm.rotate_lines(wb, n, s).astype(np.float64)
        assert np.allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(xv, axis=1), rtol=1e-6)
        # the same rotation on both operands along K cancels in the product
        assert np.allclose(xr @ wr.T, xv @ wv.T, rtol=1e-5, atol=1e-4)
        # exact-arithmetic cancellation of the transform itself
        hd = Hm.sylvester(n) * s[None, :]
        blk = np.kron(np.eye(128 // n, dtype=np.int64), hd)
        assert np.allclose((xv @ blk.T) @ (wv @ blk.T).T / n, xv @ wv.T, rtol=1e-12, atol=1e-9)


def test_rotation_zero_sum_is_positive_zero_and_nonfinite_chunk_is_nan():
    bits = np.zeros((2, 32), dtype=np.uint16)
    bits[0, :] = 0x8000                                   # all -0
    bits[1, 0] = 0x7F80                                   # +inf in the chunk
    y = Hm.rotate_lines(bits, 32)
    assert np.all(y[0] == 0) and not np.any(np.signbit(y[0]))
    assert np.all(np.isnan(y[1]))


def test_inv_sqrt_constants():
    assert Hm.inv_sqrt_f32(16) == np.float32(0.25)
    c = Hm.inv_sqrt_f32(32)
    exact = 1 / math.sqrt(32)
    up = np.nextafter(c, np.float32(1)); dn = np.nextafter(c, np.float32(0))
    assert abs(float(c) - exact) <= min(abs(float(up) - exact), abs(float(dn) - exact))
