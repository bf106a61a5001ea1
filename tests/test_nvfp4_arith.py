"""The float64 shortcut the double-block kernel takes for its outer scale.

The kernel forms s_o = RN32(amax / 2688) as RN32(amax * RN64(1/2688)), one
multiply instead of a division.  That is exact when no bf16 amax / 2688 lies
within float64 rounding of a float32 midpoint; checked here for every finite
positive bf16 against exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np


def rn32_exact(fr):
    """float32 nearest to a positive Fraction, ties to the even significand."""
    f = np.float32(float(fr))
    best = None
    for c in (np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - fr)
        if best is None or d < best[0] or (d == best[0] and int(c.view(np.uint32)) & 1 == 0):
            best = (d, c)
    return best[1]


def test_outer_scale_product_is_exact():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    a = (bits << 16).view(np.float32).astype(np.float64)
    fast = (a * (1.0 / 2688.0)).astype(np.float32).view(np.uint32)
    for i in range(0, len(a)):
        want = rn32_exact(Fraction(float(a[i])) / 2688).view(np.uint32)
        assert fast[i] == want, hex(int(bits[i]))
