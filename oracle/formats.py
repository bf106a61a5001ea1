"""Element grids, the shared power-of-two block scale, and exact fp32 rounding.

Test infrastructure only: see the package docstring.

Sources, by page title and section:
* "Ripensare il Bias di Shrinkage nel Pretraining di LLM in FP4", Problematica
  and Metodologia 1: E2M1 has two exponent bits and one mantissa bit, so its
  magnitudes are non-uniform (0.5, 1, 1.5, ... with the spacing growing).
  Metodologia 2 (La Ricetta UFP4): the uniform E1M2/INT4 grid, equal spacing.
* "MXNorm: Reusing MXFP block scales ...", Sommario tecnico 2: each block gets
  one shared scale derived from its absolute maximum.
The block size 32, the E8M0 scale byte and the rule
scale = 2^(floor(log2 amax) - emax) are the OCP MX layout, which the pages use
by name without spelling it out.
"""
import math

import numpy as np

E2M1 = "e2m1"
E1M2 = "e1m2"
GRIDS = (E2M1, E1M2)

# The E2M1 magnitudes (two exponent bits, one mantissa bit), by 3-bit code.
E2M1_LEVELS = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
# The uniform grid: code k is k/4 (E1M2 with exponent bias 1, or a
# sign-magnitude INT4 scaled by 1/4).
E1M2_LEVELS = tuple(k / 4 for k in range(8))

# floor(log2) of the largest level, so that amax / 2^e lands in the top binade.
EMAX = {E2M1: 2, E1M2: 0}

E8M0_BIAS = 127
E8M0_NAN = 0xFF
SCALE_EXP_MIN = -127
SCALE_EXP_MAX = 127


def e2m1_bitfield_value(code):
    """Magnitude of a 3-bit E2M1 code from its bit fields (exponent bias 1)."""
    exp, man = code >> 1, code & 1
    if exp == 0:                      # subnormal: 0.man x 2^(1-bias)
        return 0.5 * man
    return 2.0 ** (exp - 1) * (1.0 + man / 2.0)


def e1m2_bitfield_value(code):
    """Magnitude of a 3-bit E1M2 code from its bit fields (exponent bias 1)."""
    exp, man = code >> 2, code & 3
    if exp == 0:
        return man / 4.0              # 0.man x 2^0 with two mantissa bits
    return 1.0 + man / 4.0


def levels(grid):
    return np.array(E2M1_LEVELS if grid == E2M1 else E1M2_LEVELS, dtype=np.float64)


def floor_log2(a):
    """Exact floor(log2 a) for a finite a > 0 (frexp is exact, also for subnormals)."""
    _, ex = math.frexp(a)
    return ex - 1


def scale_exponent(amax, grid):
    """Shared block exponent e: floor(log2 amax) - emax, clamped to [-127, 127].

    An all-zero block (amax = 0) takes the smallest exponent, -127.
    """
    if amax == 0.0:
        return SCALE_EXP_MIN
    return max(SCALE_EXP_MIN, min(SCALE_EXP_MAX, floor_log2(float(amax)) - EMAX[grid]))


def e8m0_byte(e):
    return e + E8M0_BIAS


def e8m0_value(byte):
    """2^(byte - 127); 0xFF is the E8M0 NaN."""
    if byte == E8M0_NAN:
        return float("nan")
    return math.ldexp(1.0, int(byte) - E8M0_BIAS)


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16 array) -> exact float64 values."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def rn32_scaled_int(n, q):
    """Round the exact value n * 2^q (Python ints) to the nearest fp32, ties to even.

    Returns a numpy float32.  Overflow gives +-inf; an exact zero gives +0.
    This is used where the exact value has too many significant bits for a
    float64 to hold, so a float64 -> float32 conversion would round twice.
    """
    if n == 0:
        return np.float32(0.0)
    neg = n < 0
    n = -n if neg else n
    top = n.bit_length() - 1 + q            # floor(log2 |value|)
    if top > 127:
        return np.float32(-np.inf if neg else np.inf)
    quantum = max(top - 23, -149)           # fp32 ulp at this magnitude (subnormals: 2^-149)
    shift = quantum - q
    if shift <= 0:
        mant = n << (-shift)
    else:
        mant, rem = divmod(n, 1 << shift)
        half = 1 << (shift - 1)
        if rem > half or (rem == half and (mant & 1)):
            mant += 1
    val = math.ldexp(mant, quantum)         # mant <= 2^24: exact in float64
    if val >= 2.0 ** 128:
        val = math.inf
    return np.float32(-val if neg else val)
