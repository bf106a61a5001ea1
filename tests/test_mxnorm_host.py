"""The offline MXNorm correction constant (CPU only)."""
import pytest

from block_scaled_fp4_hadamard_amd.mxnorm_constant import correction
from oracle.mxnorm import correction_constant


@pytest.mark.parametrize("power", [1, 2])
def test_monte_carlo_correction_matches_the_integral(power):
    # 2^21 seeded blocks: the estimate's relative standard error is a few 1e-4
    assert correction(power) == pytest.approx(correction_constant(power), rel=2e-3)
