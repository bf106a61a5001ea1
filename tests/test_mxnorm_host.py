"""Host-side logic of the MXNorm entry point (CPU only)."""
import pytest

from block_scaled_fp4_hadamard_amd import mxnorm_correction
from oracle.mxnorm import correction_constant


@pytest.mark.parametrize("power", [1, 2])
def test_monte_carlo_correction_matches_the_integral(power):
    # 2^21 seeded blocks: the estimate's relative standard error is a few 1e-4
    assert mxnorm_correction(power) == pytest.approx(correction_constant(power), rel=2e-3)
