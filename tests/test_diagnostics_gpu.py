"""GPU parity of the quantization diagnostics (mx_quant_stats) against the oracle.

"Ripensare il Bias di Shrinkage nel Pretraining di LLM in FP4", Risultati Sperimentali (Diagnostica).
Code counts and block counts exact; the float64 sums (added with atomics) to 1e-9 relative.
"""
import numpy as np
import pytest
import torch

from oracle.diagnostics import quant_stats_ref
from block_scaled_fp4_hadamard_amd import quantize, synth
from block_scaled_fp4_hadamard_amd.api import quant_stats
from gpu_helpers import announce, to_gpu_bits, qt_to_np

pytestmark = pytest.mark.gpu


def tensors():
    rng = np.random.default_rng(61)
    a = synth.activation(96, 512, rng)
    g = synth.gradient(64, 288, rng)
    a2 = a.copy()
    a2[5, 70] = 0x7FC0                                   # a NaN block in each output
    return {"activation": a, "gradient": g, "with-nan": a2}


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("had_n,had_kind", [(0, "det"), (16, "det"), (32, "rand")])
def test_stats_match_the_oracle(axis, grid, had_n, had_kind):
    for name, bits in tensors().items():
        announce("quant stats %s %s %s H%d %s" % (name, axis, grid, had_n, had_kind))
        x = to_gpu_bits(bits)
        q = quantize(x, axis=axis, grid=grid, had_n=had_n, had_kind=had_kind, had_seed=5)[axis]
        got = quant_stats(x, q, axis, grid, had_n, had_kind, 5)
        torch.cuda.synchronize()
        codes, scales = qt_to_np(q)
        s2, e2, hist, blocks = quant_stats_ref(bits, codes, scales, axis, grid, had_n, had_kind, 5)
        assert got["blocks"] == blocks and got["hist"] == hist.tolist()
        assert got["sum_sq"] == pytest.approx(s2, rel=1e-9)
        assert got["sum_err_sq"] == pytest.approx(e2, rel=1e-9)
