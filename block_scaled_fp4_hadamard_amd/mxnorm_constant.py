"""The correction constant c(p, B) of the MXNorm estimate, precomputed on the host.

"MXNorm: Reusing MXFP block scales for efficient tensor normalisation",
Sommario tecnico 2: the estimate rho = c * ((1/K) sum_k m_k^p)^(-1/p) of a
row's inverse RMS uses a constant c(p, B) that the page obtains once, offline,
by Monte Carlo on the CPU: for standard normal values it is E[M^p]^(1/p), M the
largest |value| of a block of B.  This module is that offline step.  It is not
part of the quantization path: mx_mxnorm_quantize takes c as an argument, and
a caller computes it once (or uses a stored value) and passes it in.
"""
from functools import lru_cache

import numpy as np


@lru_cache(maxsize=None)
def correction(power=2, block=32, samples=1 << 21, seed=20260121):
    """c(power, block) from `samples` seeded blocks of standard normal values (relative error about 1e-3 at the
    default size), returned as a float32 value."""
    rng = np.random.default_rng(seed)
    acc, done = 0.0, 0
    while done < samples:
        n = min(1 << 16, samples - done)
        m = np.abs(rng.standard_normal((n, block))).max(axis=1)
        acc += float(np.sum(m ** power))
        done += n
    return float(np.float32((acc / samples) ** (1.0 / power)))
