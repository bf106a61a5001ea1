"""MI355X-native block-scaled 4-bit (MXFP4) quantizer with block Hadamard
rotation, and the MXFP4 GEMM that consumes it.

The compute path lives in libmxfp4.so (HIP kernels for gfx950 behind the C ABI
of include/mxfp4.h).  This package holds its ctypes binding, torch-facing
wrappers (torch supplies device memory and streams only), the training-step
orchestration of the three GEMMs, and the seeded synthetic inputs.
"""
from .api import QTensor, quantize, gemm, gemm_grouped, empty_qtensor, mxnorm_quantize  # noqa: F401
