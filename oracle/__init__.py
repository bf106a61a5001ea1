"""CPU oracle for block-scaled 4-bit quantization with block Hadamard rotation,
and for the GEMM on the quantized operands.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It shares no code, table or constant with the HIP
library; both sides only share the seeded input generators, which hold none of
the method's arithmetic.

It is plain, slow and written to be checked by eye against the pages:
  formats   - E2M1 / E1M2 grids, the E8M0 block scale, exact fp32 rounding
  philox    - Philox4x32-10 from its published definition
  hadamard  - Sylvester H16/H32, random signs, the exact-sum rotation
  quantize  - rotate, block absmax, scale, RTNE/SR cast, pack
  gemm      - decode and the float64 GEMM with its tolerance scale
  recipe    - which operand is quantized along which axis for the three GEMMs
  osci_reset - oscillation tracking and reset of master weights (TetraJet-v2's OsciReset)
Every part is pinned by the CPU tests against closed forms, brute force or an
independent construction (scipy's Hadamard, torch's Philox header).
"""
from .formats import E2M1, E1M2
from .quantize import quantize_ref, quantize_lines, RTNE, SR
from .gemm import gemm_ref, decode

__all__ = ["E2M1", "E1M2", "RTNE", "SR", "quantize_ref", "quantize_lines", "gemm_ref", "decode"]
