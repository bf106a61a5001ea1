"""PyTorch-facing wrappers over the C ABI: they allocate outputs with torch on
the tensor's device and launch on torch's current stream.  No arithmetic of
the method happens here.
"""
from dataclasses import dataclass
from functools import lru_cache

import numpy as np
import torch

from . import _lib


@dataclass
class QTensor:
    """A block-scaled 4-bit operand: L lines of length K, K-contiguous.

    codes  uint8 (L, K/2): element 2j of a line in the low nibble of byte j
    scales uint8 (L, K/32): E8M0 exponent byte per 32-element block
    """
    codes: torch.Tensor
    scales: torch.Tensor
    grid: str = "e2m1"

    @property
    def lines(self):
        return self.codes.shape[0]

    @property
    def k(self):
        return self.codes.shape[1] * 2

    def c_struct(self):
        return _lib.qtensor(self.codes.data_ptr(), self.codes.stride(0),
                            self.scales.data_ptr(), self.scales.stride(0))


def _stream(dev):
    return ctypes_void(torch.cuda.current_stream(dev).cuda_stream)


def ctypes_void(handle):
    return handle if handle else None


def _bits_view(x):
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16)
    if x.dtype in (torch.int16, torch.uint16):
        return x
    raise TypeError("x must be bfloat16 (or its 16-bit patterns), got %s" % x.dtype)


def empty_qtensor(lines, k, device, grid="e2m1", block=32):
    """An output operand; scale rows are padded to a multiple of 4 bytes, which the GEMM's copy path needs
    (the padding is never read as data)."""
    nb = k // block
    scales = torch.empty((lines, (nb + 3) // 4 * 4), dtype=torch.uint8, device=device)[:, :nb]
    return QTensor(torch.empty((lines, k // 2), dtype=torch.uint8, device=device), scales, grid)


def quantize(x, axis="row", grid="e2m1", rounding="rtne", seed=0, had_n=0, had_kind="det", had_seed=0,
             block=32, row_out=None, col_out=None):
    """Quantize a 2-D bf16 CUDA tensor; returns {"row": QTensor, "col": QTensor} as requested.

    had_n 0 means no rotation; otherwise 16 or 32 with had_kind "det" or "rand".
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    xb = _bits_view(x)
    rows, cols = x.shape
    dev = x.device
    do_row, do_col = axis in ("row", "both"), axis in ("col", "both")
    out = {}
    rq = cq = None
    if do_row:
        out["row"] = row_out if row_out is not None else empty_qtensor(rows, cols, dev, grid, block)
        rq = out["row"].c_struct()
    if do_col:
        out["col"] = col_out if col_out is not None else empty_qtensor(cols, rows, dev, grid, block)
        cq = out["col"].c_struct()
    stream = _stream(dev)
    if had_n:
        st = _lib.mx_hadamard_quantize(xb.data_ptr(), rows, cols, xb.stride(0), block, _lib.GRID[grid],
                                       _lib.ROUND[rounding], _lib.AXIS[axis], seed, had_n, _lib.HAD[had_kind],
                                       had_seed, rq, cq, stream)
        _lib.check(st, "mx_hadamard_quantize")
    else:
        st = _lib.mx_quantize(xb.data_ptr(), rows, cols, xb.stride(0), block, _lib.GRID[grid],
                              _lib.ROUND[rounding], _lib.AXIS[axis], seed, rq, cq, stream)
        _lib.check(st, "mx_quantize")
    return out


def gemm(a, b, out_dtype=torch.float32, out=None, grid=None):
    """C = A B^T on the decoded operands (M x N), fp32 accumulation, fp32 or bf16 output."""
    if a.k != b.k:
        raise ValueError("operands disagree on K: %d vs %d" % (a.k, b.k))
    grid = grid or a.grid
    M, N, K = a.lines, b.lines, a.k
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.codes.device)
    kind = {torch.float32: "f32", torch.bfloat16: "bf16"}[out.dtype]
    st = _lib.mx_gemm(a.c_struct(), b.c_struct(), M, N, K, _lib.GRID[grid], 32, out.data_ptr(), out.stride(0),
                      _lib.OUT[kind], _stream(out.device))
    _lib.check(st, "mx_gemm")
    return out


@lru_cache(maxsize=None)
def mxnorm_correction(power=2, block=32, samples=1 << 21, seed=20260121):
    """The correction constant c(p, B) of the MXNorm estimate, by Monte Carlo.

    "MXNorm: Reusing MXFP block scales ...", Sommario tecnico 2: the constant that
    makes c * (mean of m^p)^(-1/p) the inverse RMS of rows of i.i.d. values; for
    standard normal values it is E[M^p]^(1/p) with M the largest |value| of a
    block.  Estimated from `samples` seeded blocks on the host (relative error
    about 1e-3 at the default size), returned as a float32 value.
    """
    rng = np.random.default_rng(seed)
    acc, done = 0.0, 0
    while done < samples:
        n = min(1 << 16, samples - done)
        m = np.abs(rng.standard_normal((n, block))).max(axis=1)
        acc += float(np.sum(m ** power))
        done += n
    return float(np.float32((acc / samples) ** (1.0 / power)))


def mxnorm_quantize(x, power=2, c=None, grid="e2m1", rounding="rtne", seed=0, out=None, rho=None):
    """MXNorm of every row of a 2-D bf16 CUDA tensor fused with its row-wise MX cast.

    Returns (QTensor of the normalized rows, rho float32 (rows,)).  c defaults to
    mxnorm_correction(power).
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    xb = _bits_view(x)
    rows, cols = x.shape
    dev = x.device
    c = mxnorm_correction(power) if c is None else float(c)
    q = out if out is not None else empty_qtensor(rows, cols, dev, grid)
    r = rho if rho is not None else torch.empty((rows,), dtype=torch.float32, device=dev)
    st = _lib.mx_mxnorm_quantize(xb.data_ptr(), rows, cols, xb.stride(0), power, c, _lib.GRID[grid],
                                 _lib.ROUND[rounding], seed, q.c_struct(), r.data_ptr(), _stream(dev))
    _lib.check(st, "mx_mxnorm_quantize")
    return q, r


def quant_stats(x, q, axis="row", grid=None, had_n=0, had_kind="det", had_seed=0, stats=None):
    """Diagnostics of one quantized output q of x: SQNR (dB), noise and signal energy, magnitude-code counts,
    effective bucket ratio (exp(entropy) / 8).  stats: an optional zeroed float64 (12,) CUDA tensor to reuse.
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    xb = _bits_view(x)
    rows, cols = x.shape
    grid = grid or q.grid
    buf = stats if stats is not None else torch.zeros(12, dtype=torch.float64, device=x.device)
    st = _lib.mx_quant_stats(xb.data_ptr(), rows, cols, xb.stride(0), _lib.AXIS[axis], _lib.GRID[grid],
                             had_n, _lib.HAD["none" if not had_n else had_kind], had_seed, q.c_struct(),
                             buf.data_ptr(), _stream(x.device))
    _lib.check(st, "mx_quant_stats")
    host = buf.cpu()
    sums = host[:2].numpy()
    counts = host[2:].view(torch.int64).numpy()
    hist, blocks = counts[:8].copy(), int(counts[8])
    p = hist[hist > 0] / max(hist.sum(), 1)
    ratio = float(np.exp(-np.sum(p * np.log(p))) / 8.0) if p.size else 0.0
    sqnr = float("inf") if sums[1] == 0 else float(10.0 * np.log10(sums[0] / sums[1]))
    return {"sqnr_db": sqnr, "sum_sq": float(sums[0]), "sum_err_sq": float(sums[1]), "hist": hist.tolist(),
            "blocks": blocks, "bucket_ratio": ratio}


@dataclass
class NVTensor:
    """An NVFP4-style double-block operand: L lines of length K.

    codes uint8 (L, K/2) E2M1 as QTensor; inner uint8 (L, K/16) E4M3 scales; outer float32 (L, K/128)
    """
    codes: torch.Tensor
    inner: torch.Tensor
    outer: torch.Tensor

    def c_struct(self):
        return _lib.nvtensor(self.codes.data_ptr(), self.codes.stride(0), self.inner.data_ptr(),
                             self.inner.stride(0), self.outer.data_ptr(), self.outer.stride(0))


def nvfp4_quantize(x, axis="row", rounding="rtne", seed=0, row_out=None, col_out=None):
    """NVFP4-style double-block quantization of a 2-D bf16 CUDA tensor; {"row": NVTensor, "col": NVTensor}.

    row_out / col_out reuse NVTensors from an earlier call of the same shape.
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    xb = _bits_view(x)
    rows, cols = x.shape
    dev = x.device

    def empty(lines, k):
        return NVTensor(torch.empty((lines, k // 2), dtype=torch.uint8, device=dev),
                        torch.empty((lines, k // 16), dtype=torch.uint8, device=dev),
                        torch.empty((lines, k // 128), dtype=torch.float32, device=dev))
    out = {}
    if axis in ("row", "both"):
        out["row"] = row_out if row_out is not None else empty(rows, cols)
    if axis in ("col", "both"):
        out["col"] = col_out if col_out is not None else empty(cols, rows)
    rq = out["row"].c_struct() if "row" in out else None
    cq = out["col"].c_struct() if "col" in out else None
    st = _lib.mx_nvfp4_quantize(xb.data_ptr(), rows, cols, xb.stride(0), _lib.ROUND[rounding], _lib.AXIS[axis],
                                seed, rq, cq, _stream(dev))
    _lib.check(st, "mx_nvfp4_quantize")
    return out
