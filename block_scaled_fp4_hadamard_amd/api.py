"""PyTorch-facing wrappers over the C ABI: they allocate outputs with torch on
the tensor's device and launch on torch's current stream.  No arithmetic of
the method happens here.
"""
from dataclasses import dataclass

import torch

from . import _lib

GEMM_GROUP_MAX = _lib.GEMM_GROUP_MAX    # problems per gemm_grouped call


@dataclass
class QTensor:
    """A block-scaled 4-bit operand: L lines of length K, K-contiguous.

    codes  uint8 (L, K/2): element 2j of a line in the low nibble of byte j
    scales uint8 (L, K/block): E8M0 exponent byte per block of `block` (32, or 16) elements
    """
    codes: torch.Tensor
    scales: torch.Tensor
    grid: str = "e2m1"
    block: int = 32           # values per E8M0 scale: scales hold K / block bytes per line

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
    if dev.type != "cuda":
        return None       # host tensors reach only the library's argument checks, which launch nothing
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
    return QTensor(torch.empty((lines, k // 2), dtype=torch.uint8, device=device), scales, grid, block)


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
    for given in (row_out, col_out):
        if given is not None and given.block != block:
            raise ValueError("an output operand of block %d given for block %d" % (given.block, block))
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
    """C = A B^T on the decoded operands (M x N), fp32 accumulation, fp32 or bf16 output.

    The operands' block size goes to the library as it is (a 16-value operand is refused there: the matrix
    cores take 32-value blocks).
    """
    if a.k != b.k:
        raise ValueError("operands disagree on K: %d vs %d" % (a.k, b.k))
    if a.block != b.block:
        raise ValueError("operands disagree on the block size: %d vs %d" % (a.block, b.block))
    for name, q in (("a", a), ("b", b)):
        if q.scales.shape[1] * q.block != q.k:
            raise ValueError("%s: %d scale bytes per line do not cover K = %d in blocks of %d"
                             % (name, q.scales.shape[1], q.k, q.block))
    grid = grid or a.grid
    M, N, K = a.lines, b.lines, a.k
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.codes.device)
    elif out.dim() != 2 or out.shape[0] != M or out.shape[1] != N or out.stride(1) != 1:
        raise ValueError("out must be a row-major (%d, %d) view" % (M, N))
    kind = {torch.float32: "f32", torch.bfloat16: "bf16"}[out.dtype]
    st = _lib.mx_gemm(a.c_struct(), b.c_struct(), M, N, K, _lib.GRID[grid], a.block, out.data_ptr(), out.stride(0),
                      _lib.OUT[kind], _stream(out.device))
    _lib.check(st, "mx_gemm")
    return out


def gemm_grouped(problems, grid=None):
    """Several GEMMs C_i = A_i B_i^T of one K, grid and output dtype in one library call.

    problems: list of (a, b, out) with out a preallocated (M_i, N_i) fp32 or bf16 tensor.  Each result is
    the one gemm(a, b, out=out) gives, to the bit; the library runs them as one launch when they can share
    it and one launch each otherwise.
    """
    if not problems:
        return []
    if len(problems) > GEMM_GROUP_MAX:
        raise ValueError("at most %d problems per call" % GEMM_GROUP_MAX)
    a0, _, out0 = problems[0]
    grid = grid or a0.grid
    kinds = {torch.float32: "f32", torch.bfloat16: "bf16"}
    args = []
    for i, (a, b, out) in enumerate(problems):
        if a.k != a0.k or b.k != a0.k:
            raise ValueError("problem %d: every operand must have K = %d" % (i, a0.k))
        if a.block != a0.block or b.block != a0.block:
            raise ValueError("problem %d: operands disagree on the block size" % i)
        if out.dtype != out0.dtype:
            raise ValueError("problem %d: every output must be %s" % (i, out0.dtype))
        if out.dim() != 2 or out.shape[0] != a.lines or out.shape[1] != b.lines or out.stride(1) != 1:
            raise ValueError("problem %d: out must be a row-major (%d, %d) view" % (i, a.lines, b.lines))
        for name, q in (("a", a), ("b", b)):
            if q.scales.shape[1] * q.block != q.k:
                raise ValueError("problem %d, %s: %d scale bytes per line do not cover K = %d in blocks of %d"
                                 % (i, name, q.scales.shape[1], q.k, q.block))
        args.append((a.c_struct(), b.c_struct(), a.lines, b.lines, out.data_ptr(), out.stride(0)))
    st = _lib.mx_gemm_grouped(args, a0.k, _lib.GRID[grid], a0.block, _lib.OUT[kinds[out0.dtype]],
                              _stream(out0.device))
    _lib.check(st, "mx_gemm_grouped")
    return [out for _, _, out in problems]


def mxnorm_quantize(x, power, c, grid="e2m1", rounding="rtne", seed=0, out=None, rho=None):
    """MXNorm of every row of a 2-D bf16 CUDA tensor fused with its row-wise MX cast.

    Returns (QTensor of the normalized rows, rho float32 (rows,)).  c is the caller's correction constant
    c(power, 32) (precomputed once on the host, e.g. by mxnorm_constant.correction).
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    xb = _bits_view(x)
    rows, cols = x.shape
    dev = x.device
    c = float(c)
    q = out if out is not None else empty_qtensor(rows, cols, dev, grid)
    r = rho if rho is not None else torch.empty((rows,), dtype=torch.float32, device=dev)
    st = _lib.mx_mxnorm_quantize(xb.data_ptr(), rows, cols, xb.stride(0), power, c, _lib.GRID[grid],
                                 _lib.ROUND[rounding], seed, q.c_struct(), r.data_ptr(), _stream(dev))
    _lib.check(st, "mx_mxnorm_quantize")
    return q, r


def quant_stats(x, q, axis="row", grid=None, had_n=0, had_kind="det", had_seed=0, stats=None, to_host=True):
    """Diagnostic totals of one quantized output q of x, as the kernel accumulates them: sum of y^2, sum of
    (y - y_hat)^2, the counts of the 8 magnitude codes and the number of blocks.  stats: an optional zeroed
    float64 (12,) CUDA tensor to reuse.  Ratios built from these (SQNR, bucket usage) are the caller's.
    to_host=False returns the stats tensor itself, with no copy to the host and no synchronization (the
    kernel adds to it: zero it before a call whose totals are read).
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
    if not to_host:
        return buf
    host = buf.cpu()
    counts = host[2:].view(torch.int64)
    return {"sum_sq": float(host[0]), "sum_err_sq": float(host[1]), "hist": [int(v) for v in counts[:8]],
            "blocks": int(counts[8])}


def hadamard_rotate(x, axis="row", had_n=32, had_kind="det", had_seed=0, out=None):
    """The block Hadamard rotation alone: a float32 CUDA tensor, (rows, cols) for axis "row" (rotated along
    rows), or the transpose (cols, rows) for axis "col" (rotated along columns)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    xb = _bits_view(x)
    rows, cols = x.shape
    shape = (rows, cols) if axis == "row" else (cols, rows)
    y = out if out is not None else torch.empty(shape, dtype=torch.float32, device=x.device)
    if tuple(y.shape) != shape or y.dtype != torch.float32 or y.stride(1) != 1:
        raise ValueError("out must be a float32 %s tensor with unit column stride" % (shape,))
    st = _lib.mx_hadamard_rotate(xb.data_ptr(), rows, cols, xb.stride(0), had_n, _lib.HAD[had_kind], had_seed,
                                 _lib.AXIS[axis], y.data_ptr(), y.stride(0), _stream(x.device))
    _lib.check(st, "mx_hadamard_rotate")
    return y


def quantize_f32(y, axis="row", grid="e2m1", rounding="rtne", seed=0, out=None):
    """The MX cast of the lines of a float32 CUDA tensor y (lines, len); axis names which output of the original
    tensor the lines are ("col": y holds its transpose), which selects the stochastic-rounding stream."""
    if y.dim() != 2 or y.stride(1) != 1 or y.dtype != torch.float32:
        raise ValueError("y must be a 2-D float32 tensor with unit column stride")
    lines, length = y.shape
    q = out if out is not None else empty_qtensor(lines, length, y.device, grid)
    st = _lib.mx_quantize_f32(y.data_ptr(), lines, length, y.stride(0), _lib.GRID[grid], _lib.ROUND[rounding],
                              _lib.AXIS[axis], seed, q.c_struct(), _stream(y.device))
    _lib.check(st, "mx_quantize_f32")
    return q


@dataclass
class OsciState:
    """OsciReset's per-element state, float32 tensors shaped like the master weights."""
    w_prev: torch.Tensor
    q_prev: torch.Tensor
    dist_m: torch.Tensor
    dist_q: torch.Tensor

    @staticmethod
    def empty_like(w):
        return OsciState(*(torch.empty_like(w) for _ in range(4)))


def osci_reset(w, q, state, mode, threshold=0.0, resets=None):
    """One OsciReset step on float32 master weights w (rows, cols) given q, their row-wise quantization (a
    QTensor, block 32); mode "init", "track" or "check".  resets: an optional int64 CUDA tensor of one element
    to which the number of reset elements is added.  w is updated in place."""
    if w.dim() != 2 or w.stride(1) != 1 or w.dtype != torch.float32:
        raise ValueError("w must be a 2-D float32 tensor with unit column stride")
    for t in (state.q_prev, state.dist_m, state.dist_q):
        if t.stride() != state.w_prev.stride() or t.shape != w.shape:
            raise ValueError("the state tensors must share w's shape and one row stride")
    rows, cols = w.shape
    st = _lib.mx_osci_reset(w.data_ptr(), rows, cols, w.stride(0), q.c_struct(), _lib.GRID[q.grid],
                            state.w_prev.data_ptr(), state.q_prev.data_ptr(), state.dist_m.data_ptr(),
                            state.dist_q.data_ptr(), state.w_prev.stride(0), _lib.OSCI[mode], threshold,
                            resets.data_ptr() if resets is not None else None, _stream(w.device))
    _lib.check(st, "mx_osci_reset")
    return w


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
