"""ctypes binding of libmxfp4.so: argument marshalling only.

Every step of the quantizer and the GEMM runs in the HIP kernels behind the C
ABI declared in include/mxfp4.h; nothing here computes.  Loading fails loudly
when the library has not been built.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp4.so")

MX_OK, MX_ERR_INVALID, MX_ERR_UNSUPPORTED, MX_ERR_DEVICE = 0, 1, 2, 3
GRID = {"e2m1": 0, "e1m2": 1}
ROUND = {"rtne": 0, "sr": 1}
AXIS = {"row": 1, "col": 2, "both": 3}
HAD = {"none": 0, "det": 1, "rand": 2}
OUT = {"f32": 0, "bf16": 1}
OSCI = {"init": 0, "track": 1, "check": 2}

EXPORTS = ("mx_quantize", "mx_hadamard_quantize", "mx_gemm", "mx_gemm_grouped", "mx_mxnorm_quantize", "mx_quant_stats",
           "mx_nvfp4_quantize", "mx_hadamard_rotate", "mx_quantize_f32", "mx_osci_reset", "mx_status_str",
           "mx_version")


class MXError(RuntimeError):
    def __init__(self, status, fn):
        self.status = status
        super().__init__("%s returned %s" % (fn, status_str(status)))


class NVTensorC(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("ld_codes", ctypes.c_int64),
                ("inner", ctypes.c_void_p), ("ld_inner", ctypes.c_int64),
                ("outer", ctypes.c_void_p), ("ld_outer", ctypes.c_int64)]


class QTensorC(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("ld_codes", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("ld_scales", ctypes.c_int64)]


GEMM_GROUP_MAX = 8      # MX_GEMM_GROUP_MAX


class GemmProblemC(ctypes.Structure):
    _fields_ = [("a", ctypes.POINTER(QTensorC)), ("b", ctypes.POINTER(QTensorC)),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("c", ctypes.c_void_p), ("ldc", ctypes.c_int64)]


_lib = None


def lib():
    """The loaded library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmxfp4.so is not built; run python -m block_scaled_fp4_hadamard_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, u64, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p
        qp = ctypes.POINTER(QTensorC)
        L.mx_quantize.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, u64, qp, qp, vp]
        L.mx_quantize.restype = ctypes.c_int
        L.mx_hadamard_quantize.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, u64, i32, i32, u64, qp, qp, vp]
        L.mx_hadamard_quantize.restype = ctypes.c_int
        L.mx_gemm.argtypes = [qp, qp, i64, i64, i64, i32, i32, vp, i64, i32, vp]
        L.mx_gemm.restype = ctypes.c_int
        L.mx_gemm_grouped.argtypes = [ctypes.POINTER(GemmProblemC), i32, i64, i32, i32, i32, vp]
        L.mx_gemm_grouped.restype = ctypes.c_int
        L.mx_mxnorm_quantize.argtypes = [vp, i64, i64, i64, i32, ctypes.c_float, i32, i32, u64, qp, vp, vp]
        L.mx_mxnorm_quantize.restype = ctypes.c_int
        L.mx_quant_stats.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, u64, qp, vp, vp]
        L.mx_quant_stats.restype = ctypes.c_int
        np_ = ctypes.POINTER(NVTensorC)
        L.mx_nvfp4_quantize.argtypes = [vp, i64, i64, i64, i32, i32, u64, np_, np_, vp]
        L.mx_nvfp4_quantize.restype = ctypes.c_int
        L.mx_hadamard_rotate.argtypes = [vp, i64, i64, i64, i32, i32, u64, i32, vp, i64, vp]
        L.mx_hadamard_rotate.restype = ctypes.c_int
        L.mx_quantize_f32.argtypes = [vp, i64, i64, i64, i32, i32, i32, u64, qp, vp]
        L.mx_quantize_f32.restype = ctypes.c_int
        L.mx_osci_reset.argtypes = [vp, i64, i64, i64, qp, i32, vp, vp, vp, vp, i64, i32, ctypes.c_float, vp, vp]
        L.mx_osci_reset.restype = ctypes.c_int
        L.mx_status_str.argtypes = [ctypes.c_int]
        L.mx_status_str.restype = ctypes.c_char_p
        L.mx_version.argtypes = []
        L.mx_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def status_str(status):
    return lib().mx_status_str(status).decode()


def check(status, fn):
    if status != MX_OK:
        raise MXError(status, fn)


def qtensor(codes_ptr, ld_codes, scales_ptr, ld_scales):
    return QTensorC(codes_ptr, ld_codes, scales_ptr, ld_scales)


def mx_quantize(x_ptr, rows, cols, ld_x, block, grid, rnd, axis, seed, row_q, col_q, stream):
    return lib().mx_quantize(x_ptr, rows, cols, ld_x, block, grid, rnd, axis, seed,
                             ctypes.byref(row_q) if row_q is not None else None,
                             ctypes.byref(col_q) if col_q is not None else None, stream)


def mx_hadamard_quantize(x_ptr, rows, cols, ld_x, block, grid, rnd, axis, seed, had_n, had_kind, had_seed,
                         row_q, col_q, stream):
    return lib().mx_hadamard_quantize(x_ptr, rows, cols, ld_x, block, grid, rnd, axis, seed, had_n, had_kind,
                                      had_seed, ctypes.byref(row_q) if row_q is not None else None,
                                      ctypes.byref(col_q) if col_q is not None else None, stream)


def mx_gemm(a_q, b_q, M, N, K, grid, block, c_ptr, ldc, out, stream):
    return lib().mx_gemm(ctypes.byref(a_q), ctypes.byref(b_q), M, N, K, grid, block, c_ptr, ldc, out, stream)


def mx_gemm_grouped(problems, K, grid, block, out, stream):
    """problems: list of (a QTensorC, b QTensorC, M, N, c_ptr, ldc)."""
    qs = [(a, b) for a, b, *_ in problems]     # kept alive through the call
    arr = (GemmProblemC * max(1, len(problems)))()
    for i, ((a, b), (_, _, M, N, c_ptr, ldc)) in enumerate(zip(qs, problems)):
        arr[i] = GemmProblemC(ctypes.pointer(a), ctypes.pointer(b), M, N, c_ptr, ldc)
    return lib().mx_gemm_grouped(arr, len(problems), K, grid, block, out, stream)


def mx_mxnorm_quantize(x_ptr, rows, cols, ld_x, power, c, grid, rnd, seed, out_q, rho_ptr, stream):
    return lib().mx_mxnorm_quantize(x_ptr, rows, cols, ld_x, power, c, grid, rnd, seed, ctypes.byref(out_q),
                                    rho_ptr, stream)


def mx_quant_stats(x_ptr, rows, cols, ld_x, axis, grid, had_n, had_kind, had_seed, q, stats_ptr, stream):
    return lib().mx_quant_stats(x_ptr, rows, cols, ld_x, axis, grid, had_n, had_kind, had_seed, ctypes.byref(q),
                                stats_ptr, stream)


def nvtensor(codes_ptr, ld_codes, inner_ptr, ld_inner, outer_ptr, ld_outer):
    return NVTensorC(codes_ptr, ld_codes, inner_ptr, ld_inner, outer_ptr, ld_outer)


def mx_nvfp4_quantize(x_ptr, rows, cols, ld_x, rnd, axis, seed, row_q, col_q, stream):
    return lib().mx_nvfp4_quantize(x_ptr, rows, cols, ld_x, rnd, axis, seed,
                                   ctypes.byref(row_q) if row_q is not None else None,
                                   ctypes.byref(col_q) if col_q is not None else None, stream)


def mx_hadamard_rotate(x_ptr, rows, cols, ld_x, had_n, had_kind, had_seed, axis, y_ptr, ld_y, stream):
    return lib().mx_hadamard_rotate(x_ptr, rows, cols, ld_x, had_n, had_kind, had_seed, axis, y_ptr, ld_y, stream)


def mx_quantize_f32(y_ptr, lines, length, ld_y, grid, rnd, axis, seed, out_q, stream):
    return lib().mx_quantize_f32(y_ptr, lines, length, ld_y, grid, rnd, axis, seed, ctypes.byref(out_q), stream)


def mx_osci_reset(w_ptr, rows, cols, ld_w, q, grid, w_prev, q_prev, dist_m, dist_q, ld_state, mode, threshold,
                  resets_ptr, stream):
    return lib().mx_osci_reset(w_ptr, rows, cols, ld_w, ctypes.byref(q), grid, w_prev, q_prev, dist_m, dist_q,
                               ld_state, mode, threshold, resets_ptr, stream)
