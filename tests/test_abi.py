"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before touching a device (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re
import shutil

import pytest

from block_scaled_fp4_hadamard_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4.h")



@pytest.fixture(autouse=True)
def library_built():
    """Where hipcc exists the library must have been built: a missing build fails these tests instead of
    skipping them.  Only a machine without the ROCm compiler skips."""
    if not os.path.exists(_lib.LIB_PATH):
        if shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc"):
            pytest.fail("libmxfp4.so is not built: run python -m block_scaled_fp4_hadamard_amd.build")
        pytest.skip("no ROCm compiler on this machine, so no libmxfp4.so")

FAKE = 0x10000          # an aligned non-null address; validation never dereferences it


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings_and_version():
    assert _lib.status_str(0) == "MX_OK"
    assert "INVALID" in _lib.status_str(1)
    assert "UNSUPPORTED" in _lib.status_str(2)
    assert "DEVICE" in _lib.status_str(3)
    assert _lib.lib().mx_version() >= 100


def q(ld_codes=64, ld_scales=4, codes=FAKE, scales=FAKE):
    return _lib.qtensor(codes, ld_codes, scales, ld_scales)


def quant(x=FAKE, rows=32, cols=128, ld=128, block=32, grid=0, rnd=0, axis=1, rq="d", cq="d"):
    rq = q() if rq == "d" else rq
    cq = q(ld_codes=16, ld_scales=1) if cq == "d" else cq
    return _lib.mx_quantize(x, rows, cols, ld, block, grid, rnd, axis, 0, rq, cq, None)


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-1), 1), (dict(cols=-5), 1), (dict(grid=7), 1), (dict(rnd=9), 1), (dict(axis=0), 1),
    (dict(axis=4), 1), (dict(block=64), 1), (dict(x=0), 1), (dict(x=FAKE + 2), 1),
    (dict(ld=100), 1), (dict(cols=120, ld=128), 1),          # row output needs cols % 32
    (dict(ld=1 << 25), 1),                                      # row pitch below 2^25 elements
    (dict(cols=12, ld=16, axis=2), 1),                          # cols % 8
    (dict(rows=40, axis=2), 1),                                 # column output needs rows % 32
    (dict(rq=None), 1), (dict(rq=q(codes=FAKE + 8)), 1), (dict(rq=q(ld_codes=32)), 1),
    (dict(rq=q(ld_codes=72)), 1), (dict(rq=q(ld_scales=2)), 1), (dict(rq=q(scales=0)), 1),
    (dict(block=16, rq=q(ld_codes=68, ld_scales=8)), 1),       # block 16: ld_codes % 8
    (dict(block=16, rq=q(codes=FAKE + 4, ld_scales=8)), 1),    # block 16: codes 8-byte aligned
    (dict(rows=0), 0), (dict(cols=0), 0),                       # empty: nothing to do
])
def test_quantize_validation(kw, want):
    assert quant(**kw) == want


def test_hadamard_validation():
    L = _lib
    def hq(had_n=32, kind=1, block=32, rq=None):
        rq = q() if rq is None else rq
        return L.mx_hadamard_quantize(FAKE, 32, 128, 128, block, 0, 0, 1, 0, had_n, kind, 0, rq, None, None)
    assert hq(had_n=8) == 1
    assert hq(had_n=64) == 1
    assert hq(kind=0) == 1        # the rotating entry point needs a rotation
    assert hq(kind=5) == 1
    assert hq(had_n=32, block=16) == 1   # the rotation must fit in a block
    assert hq(had_n=16, block=16, rq=q(ld_scales=8)) == 2   # 16-value blocks: no rotation


def gemm(M=64, N=64, K=128, grid=0, block=32, c=FAKE, ldc=64, out=0, a="d", b="d"):
    a = q(ld_codes=64, ld_scales=4) if a == "d" else a
    b = q(ld_codes=64, ld_scales=4) if b == "d" else b
    return _lib.mx_gemm(a, b, M, N, K, grid, block, c, ldc, out, None)


@pytest.mark.parametrize("kw,want", [
    (dict(K=0), 1), (dict(K=100), 1), (dict(M=-1), 1), (dict(grid=3), 1), (dict(out=2), 1),
    (dict(c=0), 1), (dict(c=FAKE + 2), 1), (dict(c=FAKE + 3, out=1), 1), (dict(ldc=60), 1),
    (dict(a=q(ld_codes=32)), 1), (dict(b=q(scales=0)), 1), (dict(block=8), 1),
    (dict(block=16, a=q(ld_scales=8), b=q(ld_scales=8)), 2), (dict(M=0), 0), (dict(N=0), 0),
])
def test_gemm_validation(kw, want):
    assert gemm(**kw) == want


def grouped(problems, K=128, grid=0, block=32, out=0):
    """problems: list of dicts of gemm()'s per-problem keywords (M, N, c, ldc, a, b)."""
    args = []
    for kw in problems:
        d = dict(M=64, N=64, c=FAKE, ldc=64, a=q(ld_codes=64, ld_scales=4), b=q(ld_codes=64, ld_scales=4))
        d.update(kw)
        args.append((d["a"], d["b"], d["M"], d["N"], d["c"], d["ldc"]))
    return _lib.mx_gemm_grouped(args, K, grid, block, out, None)


@pytest.mark.parametrize("problems,kw,want", [
    ([], {}, 1),                                            # count 0
    ([dict(M=0)] * 9, {}, 1),                                # count above MX_GEMM_GROUP_MAX
    ([dict(), dict()], dict(K=100), 1), ([dict()], dict(grid=3), 1), ([dict()], dict(out=2), 1),
    ([dict(), dict(c=0)], {}, 1),                           # one bad problem: nothing runs
    ([dict(c=0), dict()], {}, 1),
    ([dict(), dict(ldc=60)], {}, 1), ([dict(a=q(ld_codes=32)), dict()], {}, 1),
    ([dict(M=-1)], {}, 1),
    ([dict(a=q(ld_scales=8), b=q(ld_scales=8))], dict(block=16), 2),
    ([dict(M=0), dict(N=0)], {}, 0),                        # all empty: nothing to do
])
def test_gemm_grouped_validation(problems, kw, want):
    assert grouped(problems, **kw) == want


def test_gemm_grouped_rejects_a_null_array():
    assert _lib.lib().mx_gemm_grouped(None, 1, 128, 0, 32, 0, None) == 1


def mxnorm(x=FAKE, rows=8, cols=128, ld=128, power=2, c=2.39, grid=0, rnd=0, out="d", rho=FAKE):
    out = q() if out == "d" else out
    return _lib.mx_mxnorm_quantize(x, rows, cols, ld, power, c, grid, rnd, 0, out, rho, None)


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-1), 1), (dict(power=3), 1), (dict(power=0), 1), (dict(c=0.0), 1), (dict(c=-1.0), 1),
    (dict(c=float("nan")), 1), (dict(c=float("inf")), 1), (dict(grid=5), 1), (dict(rnd=2), 1),
    (dict(cols=120, ld=128), 1),                                # cols % 32
    (dict(cols=65568, ld=65568, out=q(ld_codes=32784, ld_scales=2049)), 1),   # cols <= 65536
    (dict(x=0), 1), (dict(x=FAKE + 8), 1), (dict(ld=100), 1), (dict(ld=132), 1),
    (dict(out=q(ld_codes=32)), 1), (dict(out=q(codes=FAKE + 4)), 1), (dict(rho=0), 1), (dict(rho=FAKE + 2), 1),
    (dict(rows=0), 0), (dict(cols=0), 0),                       # empty: nothing to do
])
def test_mxnorm_validation(kw, want):
    assert mxnorm(**kw) == want


def stats_call(x=FAKE, rows=64, cols=128, ld=128, axis=1, grid=0, had_n=0, kind=0, q_="d", st=FAKE):
    qq = q() if q_ == "d" else q_
    return _lib.mx_quant_stats(x, rows, cols, ld, axis, grid, had_n, kind, 0, qq, st, None)


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-1), 1), (dict(axis=3), 1), (dict(axis=0), 1), (dict(grid=4), 1), (dict(kind=7), 1),
    (dict(had_n=8, kind=1), 1), (dict(st=0), 1), (dict(st=FAKE + 4), 1), (dict(x=0), 1), (dict(x=FAKE + 1), 1),
    (dict(ld=100), 1), (dict(cols=120, ld=128), 1), (dict(rows=40, axis=2, q_=q(ld_codes=16, ld_scales=1)), 1),
    (dict(q_=q(ld_codes=32)), 1), (dict(rows=0), 0), (dict(cols=0), 0),
])
def test_quant_stats_validation(kw, want):
    assert stats_call(**kw) == want


def nv(x=FAKE, rows=128, cols=256, ld=256, rnd=0, axis=1, rq="d", cq="d"):
    rq = _lib.nvtensor(FAKE, 128, FAKE, 16, FAKE, 2) if rq == "d" else rq
    cq = _lib.nvtensor(FAKE, 64, FAKE, 8, FAKE, 1) if cq == "d" else cq
    return _lib.mx_nvfp4_quantize(x, rows, cols, ld, rnd, axis, 0, rq, cq, None)


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-1), 1), (dict(rnd=3), 1), (dict(axis=0), 1), (dict(x=0), 1), (dict(x=FAKE + 8), 1),
    (dict(ld=200), 1), (dict(cols=192, ld=192), 1),             # the quantized axis a multiple of 128
    (dict(rows=96, axis=2), 1), (dict(rq=None), 1),
    (dict(rq=_lib.nvtensor(FAKE + 8, 128, FAKE, 16, FAKE, 2)), 1), (dict(rq=_lib.nvtensor(FAKE, 120, FAKE, 16, FAKE, 2)), 1),
    (dict(rq=_lib.nvtensor(FAKE, 128, FAKE, 15, FAKE, 2)), 1), (dict(rq=_lib.nvtensor(FAKE, 128, FAKE, 16, FAKE + 2, 2)), 1),
    (dict(rq=_lib.nvtensor(FAKE, 128, FAKE, 16, FAKE, 1)), 1), (dict(rq=_lib.nvtensor(FAKE, 128, 0, 16, FAKE, 2)), 1),
    (dict(rows=0), 0), (dict(cols=0), 0),
])
def test_nvfp4_validation(kw, want):
    assert nv(**kw) == want


def test_binding_passes_the_operand_block_size():
    """A 16-value operand reaches mx_gemm with block 16 and is refused there (MX_ERR_UNSUPPORTED), instead of
    being read as 32-value blocks; operands whose scale rows do not cover K are refused by the binding.
    Host tensors: the call stops in the library's argument checks."""
    import torch
    from block_scaled_fp4_hadamard_amd import api
    a16 = api.empty_qtensor(256, 512, "cpu", block=16)
    b16 = api.empty_qtensor(256, 512, "cpu", block=16)
    assert a16.scales.shape[1] == 32
    with pytest.raises(_lib.MXError) as e:
        api.gemm(a16, b16)
    assert e.value.status == _lib.MX_ERR_UNSUPPORTED
    a32 = api.empty_qtensor(256, 512, "cpu")
    with pytest.raises(ValueError):
        api.gemm(a32, b16)                       # block sizes disagree
    bad = api.QTensor(a32.codes, a32.scales, "e2m1", 16)     # 16 scale bytes per line cannot cover K = 512
    with pytest.raises(ValueError):
        api.gemm(bad, bad)
    with pytest.raises(ValueError):
        api.quantize(torch.zeros((32, 512), dtype=torch.bfloat16), row_out=a16)    # block 32 into a 16 operand


def rot(x=FAKE, rows=64, cols=128, ld=128, had_n=32, kind=1, axis=1, y=FAKE, ldy=128):
    return _lib.mx_hadamard_rotate(x, rows, cols, ld, had_n, kind, 0, axis, y, ldy, None)


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-1), 1), (dict(had_n=8), 1), (dict(kind=0), 1), (dict(kind=3), 1), (dict(axis=3), 1),
    (dict(axis=0), 1), (dict(cols=120, ld=128), 1), (dict(rows=40, axis=2, ldy=40), 1), (dict(x=0), 1),
    (dict(x=FAKE + 1), 1), (dict(x=FAKE + 8), 1), (dict(ld=100), 1), (dict(ld=132), 1), (dict(y=0), 1),
    (dict(y=FAKE + 8), 1), (dict(ldy=100), 1), (dict(ldy=130), 1), (dict(rows=64, cols=36, ld=40, axis=2), 1),
    (dict(rows=0), 0), (dict(cols=0), 0),
])
def test_rotate_validation(kw, want):
    assert rot(**kw) == want


def qf32(y=FAKE, lines=64, length=128, ldy=128, grid=0, rnd=0, axis=1, out="d"):
    out = q() if out == "d" else out
    if out is None:
        return _lib.lib().mx_quantize_f32(y, lines, length, ldy, grid, rnd, axis, 0, None, None)
    return _lib.mx_quantize_f32(y, lines, length, ldy, grid, rnd, axis, 0, out, None)


@pytest.mark.parametrize("kw,want", [
    (dict(lines=-1), 1), (dict(grid=2), 1), (dict(rnd=3), 1), (dict(axis=3), 1), (dict(length=120, ldy=120), 1),
    (dict(y=0), 1), (dict(y=FAKE + 4), 1), (dict(ldy=100), 1), (dict(ldy=130), 1), (dict(out=q(ld_codes=32)), 1),
    (dict(out=None), 1), (dict(lines=0), 0), (dict(length=0), 0),
])
def test_quantize_f32_validation(kw, want):
    assert qf32(**kw) == want


def osci(w=FAKE, rows=64, cols=128, ldw=128, q_="d", grid=0, st=FAKE, lds=128, mode=1, thr=2.0, resets=None):
    qq = q() if q_ == "d" else q_
    if qq is None:
        return _lib.lib().mx_osci_reset(w, rows, cols, ldw, None, grid, st, st, st, st, lds, mode, thr, resets, None)
    return _lib.mx_osci_reset(w, rows, cols, ldw, qq, grid, st, st, st, st, lds, mode, thr, resets, None)


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-1), 1), (dict(grid=2), 1), (dict(mode=3), 1), (dict(mode=2, thr=-1.0), 1),
    (dict(mode=2, thr=float("nan")), 1), (dict(mode=2, thr=float("inf")), 1), (dict(cols=120, ldw=120, lds=120), 1),
    (dict(w=0), 1), (dict(w=FAKE + 4), 1), (dict(st=0), 1), (dict(st=FAKE + 8), 1), (dict(ldw=100), 1),
    (dict(ldw=130), 1), (dict(lds=126), 1), (dict(q_=None), 1), (dict(q_=q(ld_codes=32)), 1),
    (dict(resets=FAKE + 4), 1), (dict(rows=0), 0), (dict(cols=0), 0),
])
def test_osci_validation(kw, want):
    assert osci(**kw) == want


def test_probe_library_exports_and_rejects_bad_launches():
    """The benchmark's rate probes (libmxprobe.so, not part of the path) load, export their two entry points,
    and refuse launches outside their bounds before any device work."""
    path = os.path.join(os.path.dirname(_lib.LIB_PATH), "libmxprobe.so")
    if not os.path.exists(path):
        pytest.fail("libmxprobe.so is not built: run python -m block_scaled_fp4_hadamard_amd.build")
    P = ctypes.CDLL(path)
    P.mxp_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p, ctypes.c_void_p]
    P.mxp_valu_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert P.mxp_mfma_rate(None, FAKE, 1, 1, 64, FAKE, None) == 1
    assert P.mxp_mfma_rate(FAKE, FAKE, 0, 1, 64, FAKE, None) == 1
    assert P.mxp_mfma_rate(FAKE, FAKE, 1, 1, 96, FAKE, None) == 1          # not a multiple of 64
    assert P.mxp_mfma_rate(FAKE, FAKE, 1, 1, 2048, FAKE, None) == 1
    assert P.mxp_valu_rate(8, 1, FAKE, None) == 1
    assert P.mxp_valu_rate(0, 0, FAKE, None) == 1
    assert P.mxp_valu_rate(0, 1, None, None) == 1
