"""Build the gfx950 shared libraries in-tree with hipcc.

    python -m block_scaled_fp4_hadamard_amd.build

Compiles every source under csrc/ for gfx950 only, then links
block_scaled_fp4_hadamard_amd/libmxfp4.so (the quantize/GEMM library) and
block_scaled_fp4_hadamard_amd/libmxprobe.so (matrix-core and vector-instruction
rate probes that the benchmark uses as ceilings; not part of the path).  Packed-FP32
instruction generation is disabled for all device code.
"""
import os
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["quant.hip", "gemm.hip", "mxnorm.hip", "diag.hip", "nvfp4.hip", "osci.hip", "mx_abi.cpp"]
PROBE_SOURCES = ["probe/mfma_rate.hip", "probe/valu_rate.hip"]
PROBE_LIB = os.path.join(PKG, "libmxprobe.so")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0].replace("/", "_") + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build_library(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built %s and %s in %.1f s" % (LIB, os.path.basename(PROBE_LIB), time.time() - t0))
    return LIB


if __name__ == "__main__":
    build_library()
    sys.exit(0)
