"""The GEMM's choice between the whole-tile kernel and the bounds-checked kernel (CPU only).

The whole-tile kernel addresses each 256-row tile's operand bytes with 32-bit offsets from the tile's first
row, so a shape whose tile spans 4 GiB or more (a huge K, or a strided view with a huge pitch) must take the
bounds-checked kernel, whose addresses are 64-bit.  The predicate is plain host C++
(csrc/gemm_path.h); this test compiles it with g++ and checks its edges.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_fp4_hadamard_amd", "csrc")

SRC = r"""
#include "gemm_path.h"
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  // args: M N K lda_codes ldb_codes lda_scales ldb_scales ldc c_align out_f32, repeated
  for (int a = 1; a + 9 < argc; a += 10) {
    long long v[10];
    for (int i = 0; i < 10; ++i) v[i] = strtoll(argv[a + i], 0, 0);
    printf("%d\n", (int)mx::gemm_full_path(v[0], v[1], v[2], 4096, 4096, v[3], v[4], v[5], v[6],
                                           (uintptr_t)v[8], v[7], v[9] != 0));
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def full_path():
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tempfile.mkdtemp()
    src, exe = os.path.join(d, "p.cpp"), os.path.join(d, "p")
    with open(src, "w") as f:
        f.write(SRC)
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-I" + CSRC, src, "-o", exe])

    def run(cases):
        args = [exe] + [str(int(x)) for c in cases for x in c]
        return [bool(int(t)) for t in subprocess.check_output(args).decode().split()]
    yield run
    shutil.rmtree(d, ignore_errors=True)


def case(M=8192, N=4096, K=4096, lda=None, ldb=None, lsa=None, lsb=None, ldc=None, c_align=4096, f32=1):
    lda = K // 2 if lda is None else lda
    ldb = K // 2 if ldb is None else ldb
    lsa = (K // 32 + 3) // 4 * 4 if lsa is None else lsa
    lsb = (K // 32 + 3) // 4 * 4 if lsb is None else lsb
    ldc = N if ldc is None else ldc
    return (M, N, K, lda, ldb, lsa, lsb, ldc, c_align, f32)


def test_llama_shapes_take_the_whole_tile_kernel(full_path):
    shapes = [(8192, 6144, 4096), (8192, 4096, 14336), (14336, 14336, 8192), (6144, 4096, 8192),
              (8192, 28672, 4096), (4096, 14336, 8192)]
    assert all(full_path([case(M, N, K) for M, N, K in shapes]))


def test_small_or_misaligned_shapes_take_the_checked_kernel(full_path):
    got = full_path([case(M=255), case(N=255), case(K=480), case(N=4100 - 2), case(lsa=130),
                     case(ldc=4098), case(c_align=4100), case(c_align=4104, f32=0), case(c_align=4104, f32=1)])
    assert got == [False, False, False, False, False, False, False, True, False]


def test_tile_span_of_4_gib_takes_the_checked_kernel(full_path):
    lim = 1 << 32
    ok_ld = (lim - 1 - 4096 // 2) // 255 // 16 * 16        # the largest 16-byte multiple pitch that still fits
    got = full_path([
        case(lda=ok_ld), case(lda=ok_ld + 16), case(ldb=ok_ld + 16),
        case(K=1 << 25, lda=1 << 24, ldb=1 << 24),            # K = 2^25: 255 * 2^24 + 2^24 = 2^32
        case(K=(1 << 25) - 512, lda=(1 << 24) - 256, ldb=(1 << 24) - 256),
        case(lsa=(lim // 255) // 4 * 4 + 4), case(lsb=(lim // 255) // 4 * 4 + 4),
    ])
    assert got == [True, False, False, False, True, False, False]
