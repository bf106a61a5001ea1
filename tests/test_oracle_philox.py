"""Pin the oracle's Philox4x32-10 to an independent implementation (CPU only).

PyTorch ships a header-only Philox4x32-10 engine (ATen/core/PhiloxRNGEngine.h)
whose key is (seed lo, seed hi) and whose counter is (offset lo, offset hi,
subsequence lo, subsequence hi); successive calls return words 0..3.  The test
compiles a tiny program against that header with g++ and compares outputs;
nothing is stored.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle.philox import philox4x32_10, split64, uniform_halfwords

KAT_SRC = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  for (int a = 1; a + 2 < argc; a += 3) {
    unsigned long long seed = strtoull(argv[a], 0, 0), sub = strtoull(argv[a+1], 0, 0), off = strtoull(argv[a+2], 0, 0);
    at::Philox4_32 eng(seed, sub, off);
    for (int i = 0; i < 4; i++) printf("%u\n", (unsigned)eng());
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def torch_philox():
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    from torch.utils.cpp_extension import include_paths
    inc = [p for p in include_paths() if os.path.exists(os.path.join(p, "ATen/core/PhiloxRNGEngine.h"))]
    if not inc:
        pytest.skip("torch Philox header not found")
    d = tempfile.mkdtemp()
    src, exe = os.path.join(d, "kat.cpp"), os.path.join(d, "kat")
    with open(src, "w") as f:
        f.write(KAT_SRC)
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-I" + inc[0], src, "-o", exe])

    def run(triples):
        args = [exe] + [str(int(v)) for t in triples for v in t]
        out = subprocess.check_output(args).decode().split()
        return np.array([int(v) for v in out], dtype=np.uint64).reshape(-1, 4)
    yield run
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_torch_header(torch_philox):
    rng = np.random.default_rng(0)
    triples = [(0, 0, 0), (1, 0, 0), (2 ** 64 - 1, 2, 2 ** 40 + 3)]
    triples += [(int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 3)), int(rng.integers(0, 2 ** 50)))
                for _ in range(40)]
    ref = torch_philox(triples)
    for (seed, sub, off), want in zip(triples, ref):
        k0, k1 = split64(np.uint64(seed))
        o0, o1 = split64(np.uint64(off))
        s0, s1 = split64(np.uint64(sub))
        got = np.array([int(w) for w in philox4x32_10(o0, o1, s0, s1, k0, k1)], dtype=np.uint64)
        assert np.array_equal(got, want), (seed, sub, off)


def test_uniform_halfwords_index_layout(torch_philox):
    # element i takes the (i % 2) half (low first) of word (i % 8) // 2 of the call with offset i // 8
    seed, stream = 0xDEADBEEF12345, 1
    idx = np.arange(80, dtype=np.uint64)
    got = uniform_halfwords(seed, stream, idx).astype(np.uint64)
    words = torch_philox([(seed, stream, i) for i in range(10)]).reshape(-1)      # 4 words per call
    want = np.array([(int(words[4 * (i // 8) + (i % 8) // 2]) >> (16 * (i % 2))) & 0xFFFF for i in range(80)])
    assert np.array_equal(got, want.astype(np.uint64))
    # indices far from zero use both counter words
    big = np.array([2 ** 35 + 13, 2 ** 40 + 6], dtype=np.uint64)
    got = uniform_halfwords(seed, 0, big)
    for i, g in zip(big, got):
        w = torch_philox([(seed, 0, int(i) // 8)])[0]
        assert g == (int(w[(int(i) % 8) // 2]) >> (16 * (int(i) % 2))) & 0xFFFF


def test_rht_signs_from_torch_philox(torch_philox):
    """The random-sign vector of the randomized rotation: s_j = -1 iff bit j of word 0 of the draw with
    counter (0, 0, 2, 0) (offset 0, subsequence 2) under key had_seed; one draw serves H16 and H32."""
    from oracle.hadamard import rht_signs, sylvester, rotate_lines
    seeds = [0, 1, 20250, 2 ** 64 - 1, 0x123456789ABCDEF]
    ref = torch_philox([(s, 2, 0) for s in seeds])
    for seed, words in zip(seeds, ref):
        w0 = int(words[0])
        for n in (16, 32):
            want = np.array([-1 if (w0 >> j) & 1 else 1 for j in range(n)])
            assert np.array_equal(rht_signs(n, seed), want), (seed, n)
    # the signs multiply the INPUTS before H: rotating the unit vector e_j gives s_j * column j of H / sqrt(n)
    s = rht_signs(32, 20250)
    h = sylvester(32)
    for j in (0, 5, 31):
        e = np.zeros((1, 32), dtype=np.uint16)
        e[0, j] = 0x3F80                                  # bf16 1.0
        y = rotate_lines(e, 32, s)[0].astype(np.float64)
        assert np.array_equal(np.sign(y), s[j] * h[:, j]), j
