"""Helpers shared by the GPU parity tests (the oracle side stays in oracle/)."""
import sys

import numpy as np
import torch


def announce(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def to_gpu_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def qt_to_np(q):
    return q.codes.cpu().numpy(), q.scales.cpu().numpy()


def assert_bytes_equal(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d bytes differ; first at %s: gpu %#x oracle %#x"
                             % (what, len(bad), got.size, i, got[i], want[i]))


def assert_gemm_close(c_gpu, c_ref, g, what, bf16=False):
    """|C - C_ref| <= 1e-5 * G elementwise (bf16 output: plus the bf16 rounding, 2^-8 relative)."""
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    tol = 1e-5 * g
    if bf16:
        tol = tol + 2.0 ** -8 * (np.abs(c_ref) + tol)
    err = np.abs(c_gpu - c_ref)
    bad = np.argwhere(~(err <= tol))
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d outside tolerance; first at %s: gpu %r ref %r G %r"
                             % (what, len(bad), err.size, i, c_gpu[i], c_ref[i], g[i]))
    return float(np.max(err / np.maximum(g, 1e-300)))
