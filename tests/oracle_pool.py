"""The oracle's quantization of large tensors split over worker processes (test infrastructure).

A worker imports numpy and oracle/ only (never torch or the HIP library): it
memory-maps a bf16 tensor written by the test as .npy, quantizes a range of
output lines with oracle.quantize.quantize_ref, and returns those lines'
codes and scales.  Each line keeps its place in the whole output, so the
stochastic-rounding element indices are those of the whole tensor.
Workers are started with the "spawn" method: a fresh interpreter, nothing
inherited from a parent that may hold a GPU context.
"""
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

LINES_PER_TASK_ELEMS = 1 << 22          # about 4 M elements per task


def _quantize_lines(path, axis, start, stop, kw):
    from oracle.quantize import quantize_ref
    x = np.load(path, mmap_mode="r")
    q = quantize_ref(np.asarray(x), axis, lines=np.arange(start, stop), **kw)[axis]
    return start, q[0], q[1]


def workers():
    """Worker count: the machine's cores up to 12 (some hosts give one process only 16 of their cores)."""
    return max(1, min(12, os.cpu_count() or 1))


class OraclePool:
    def __init__(self, n=None):
        self.ex = ProcessPoolExecutor(max_workers=n or workers(), mp_context=mp.get_context("spawn"))

    def close(self):
        self.ex.shutdown(wait=True)

    def submit_tensor(self, path, shape, axis, **kw):
        """Futures for every line range of one output of the tensor stored at path; collect() joins them."""
        rows, cols = shape
        lines, length = (rows, cols) if axis == "row" else (cols, rows)
        step = max(32, LINES_PER_TASK_ELEMS // length)
        return (lines, length, [self.ex.submit(_quantize_lines, path, axis, s, min(lines, s + step), kw)
                                for s in range(0, lines, step)])

    @staticmethod
    def collect(job, block=32):
        lines, length, futs = job
        codes = np.empty((lines, length // 2), dtype=np.uint8)
        scales = np.empty((lines, length // block), dtype=np.uint8)
        for f in futs:
            s, c, sc = f.result()
            codes[s:s + len(c)] = c
            scales[s:s + len(sc)] = sc
        return codes, scales
