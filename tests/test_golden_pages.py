"""The oracle against what the pages state about the grids (tests/golden/page_facts.json, each entry cited).

No page works a numeric example of the quantizer or the GEMM, so the fixture holds the fragments the pages do
print: named E2M1 levels, an adjacent pair of bins, the sign of the shrinkage bias and the uniform grid's
equal bins.  The bias is measured on the oracle's RTNE cast over a midpoint lattice of each bin, so a wrong
level, tie rule or saturation point in the oracle shows here.
"""
import json
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle.quantize import rtne_magnitude_codes

FACTS = {f["id"]: f for f in json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))["facts"]}


def consecutive_in(seq, run):
    seq = list(seq)
    return any(seq[i:i + len(run)] == list(run) for i in range(len(seq) - len(run) + 1))


def test_named_e2m1_levels_are_successive_levels():
    assert consecutive_in(F.levels(F.E2M1), FACTS["e2m1_consecutive_levels"]["values"])


def test_named_adjacent_bins_are_adjacent_levels():
    assert consecutive_in(F.levels(F.E2M1), FACTS["e2m1_adjacent_bins"]["values"])


def rtne_bias(grid, i):
    """Mean of Q(v) - v for v uniform on the RTNE bin of interior level i (midpoint lattice, no ties)."""
    lv = F.levels(grid)
    a, b = (lv[i - 1] + lv[i]) / 2, (lv[i] + lv[i + 1]) / 2
    n = 1 << 18
    v = a + (np.arange(n) + 0.5) * (b - a) / n
    return float(np.mean(lv[rtne_magnitude_codes(v, grid)] - v)), (lv[i] - lv[i - 1]) / 2, (lv[i + 1] - lv[i]) / 2


@pytest.mark.parametrize("i", range(1, 7))
def test_shrinkage_sign_on_interior_e2m1_levels(i):
    bias, left, right = rtne_bias(F.E2M1, i)
    if right > left:
        assert bias < 0
    else:
        assert abs(bias) < 1e-12
    assert abs(bias - (left - right) / 2) < 1e-9


@pytest.mark.parametrize("i", range(1, 7))
def test_uniform_grid_has_equal_bins_and_no_bias(i):
    bias, left, right = rtne_bias(F.E1M2, i)
    assert left == right and abs(bias) < 1e-12


def test_some_e2m1_level_shrinks():
    # the page's point: the non-uniform grid has levels whose right bin half is wider
    assert any(rtne_bias(F.E2M1, i)[0] < 0 for i in range(1, 7))
