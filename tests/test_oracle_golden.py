"""The oracle still gives the answers frozen by tests/golden/make_golden.py.

Hashes of integer data must match exactly; float64 samples may differ in the
last bits between BLAS builds, so they are compared to 1e-12 relative.
"""
import json
import math
import os

from tests.golden import make_golden

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _same(got, want):
    assert got.keys() == want.keys()
    for key, w in want.items():
        g = got[key]
        if key == "y64_samples":
            for (i, j, gv), (wi, wj, wv) in zip(g, w):
                assert (i, j) == (wi, wj) and math.isclose(gv, wv, rel_tol=1e-12)
        elif isinstance(w, float):
            assert math.isclose(g, w, rel_tol=1e-12)
        else:
            assert g == w, key


def test_oracle_regression_fixture():
    with open(os.path.join(HERE, "oracle_regression.json")) as f:
        stored = json.load(f)
    _same(make_golden.tiny_w4a16(), stored["tiny_w4a16"])
    _same(make_golden.small_moe_align(), stored["moe_align_t64"])
