"""Hand-worked examples (tests/golden/*.txt) run through the oracle.

The pages print no numerical worked example for the scan, so each fixture is
worked by hand from the rule it cites, in dyadic rationals: every value is
exact in binary floating point and the oracle must reproduce it bit for bit.
"""
import glob
import os

import numpy as np
import pytest

import oracle

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.txt")))


def _parse(path):
    d = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, val = line.split(":", 1)
        d[key.strip()] = val.split()
    return d


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_golden(path):
    g = _parse(path)
    variant = g["variant"][0]
    T, dk, dv = int(g["T"][0]), int(g["dk"][0]), int(g["dv"][0])
    arr = lambda n, *shape: np.array([float(x) for x in g[n]]).reshape(shape) if n in g else None
    q, k = arr("q", 1, T, 1, dk), arr("k", 1, T, 1, dk)
    v = arr("v", 1, T, 1, dv)
    alpha = arr("alpha", 1, T, 1, dk) if variant == "kda" else arr("alpha", 1, T, 1)
    out, st = oracle.delta_forward(variant, q, k, v, arr("beta", 1, T, 1), alpha=alpha,
                                   erase_b=arr("erase_b", 1, T, 1, dk),
                                   write_w=arr("write_w", 1, T, 1, dv),
                                   state_in=arr("state_in", 1, 1, dv, dk))
    np.testing.assert_array_equal(out, arr("out", 1, T, 1, dv))
    np.testing.assert_array_equal(st, arr("state_out", 1, 1, dv, dk))


def test_golden_fixtures_present():
    assert len(GOLDEN) >= 3
