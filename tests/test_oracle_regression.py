"""Regression lock of the oracle on a small dyadic case (not gpu).

The stored values were written by tests/golden/make_oracle_fixture.py, which
calls only the oracle; see tests/golden/README.md.
"""
import json
import os

import numpy as np

from tests.golden.make_oracle_fixture import compute, small_case

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_matches_stored_small_case():
    with open(os.path.join(HERE, "oracle_small_case.json")) as f:
        ref = json.load(f)
    got = compute(small_case())
    assert got["perm"] == ref["perm"]
    assert got["idx"] == ref["idx"]
    for key in ("O_full", "R", "O_reuse"):
        np.testing.assert_allclose(np.array(got[key]), np.array(ref[key]), rtol=0, atol=1e-12)
