"""The oracle against its committed regression fixture (tests/golden/).

The fixture was written by tests/golden/make_golden.py, which calls only the
oracle; a mismatch means the oracle's arithmetic changed and the change must
name the passage of the pages that justifies it."""
import json
import os

import numpy as np

from tests.golden.make_golden import compute

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_matches_golden_fixture():
    with open(os.path.join(HERE, "oracle_tiny.json")) as f:
        gold = json.load(f)
    now = compute()
    assert now["ids"] == gold["ids"]
    for key in ("lut_rows", "y"):
        a = np.array([float.fromhex(x) for x in now[key]])
        b = np.array([float.fromhex(x) for x in gold[key]])
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-18)
    assert now["nf3_codes_hex"] == gold["nf3_codes_hex"]
    assert now["nf3_scales"] == gold["nf3_scales"]
