"""The oracle still reproduces its committed small-case outputs."""
import json
import os

import numpy as np

from tests.golden.make_oracle_golden import compute

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_small.json")


def test_oracle_matches_committed_golden():
    want = json.load(open(HERE))
    got = compute()
    assert got["case"] == want["case"]
    for a, b in zip(got["samples"], want["samples"]):
        for key in ("y", "y_gla", "y_win"):
            np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-14)
    for key in ("y", "y_gla", "y_win"):
        np.testing.assert_allclose(got["norms"][key], want["norms"][key], rtol=1e-12)
