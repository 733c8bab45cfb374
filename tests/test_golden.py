"""The oracle still reproduces its frozen output on the tiny_f32 workload (CPU only)."""
import json
import os

import numpy as np

import golden.make_golden as G

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_frozen_fixture():
    with open(os.path.join(HERE, "golden", "tiny_f32_oracle.json")) as f:
        ref = json.load(f)
    got = G.compute()
    assert got["rows"] == ref["rows"] and got["seed"] == ref["seed"]
    for key in ("y_rows", "lambda_rows", "lambda_T", "M_T_diag"):
        np.testing.assert_allclose(np.array(got[key]), np.array(ref[key]), rtol=1e-13, atol=1e-15)
