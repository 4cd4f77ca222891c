"""The oracle still computes what the committed fixture froze (regression pin)."""
import json
import os

import numpy as np

from tests.golden import make_golden


def test_oracle_matches_frozen_fixture():
    with open(make_golden.OUT) as fh:
        ref = json.load(fh)
    now = make_golden.compute()
    for key, val in ref.items():
        if key == "workload":
            continue
        if isinstance(val, dict):
            for n, x in val.items():
                np.testing.assert_allclose(now[key][n], x, rtol=1e-12, atol=0)
        else:
            np.testing.assert_allclose(now[key], val, rtol=1e-12, atol=1e-300)
