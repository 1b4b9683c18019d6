"""Regression guard: the oracle reproduces its stored small-case outputs.

The fixture was written by tests/golden/make_golden.py, which calls only the
oracle; the pages hold no numeric worked example to take it from.
"""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "osr_tiny.json")


def test_oracle_matches_stored_outputs():
    with open(GOLDEN) as f:
        data = json.load(f)
    assert len(data["cases"]) == 4
    for c in data["cases"]:
        arr = {k: np.array(c[k]) for k in ("q", "k", "v", "gamma", "mu", "state_in", "y",
                                            "state_out")}
        y, S = oracle.osr_forward(arr["q"], arr["k"], arr["v"], arr["gamma"], arr["mu"],
                                  arr["state_in"], chunk_size=c["chunk_size"], mode=c["mode"])
        np.testing.assert_allclose(y, arr["y"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(S, arr["state_out"], rtol=0, atol=1e-13)
