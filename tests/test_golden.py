"""Regression of the oracle against its stored fixture (tests/golden/tiny_layer.json,
written by tests/golden/make_golden.py from the oracle alone)."""
import json
import os

import numpy as np

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "tiny_layer.json")


def test_oracle_matches_stored_fixture():
    g = json.load(open(GOLD))
    fn = lambda e: [np.array(m) for m in g["experts"][e]]  # noqa: E731
    for name, c in g["cases"].items():
        cap = tuple(c["capacity"]) if c["capacity"] else None
        res = O.moe_layer(np.array(g["x"]), np.array(g["w_router"]), fn, g["E"], g["k"],
                          logit_bias=np.array(g["logit_bias"]), capacity=cap)
        assert res["idx"].tolist() == c["idx"], name
        assert res["drop"].tolist() == c["drop"], name
        assert res["slot_row"].tolist() == c["slot_row"], name
        assert np.allclose(res["gates"], c["gates"], rtol=1e-14, atol=0)
        assert np.allclose(res["out"], c["out"], rtol=1e-13, atol=1e-15)
    assert np.array(g["cases"]["cap_half"]["drop"]).any()
