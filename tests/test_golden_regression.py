"""The oracle still reproduces the fixture that tests/golden/make_golden.py wrote (CPU only)."""
import json
import os

import numpy as np

import oracle
import wkv_inputs

PATH = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")


def test_oracle_matches_frozen_fixture():
    with open(PATH) as f:
        g = json.load(f)
    shape = tuple(g["shape"])
    x = {n: np.array([float.fromhex(s) for s in v]) for n, v in g["inputs_fp32_hex"].items()}
    # the fixture's inputs are still what the generator draws
    ref = wkv_inputs.generate("small")
    assert np.array_equal(x["k"].reshape(shape), ref["k"][:, :12, :2].astype(np.float64))
    w, u = x["w"], x["u"]
    k, v, dy = (x[n].reshape(shape) for n in ("k", "v", "dy"))
    y = oracle.forward_direct(w, u, k, v)
    np.testing.assert_allclose(y.ravel(), g["y"], rtol=1e-13, atol=1e-15)
    for got, key in zip(oracle.backward_direct(w, u, k, v, dy), ("dk", "dv", "dw", "du")):
        np.testing.assert_allclose(np.ravel(got), g[key], rtol=1e-12, atol=1e-14)
