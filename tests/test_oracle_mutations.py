"""Planted mistakes: broken copies of the oracle source must fail the pins (CPU only).

Each case copies oracle/wkv_oracle.c, applies one textual change that models a plausible
slip (decay offset, dropped bonus, wrong sign, missing term, wrong update order), builds
it with gcc into a temporary directory, routes the oracle module through it and checks
that at least one pin rejects it. The real oracle source is never modified.
"""
import json
import math
import os
import subprocess

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "wkv_oracle.c")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MUTATIONS = [
    ("decay offset t-i", "(double)(t - 1 - i) * w[c]", "(double)(t - i) * w[c]", "direct"),
    ("bonus dropped", ": u[c] + k[IDX(b, t, c)];", ": k[IDX(b, t, c)];", "direct"),
    ("decay sign", "- (double)(t - 1 - i) * w[c]", "+ (double)(t - 1 - i) * w[c]", "direct"),
    ("recurrent: no decay", "double decay = exp(-w[c]);", "double decay = 1.0;", "recurrent"),
    ("recurrent: bonus on state", "double cur = exp(u[c] + kk);\n            y[IDX",
     "double cur = exp(kk);\n            y[IDX", "recurrent"),
    ("rescaled: no decay", "double pw = p - w[c];", "double pw = p;", "rescaled"),
    ("backward: dk misses -y", "dk[IDX(b, i, c)] += g * P * (vi - yt);",
     "dk[IDX(b, i, c)] += g * P * vi;", "bdirect"),
    ("backward: dw age off by one", "sw -= (double)(t - 1 - i) * g * P * (vi - yt);",
     "sw -= (double)(t - i) * g * P * (vi - yt);", "bdirect"),
    ("backward rec: dw sign", "sw -= s * (Ap - yt * Bp);", "sw += s * (Ap - yt * Bp);", "brec"),
    ("backward rec: age carry order", "Ap = decay * (Ap + A);", "Ap = decay * Ap + A;", "brec"),
    ("backward rec: G undecayed", "G = decay * G + ss[i];", "G = G + ss[i];", "brec"),
    ("backward rec: H uses s", "H = decay * H + ss[i] * ys[i];", "H = decay * H + ss[i];", "brec"),
]


def _val(s):
    named = {"ln2": math.log(2.0), "ln4": math.log(4.0)}
    return named[s] if s in named else float(s)


def _forward(kind):
    if kind == "direct":
        return oracle.forward_direct
    if kind == "recurrent":
        return oracle.forward_recurrent
    return lambda w, u, k, v: oracle.forward_rescaled(w, u, k, v)[0]


def _forward_pins_pass(fwd) -> bool:
    with open(os.path.join(GOLDEN, "hand_forward.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        T = len(case["v"])
        y = fwd(np.array([_val(case["w"])]), np.array([_val(case["u"])]),
                np.array([_val(s) for s in case["k"]]).reshape(1, T, 1),
                np.array(case["v"], float).reshape(1, T, 1))[0, :, 0]
        if not np.allclose(y, case["y"], rtol=1e-12, atol=1e-13):
            return False
    rng = np.random.default_rng(5)
    w = np.exp(rng.uniform(-3, 1, 4))
    u = rng.uniform(-1, 1, 4)
    k = rng.standard_normal((2, 9, 4))
    v = rng.standard_normal((2, 9, 4))
    y = fwd(w, u, k, v)
    a, b = np.exp(k[:, 0]), np.exp(u + k[:, 1])
    if not np.allclose(y[:, 1], (a * v[:, 0] + b * v[:, 1]) / (a + b), rtol=1e-12):
        return False
    yz = fwd(np.zeros(4), np.zeros(4), np.zeros_like(k), v)
    return bool(np.allclose(yz, np.cumsum(v, 1) / np.arange(1, 10)[None, :, None], rtol=1e-12))


def _backward_pins_pass(bwd) -> bool:
    with open(os.path.join(GOLDEN, "hand_backward.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        T = len(case["v"])
        out = bwd(np.array([_val(case["w"])]), np.array([_val(case["u"])]),
                  np.array([_val(s) for s in case["k"]]).reshape(1, T, 1),
                  np.array(case["v"], float).reshape(1, T, 1),
                  np.array(case["dy"], float).reshape(1, T, 1))
        for got, key in zip(out, ("dk", "dv", "dw", "du")):
            if not np.allclose(np.ravel(got), np.ravel(case[key]), rtol=1e-12, atol=1e-13):
                return False
    rng = np.random.default_rng(6)
    B, T, C = 2, 30, 3
    w = np.exp(rng.uniform(-3, 1, C))
    u = rng.uniform(-1, 1, C)
    k = rng.standard_normal((B, T, C))
    v = rng.standard_normal((B, T, C))
    g = rng.standard_normal((B, T, C))
    dk, dv, dw, du = bwd(w, u, k, v, g)
    if not np.allclose(dk.sum(1), 0.0, atol=1e-11):
        return False
    if not np.allclose(dv.sum(1), g.sum(1), rtol=1e-11, atol=1e-12):
        return False
    tdk = (np.arange(T)[None, :, None] * dk).sum(axis=(0, 1))
    return bool(np.allclose(tdk, dw + du, rtol=1e-10, atol=1e-10))


@pytest.mark.parametrize("label,old,new,kind", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, label, old, new, kind):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + label
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(oracle.compile_command(str(path), str(so)), check=True)
    oracle.use_library(str(so))
    try:
        if kind in ("direct", "recurrent", "rescaled"):
            try:
                ok = _forward_pins_pass(_forward(kind))
            except OverflowError:
                ok = False
        else:
            bwd = oracle.backward_direct if kind == "bdirect" else oracle.backward_recurrent
            ok = _backward_pins_pass(bwd)
    finally:
        oracle.use_library(None)
    assert not ok, "planted mistake not caught: " + label


def test_unmutated_source_passes_the_same_pins():
    for kind in ("direct", "recurrent", "rescaled"):
        assert _forward_pins_pass(_forward(kind))
    assert _backward_pins_pass(oracle.backward_direct)
    assert _backward_pins_pass(oracle.backward_recurrent)
