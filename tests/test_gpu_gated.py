"""GPU parity of the receptance-gated WKV against the fp64 references (marked gpu).

out = sigma(r) * y ("RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (9): R is
sigmoid-activated; "RWKV についての調査記録", section "コードを見ながらRWKVの構造を把握":
wkv is gated by sigma). wkv_forward_gated writes out; wkv_backward_gated takes dout and
gives dk, dv, dr, dw, du. References: tests/gate_ref.py (pinned by finite differences).
Tolerance as everywhere: |x - r| <= 1e-4 max(|r|, 0.1).
"""
import numpy as np
import pytest

import wkv_inputs
from gate_ref import backward_gated, forward_gated
from helpers import assert_wkv_close

pytestmark = pytest.mark.gpu


def _t(dev, a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _inputs(B, T, C, seed, rscale=1.0):
    x = wkv_inputs.generate("l3b", seed=seed, B=B, T=T, C=C)
    rng = np.random.default_rng(seed + 1)
    x["r"] = (rscale * rng.standard_normal((B, T, C))).astype(np.float32)
    return x


def _run(wkv, dev, x, keep_ws=True):
    import torch
    t = {n: _t(dev, x[n]) for n in ("w", "u", "k", "v", "r", "dy")}
    B, T, C = x["k"].shape
    ws = wkv.forward_workspace(B, T, C, dev)
    out = wkv.forward_gated(t["w"], t["u"], t["k"], t["v"], t["r"], workspace=ws)
    grads = wkv.backward_gated(t["w"], t["u"], t["k"], t["v"], t["r"], t["dy"],
                               fwd_workspace=ws if keep_ws else None)
    torch.cuda.synchronize()
    return out.cpu().numpy(), [g.cpu().numpy() for g in grads]


def _check(x, out, grads, what, direct=True, rtol=1e-4):
    ro = forward_gated(x["w"], x["u"], x["k"], x["v"], x["r"], direct=direct)
    worst = assert_wkv_close(out, ro, what + " out", rtol=1e-4)
    refs = backward_gated(x["w"], x["u"], x["k"], x["v"], x["r"], x["dy"], direct=direct)
    each = {"out": worst}
    for g, r, n in zip(grads, refs, ("dk", "dv", "dr", "dw", "du")):
        assert np.all(np.isfinite(g)), n
        each[n] = assert_wkv_close(g, r, "%s %s" % (what, n), rtol=rtol)
        worst = max(worst, each[n])
    print("[gated] %s max_violation=%.3g (%s)" % (
        what, worst, " ".join("%s %.2g" % kv for kv in each.items())), flush=True)


@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 37, 70), (3, 300, 130), (1, 257, 64),
                                   (2, 513, 65), (4, 31, 200)])
def test_ragged_shapes(wkv, dev, B, T, C):
    x = _inputs(B, T, C, seed=61 + B * T + C)
    out, grads = _run(wkv, dev, x)
    _check(x, out, grads, "B=%d T=%d C=%d" % (B, T, C))


def test_without_forward_workspace(wkv, dev):
    x = _inputs(2, 300, 96, seed=62)
    out, grads = _run(wkv, dev, x, keep_ws=False)
    _check(x, out, grads, "own forward")


def test_gate_extremes(wkv, dev):
    """r saturating the gate (sigma = 0 or 1 in fp32) and r spread wide."""
    x = _inputs(2, 200, 128, seed=63, rscale=3.0)
    x["r"][:, :, :32] = 100.0
    x["r"][:, :, 32:64] = -100.0
    out, grads = _run(wkv, dev, x)
    _check(x, out, grads, "gate extremes")


@pytest.mark.parametrize("case", ["spike", "u_big"])
def test_exact_paths(wkv, dev, case):
    """Chunks that take the per-token paths: keys 1000 apart (forward and backward), and
    |u| > 60 (the backward's per-token path throughout)."""
    x = _inputs(2, 400, 96, seed=64)
    if case == "spike":
        rng = np.random.default_rng(65)
        m = rng.random(x["k"].shape) < 0.02
        x["k"] = np.where(m, np.float32(1000.0) * np.sign(rng.standard_normal(x["k"].shape)),
                          x["k"]).astype(np.float32)
    else:
        x["u"] = np.linspace(-80, 80, 96).astype(np.float32)
    out, grads = _run(wkv, dev, x)
    _check(x, out, grads, case)


def test_full_layer(wkv, dev):
    """The 3B-class layer shape (references from the linear-time oracle)."""
    x = _inputs(8, 4096, 2560, seed=66)
    out, grads = _run(wkv, dev, x)
    _check(x, out, grads, "l3b", direct=False)
