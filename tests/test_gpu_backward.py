"""GPU parity of wkv_backward against the fp64 oracle (marked gpu).

Tolerance: |x - x_oracle| <= 1e-4 * max(|x_oracle|, 0.1) elementwise for dk, dv, dw, du,
and no inf/NaN. Gradients of L = sum dy * y for the operator of "RWKV解读：在Transformer的时代
的新RNN", section 二.3, formula (8) ("RWKV についての調査記録", section "Trainingについて").
"""
import numpy as np
import pytest

import oracle
import wkv_inputs
from helpers import assert_wkv_close

pytestmark = pytest.mark.gpu
NAMES = ("dk", "dv", "dw", "du")


def _gpu_backward(wkv, dev, x, use_fwd_ws=True):
    import torch
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(dev)
         for n in ("w", "u", "k", "v", "dy")}
    B, T, C = x["k"].shape
    fws = None
    if use_fwd_ws:
        fws = wkv.forward_workspace(B, T, C, dev)
        wkv.forward(t["w"], t["u"], t["k"], t["v"], workspace=fws)
    g = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=fws)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in g]


def _check(got, ref, what, rtol=1e-4):
    worst = 0.0
    for gg, rr, n in zip(got, ref, NAMES):
        worst = max(worst, assert_wkv_close(gg, rr, "%s %s" % (what, n), rtol=rtol))
    print("[backward] %s max_violation=%.3g" % (what, worst), flush=True)


def test_small_workload(wkv, dev):
    x = wkv_inputs.generate("small")
    got = _gpu_backward(wkv, dev, x)
    _check(got, oracle.backward_direct(x["w"], x["u"], x["k"], x["v"], x["dy"]), "small")


@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 37, 70), (3, 300, 130), (1, 257, 64),
                                   (2, 513, 65), (1, 1000, 5), (4, 31, 200), (1, 2049, 3)])
def test_ragged_shapes(wkv, dev, B, T, C):
    x = wkv_inputs.generate("l3b", seed=17 + B * T + C, B=B, T=T, C=C)
    got = _gpu_backward(wkv, dev, x)
    ref = oracle.backward_direct(x["w"], x["u"], x["k"], x["v"], x["dy"])
    _check(got, ref, "B=%d T=%d C=%d" % (B, T, C))


def test_without_forward_workspace_and_determinism(wkv, dev):
    x = wkv_inputs.generate("longctx", B=2, T=1100, C=130)
    a = _gpu_backward(wkv, dev, x, use_fwd_ws=True)
    b = _gpu_backward(wkv, dev, x, use_fwd_ws=False)
    c = _gpu_backward(wkv, dev, x, use_fwd_ws=True)
    for p, q, r in zip(a, b, c):
        assert np.array_equal(p, q) and np.array_equal(p, r)


@pytest.mark.parametrize("name", ["l169m", "l3b", "longctx"])
def test_full_workloads(wkv, dev, name):
    x = wkv_inputs.generate(name)
    got = _gpu_backward(wkv, dev, x)
    ref = oracle.backward_recurrent(x["w"], x["u"], x["k"], x["v"], x["dy"])
    _check(got, ref, name)


@pytest.mark.parametrize("kscale,spike", [(8.0, 0.0), (20.0, 80.0), (1.0, 1000.0)])
def test_large_keys_stay_finite(wkv, dev, kscale, spike):
    rng = np.random.default_rng(int(kscale * 10 + spike) + 1)
    B, T, C = 2, 400, 96
    x = wkv_inputs.generate("l3b", seed=19, B=B, T=T, C=C)
    k = (x["k"] * np.float32(kscale)).astype(np.float32)
    if spike:
        m = rng.random((B, T, C)) < 0.02
        k = np.where(m, np.float32(spike) * np.sign(rng.standard_normal((B, T, C))), k)
    x["k"] = k.astype(np.float32)
    got = _gpu_backward(wkv, dev, x)
    for g in got:
        assert np.all(np.isfinite(g))
    ref = oracle.backward_direct(x["w"], x["u"], x["k"], x["v"], x["dy"])
    _check(got, ref, "large-k %g/%g" % (kscale, spike))


@pytest.mark.parametrize("case", ["u_big", "w_fast", "w_slow"])
def test_parameter_extremes(wkv, dev, case):
    B, T, C = 2, 600, 128
    x = wkv_inputs.generate("l3b", seed=23, B=B, T=T, C=C)
    if case == "u_big":
        x["u"] = np.linspace(-50, 50, C).astype(np.float32)
    elif case == "w_fast":
        x["w"] = np.linspace(5, 200, C).astype(np.float32)
    else:
        x["w"] = np.geomspace(1e-7, 1e-3, C).astype(np.float32)
    got = _gpu_backward(wkv, dev, x)
    ref = oracle.backward_direct(x["w"], x["u"], x["k"], x["v"], x["dy"])
    _check(got, ref, case)


def test_large_bonus_with_a_vanishing_first_key(wkv, dev):
    # A sequence opening with a key ~95 below its chunk's largest, on channels with a large
    # bonus u (20..45): the first token's denominator is e^u e^{k_0} alone, its in-frame
    # weight e^{k_0 - ref} lies below the fp32 normal range and e^u sigma_0 above it, while
    # dv_0 ~ dy_0 is ordinary (an fp32 sweep over such a chunk overflows).
    B, T, C = 2, 96, 64
    x = wkv_inputs.generate("l3b", seed=29, B=B, T=T, C=C)
    x["k"][:, 0, :] = np.float32(-95.0)
    x["u"] = np.linspace(20, 45, C).astype(np.float32)
    got = _gpu_backward(wkv, dev, x)
    for g in got:
        assert np.all(np.isfinite(g))
    ref = oracle.backward_direct(x["w"], x["u"], x["k"], x["v"], x["dy"])
    _check(got, ref, "vanishing first key")


def test_large_bonus_on_a_whole_wave_with_a_vanishing_first_key(wkv, dev):
    # As above, with every lane of the wave at u >= 30 (no lane forces the per-token path for
    # the wave): the first key's in-frame weight is an fp32 subnormal while e^u times it is
    # not negligible, so the chunk must go per token for dk, dv (and y) to keep full precision
    B, T, C = 2, 96, 64
    x = wkv_inputs.generate("l3b", seed=31, B=B, T=T, C=C)
    x["k"][:, 0, :] = np.float32(-95.0)
    x["u"] = np.linspace(30, 45, C).astype(np.float32)
    got = _gpu_backward(wkv, dev, x)
    for g in got:
        assert np.all(np.isfinite(g))
    ref = oracle.backward_direct(x["w"], x["u"], x["k"], x["v"], x["dy"])
    _check(got, ref, "vanishing first key, whole wave")


def test_autograd_wrapper(wkv, dev):
    import torch
    x = wkv_inputs.generate("small", B=2, T=300, C=72)
    t = {n: torch.from_numpy(x[n]).to(dev).requires_grad_(n != "dy")
         for n in ("w", "u", "k", "v", "dy")}
    y = wkv.WKV.apply(t["w"], t["u"], t["k"], t["v"])
    (y * t["dy"]).sum().backward()
    ref = oracle.backward_direct(x["w"], x["u"], x["k"], x["v"], x["dy"])
    got = [t[n].grad.cpu().numpy() for n in ("k", "v", "w", "u")]
    _check(got, ref, "autograd")
