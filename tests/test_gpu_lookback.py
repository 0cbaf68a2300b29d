"""The look-back's recomputation path (marked gpu).

A unit that finds a window unpublished after the poll limit recomputes that window's
aggregate from k, v (and dy) itself and publishes it; the backward's unit then reloads and
recomputes its own chunk. With the limit at 0 this happens whenever a flag is not already
there, so these tests run the scan with that path taken everywhere and require the results
to be bitwise those of the default run (the scan folds the same records in the same order
whoever computes them), and within the parity tolerance of the fp64 oracle.
"""
import numpy as np
import pytest

import oracle
import wkv_inputs
from helpers import assert_wkv_close

pytestmark = pytest.mark.gpu


def _run(wkv, dev, x, gated, state, dtype=None):
    import torch
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(dev) for n in x}
    if dtype is not None:
        for n in ("k", "v", "dy", "r"):
            if n in t:
                t[n] = t[n].to(dtype)
    B, T, C = t["k"].shape
    fws = wkv.forward_workspace(B, T, C, dev)
    outs = {}
    if state:
        st = [t[n].clone() for n in ("sa", "sb", "sp")]
        outs["y"] = wkv.forward_state(t["w"], t["u"], t["k"], t["v"], *st, workspace=fws)
        outs["fin"] = torch.stack(st)
    elif gated:
        outs["y"] = wkv.forward_gated(t["w"], t["u"], t["k"], t["v"], t["r"], workspace=fws)
    else:
        outs["y"] = wkv.forward(t["w"], t["u"], t["k"], t["v"], workspace=fws)
    if gated:
        g = wkv.backward_gated(t["w"], t["u"], t["k"], t["v"], t["r"], t["dy"], fwd_workspace=fws)
        names = ("dk", "dv", "dr", "dw", "du")
    else:
        g = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=fws)
        names = ("dk", "dv", "dw", "du")
    outs.update(zip(names, g))
    # the backward without the forward's workspace runs its own forward scan first
    g2 = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"]) if not (gated or state) else ()
    outs.update(zip(("dk2", "dv2", "dw2", "du2"), g2))
    torch.cuda.synchronize()
    return {n: a.float().cpu().numpy() for n, a in outs.items()}


@pytest.mark.parametrize("case", ["plain", "gated", "state", "bf16"])
@pytest.mark.parametrize("B,T,C", [(2, 640, 130), (1, 1000, 64), (3, 333, 70)])
def test_recomputed_windows_are_bitwise_the_same(wkv, dev, case, B, T, C):
    x = wkv_inputs.generate("l3b", seed=61 + T, B=B, T=T, C=C)
    rng = np.random.default_rng(62 + T)
    if case == "gated":
        x["r"] = rng.standard_normal((B, T, C)).astype(np.float32)
    if case == "state":
        for n, a in zip(("sa", "sb", "sp"), wkv_inputs.random_state(B, C, seed=63 + T)):
            x[n] = a
    import torch
    dtype = torch.bfloat16 if case == "bf16" else None
    ref = _run(wkv, dev, x, case == "gated", case == "state", dtype)
    old = wkv.set_poll_limit(0)
    try:
        got = _run(wkv, dev, x, case == "gated", case == "state", dtype)
    finally:
        wkv.set_poll_limit(old)
    for n in ref:
        assert np.array_equal(got[n], ref[n]), n
    if case == "plain":
        assert_wkv_close(got["y"], oracle.forward_direct(x["w"], x["u"], x["k"], x["v"]), "y")
        for n, r in zip(("dk", "dv", "dw", "du"),
                        oracle.backward_direct(x["w"], x["u"], x["k"], x["v"], x["dy"])):
            assert_wkv_close(got[n], r, n)
            assert np.array_equal(got[n + "2"], got[n]), n + " without the forward workspace"
