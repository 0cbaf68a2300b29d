"""The forward for inference (marked gpu).

wkv_forward_infer runs the same scan as the training forward but keeps none of the states a
backward reads (its records hold a, b and P only and no chunk carries are stored), so its
outputs, and the state after the last token, must be bitwise those of wkv_forward,
wkv_forward_gated, wkv_forward_typed and wkv_forward_state on the same inputs; with the
look-back's recomputation path taken everywhere too. The prompt-then-generate use of the
recursive form ("RWKV についての調査記録", section "コードを見ながらRWKVの構造を把握").
"""
import numpy as np
import pytest

import oracle
import wkv_inputs
from helpers import assert_wkv_close

pytestmark = pytest.mark.gpu

SHAPES = [(2, 37, 70), (3, 300, 130), (1, 1000, 64), (2, 129, 128)]


def _tensors(dev, x, names, dtype=None):
    import torch
    out = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(dev) for n in names}
    if dtype is not None:
        for n in ("k", "v", "r"):
            if n in out:
                out[n] = out[n].to(dtype)
    return out


@pytest.mark.parametrize("B,T,C", SHAPES)
@pytest.mark.parametrize("poll", [None, 0])
def test_infer_equals_training_forward(wkv, dev, B, T, C, poll):
    import torch
    x = wkv_inputs.generate("l3b", seed=71 + T, B=B, T=T, C=C, with_dy=False)
    rng = np.random.default_rng(72 + T)
    x["r"] = rng.standard_normal((B, T, C)).astype(np.float32)
    t = _tensors(dev, x, ("w", "u", "k", "v", "r"))
    st = [torch.from_numpy(a).to(dev) for a in wkv_inputs.random_state(B, C, seed=73 + T)]
    ref = {"y": wkv.forward(t["w"], t["u"], t["k"], t["v"]),
           "g": wkv.forward_gated(t["w"], t["u"], t["k"], t["v"], t["r"])}
    st_ref = [a.clone() for a in st]
    ref["ys"] = wkv.forward_state(t["w"], t["u"], t["k"], t["v"], *st_ref)
    old = wkv.set_poll_limit(poll) if poll is not None else None
    try:
        got = {"y": wkv.forward_infer(t["w"], t["u"], t["k"], t["v"]),
               "g": wkv.forward_infer(t["w"], t["u"], t["k"], t["v"], r=t["r"])}
        st_got = [a.clone() for a in st]
        got["ys"] = wkv.forward_infer(t["w"], t["u"], t["k"], t["v"], state=st_got)
    finally:
        if old is not None:
            wkv.set_poll_limit(old)
    torch.cuda.synchronize()
    for n in ref:
        assert torch.equal(got[n], ref[n]), n
    for a, b_, n in zip(st_got, st_ref, "abp"):
        assert torch.equal(a, b_), "state " + n
    if poll is None:
        assert_wkv_close(got["y"].cpu().numpy(),
                         oracle.forward_direct(x["w"], x["u"], x["k"], x["v"]), "y")


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
def test_infer_16bit_equals_typed_forward(wkv, dev, dtype):
    import torch
    dt = getattr(torch, dtype)
    B, T, C = 2, 300, 130
    x = wkv_inputs.generate("l3b", seed=74, B=B, T=T, C=C, with_dy=False)
    x["r"] = np.random.default_rng(75).standard_normal((B, T, C)).astype(np.float32)
    t = _tensors(dev, x, ("w", "u", "k", "v", "r"), dt)
    for r in (None, t["r"]):
        ref = (wkv.forward(t["w"], t["u"], t["k"], t["v"]) if r is None
               else wkv.forward_gated(t["w"], t["u"], t["k"], t["v"], r))
        got = wkv.forward_infer(t["w"], t["u"], t["k"], t["v"], r=r)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)


def test_infer_3b_layer_prefill(wkv, dev):
    # the 3B-class layer from a state: y and the final state as forward_state gives them
    import torch
    x = wkv_inputs.generate("l3b", with_dy=False)
    t = _tensors(dev, x, ("w", "u", "k", "v"))
    B, T, C = x["k"].shape
    st = [torch.from_numpy(a).to(dev) for a in wkv_inputs.random_state(B, C, seed=76)]
    s1, s2 = [a.clone() for a in st], [a.clone() for a in st]
    ref = wkv.forward_state(t["w"], t["u"], t["k"], t["v"], *s1)
    got = wkv.forward_infer(t["w"], t["u"], t["k"], t["v"], state=s2)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    for a, b_ in zip(s1, s2):
        assert torch.equal(a, b_)
