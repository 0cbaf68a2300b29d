"""The operator's plain boundary called exactly as declared, through ctypes (marked gpu).

wkv_forward(B, T, C, w, u, k, v, y, stream), wkv_backward_workspace_size(B, T, C),
wkv_backward(B, T, C, w, u, k, v, dy, dk, dv, dw, du, workspace, bytes, stream) and
wkv_decode_step(B, C, w, u, k, v, a, b, p, y, stream), with device pointers from torch,
against the fp64 oracle; the training pair (wkv_forward_train / wkv_backward_train) gives
bitwise the same gradients; and a backward refuses a workspace that an inference forward
filled: on the host when this process filled it, through the workspace's stamp (NaN dw,
du) when it cannot know. Training is the parallel pass plus gradients ("RWKV
についての調査記録", section "Trainingについて"); inference takes a token and a state
("RWKV についての調査記録", section "RWKVとは？").
"""
import ctypes

import numpy as np
import pytest

import oracle
import wkv_inputs
from helpers import assert_wkv_close

pytestmark = pytest.mark.gpu

SHAPES = [(1, 64, 64), (2, 37, 70), (3, 300, 130), (1, 1000, 5)]


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _dev_inputs(dev, x):
    import torch
    return {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(dev) for n in x}


@pytest.mark.parametrize("B,T,C", SHAPES)
def test_plain_forward_and_backward_as_declared(wkv, dev, B, T, C):
    import torch
    lib = wkv.load_library()
    x = wkv_inputs.generate("small" if (B, T, C) == (1, 64, 64) else "l3b",
                            seed=None if (B, T, C) == (1, 64, 64) else 90 + T, B=B, T=T, C=C)
    t = _dev_inputs(dev, x)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    y = torch.empty_like(t["k"])
    assert lib.wkv_forward(B, T, C, _p(t["w"]), _p(t["u"]), _p(t["k"]), _p(t["v"]), _p(y),
                           st) == wkv.WKV_OK
    nbytes = lib.wkv_backward_workspace_size(B, T, C)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dk, dv = torch.empty_like(t["k"]), torch.empty_like(t["k"])
    dw, du = torch.empty_like(t["w"]), torch.empty_like(t["w"])
    assert lib.wkv_backward(B, T, C, _p(t["w"]), _p(t["u"]), _p(t["k"]), _p(t["v"]),
                            _p(t["dy"]), _p(dk), _p(dv), _p(dw), _p(du), _p(ws), nbytes,
                            st) == wkv.WKV_OK
    torch.cuda.synchronize()
    assert_wkv_close(y.cpu().numpy(), oracle.forward_direct(x["w"], x["u"], x["k"], x["v"]),
                     "y")
    refs = oracle.backward_direct(x["w"], x["u"], x["k"], x["v"], x["dy"])
    worst = 0.0
    for g, r, n in zip((dk, dv, dw, du), refs, ("dk", "dv", "dw", "du")):
        worst = max(worst, assert_wkv_close(g.cpu().numpy(), r, n))
    print("[boundary] B=%d T=%d C=%d max_violation=%.3g" % (B, T, C, worst), flush=True)

    # the training pair: same y, and bitwise the same gradients
    fbytes = lib.wkv_forward_workspace_size(B, T, C)
    fws = torch.empty(fbytes, dtype=torch.uint8, device=dev)
    y2 = torch.empty_like(y)
    assert lib.wkv_forward_train(B, T, C, _p(t["w"]), _p(t["u"]), _p(t["k"]), _p(t["v"]),
                                 _p(y2), _p(fws), fbytes, st) == wkv.WKV_OK
    bbytes = lib.wkv_backward_train_workspace_size(B, T, C)
    bws = torch.empty(bbytes, dtype=torch.uint8, device=dev)
    g2 = [torch.empty_like(a) for a in (dk, dv, dw, du)]
    assert lib.wkv_backward_train(B, T, C, _p(t["w"]), _p(t["u"]), _p(t["k"]), _p(t["v"]),
                                  _p(t["dy"]), _p(fws), *(_p(a) for a in g2), _p(bws), bbytes,
                                  st) == wkv.WKV_OK
    torch.cuda.synchronize()
    assert_wkv_close(y2.cpu().numpy(), y.cpu().numpy().astype(np.float64), "training y")
    for a, b_, n in zip(g2, (dk, dv, dw, du), ("dk", "dv", "dw", "du")):
        assert torch.equal(a, b_), n


def test_decode_step_as_declared(wkv, dev):
    import torch
    lib = wkv.load_library()
    B, C = 16, 96
    wn, un = wkv_inputs.decode_layer_params(3, C=C)
    w, u = torch.from_numpy(wn).to(dev), torch.from_numpy(un).to(dev)
    state = wkv_inputs.empty_decode_state(B, C)
    a, b, p = (torch.from_numpy(s).to(dev) for s in state)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ref = None
    for step in range(20):
        kn, vn = wkv_inputs.decode_step_inputs(step, 3, B=B, C=C)
        k, v = torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev)
        y = torch.empty(B, C, device=dev)
        assert lib.wkv_decode_step(B, C, _p(w), _p(u), _p(k), _p(v), _p(a), _p(b), _p(p), _p(y),
                                   st) == wkv.WKV_OK
        yr, ref = oracle.decode_step(wn, un, kn, vn, ref)
        torch.cuda.synchronize()
        assert_wkv_close(y.cpu().numpy(), yr, "decode step %d" % step)


def test_backward_refuses_an_inference_workspace(wkv, dev):
    import torch
    lib = wkv.load_library()
    B, T, C = 2, 200, 64
    x = wkv_inputs.generate("l3b", seed=95, B=B, T=T, C=C)
    t = _dev_inputs(dev, x)
    ws = wkv.forward_workspace(B, T, C, dev)
    wkv.forward_infer(t["w"], t["u"], t["k"], t["v"], workspace=ws)
    # this process filled it: refused on the host before any launch
    with pytest.raises(wkv.WKVError) as err:
        wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=ws)
    assert err.value.status == wkv.WKV_ERR_INVALID_ARG
    assert "wkv_forward_infer" in str(err.value)
    # sizes that differ from the forward's: refused too
    ws2 = wkv.forward_workspace(B, T, C, dev)
    wkv.forward(t["w"], t["u"], t["k"], t["v"], workspace=ws2)
    x2 = {n: (a[:1] if a.ndim == 3 else a) for n, a in x.items()}
    t2 = _dev_inputs(dev, x2)
    with pytest.raises(wkv.WKVError):
        wkv.backward(t2["w"], t2["u"], t2["k"], t2["v"], t2["dy"], fwd_workspace=ws2)
    # a copy at another address carries no host record: the stamp makes dw, du NaN
    moved = ws.clone()
    torch.cuda.synchronize()
    dk, dv, dw, du = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=moved)
    torch.cuda.synchronize()
    assert torch.isnan(dw).all() and torch.isnan(du).all()
    # while a copy of a training workspace is accepted and gives the same gradients
    good = ws2.clone()
    ref = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"])
    got = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=good)
    torch.cuda.synchronize()
    for a, b_ in zip(got, ref):
        assert torch.equal(a, b_)
