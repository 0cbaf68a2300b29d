"""GPU parity of the 16-bit storage formats (bfloat16, float16) against the fp64 oracle
(marked gpu).

k, v, dy (and r) are rounded to the format on the host; the oracle runs on those rounded
values widened exactly, so both sides see the same inputs. Outputs in the format (y, out,
dk, dv, dr) must be within the fp32 tolerance plus one unit in the last place of the format
(tests/helpers.py assert_io_close); dw, du stay fp32 and keep the plain tolerance. The
arithmetic is the fp32 path's ("RWKV解读：在Transformer的时代的新RNN", section 二.3, formula
(8)). The pages measure in float32 and leave reduced precision to later work ("RWKV について
の調査記録", section "推論実験"; "介绍RWKV – 具有Transformer优势的RNN", section
"模型压缩和加速"), so the allowance for 16-bit outputs is a reading, not a number they give.
"""
import numpy as np
import pytest

import oracle
import wkv_inputs
from gate_ref import backward_gated, forward_gated
from helpers import assert_io_close, assert_wkv_close

pytestmark = pytest.mark.gpu

FORMATS = ["bfloat16", "float16"]


def _dev_io(dev, x, fmt):
    """Device tensors of x in the format (w, u stay fp32) and the rounded values in fp64."""
    import torch
    dt = getattr(torch, fmt)
    t, rounded = {}, {}
    for n, a in x.items():
        ta = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        if a.ndim == 3:
            ta = ta.to(dt)
            rounded[n] = ta.float().cpu().numpy().astype(np.float64)
        else:
            rounded[n] = a.astype(np.float64)
        t[n] = ta
    return t, rounded


def _log(what, v):
    print("[typed] %s max=%.3g" % (what, v), flush=True)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 37, 70), (3, 300, 130), (2, 513, 65),
                                   (4, 31, 200)])
def test_forward_backward(wkv, dev, fmt, B, T, C):
    import torch
    x = wkv_inputs.generate("l3b", seed=71 + B * T + C, B=B, T=T, C=C)
    t, xr = _dev_io(dev, x, fmt)
    ws = wkv.forward_workspace(B, T, C, dev)
    y = wkv.forward(t["w"], t["u"], t["k"], t["v"], workspace=ws)
    dk, dv, dw, du = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=ws)
    torch.cuda.synchronize()
    assert y.dtype == t["k"].dtype and dk.dtype == t["k"].dtype and dw.dtype == torch.float32
    ry = oracle.forward_direct(xr["w"], xr["u"], xr["k"], xr["v"])
    rk, rv, rw, ru = oracle.backward_direct(xr["w"], xr["u"], xr["k"], xr["v"], xr["dy"])
    name = "%s B=%d T=%d C=%d" % (fmt, B, T, C)
    v = assert_io_close(y.float().cpu().numpy(), ry, fmt, name + " y")
    v = max(v, assert_io_close(dk.float().cpu().numpy(), rk, fmt, name + " dk"))
    v = max(v, assert_io_close(dv.float().cpu().numpy(), rv, fmt, name + " dv"))
    v = max(v, assert_wkv_close(dw.cpu().numpy(), rw, name + " dw"))
    v = max(v, assert_wkv_close(du.cpu().numpy(), ru, name + " du"))
    _log(name, v)


@pytest.mark.parametrize("fmt", FORMATS)
def test_gated(wkv, dev, fmt):
    import torch
    B, T, C = 2, 300, 96
    x = wkv_inputs.generate("l3b", seed=72, B=B, T=T, C=C)
    x["r"] = np.random.default_rng(73).standard_normal((B, T, C)).astype(np.float32)
    t, xr = _dev_io(dev, x, fmt)
    ws = wkv.forward_workspace(B, T, C, dev)
    o = wkv.forward_gated(t["w"], t["u"], t["k"], t["v"], t["r"], workspace=ws)
    g = wkv.backward_gated(t["w"], t["u"], t["k"], t["v"], t["r"], t["dy"], fwd_workspace=ws)
    torch.cuda.synchronize()
    ro = forward_gated(xr["w"], xr["u"], xr["k"], xr["v"], xr["r"])
    refs = backward_gated(xr["w"], xr["u"], xr["k"], xr["v"], xr["r"], xr["dy"])
    v = assert_io_close(o.float().cpu().numpy(), ro, fmt, fmt + " out")
    for got, ref, n in zip(g, refs, ("dk", "dv", "dr", "dw", "du")):
        if n in ("dw", "du"):
            v = max(v, assert_wkv_close(got.cpu().numpy(), ref, fmt + " " + n))
        else:
            v = max(v, assert_io_close(got.float().cpu().numpy(), ref, fmt, fmt + " " + n))
    _log(fmt + " gated", v)


@pytest.mark.parametrize("fmt", FORMATS)
def test_without_forward_workspace_and_large_keys(wkv, dev, fmt):
    """The backward's own forward pass, and keys 1000 apart (the per-token paths)."""
    import torch
    B, T, C = 2, 400, 96
    x = wkv_inputs.generate("l3b", seed=74, B=B, T=T, C=C)
    rng = np.random.default_rng(75)
    m = rng.random(x["k"].shape) < 0.02
    x["k"] = np.where(m, np.float32(1000.0) * np.sign(rng.standard_normal(x["k"].shape)),
                      x["k"]).astype(np.float32)
    t, xr = _dev_io(dev, x, fmt)
    y = wkv.forward(t["w"], t["u"], t["k"], t["v"])
    dk, dv, dw, du = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"])
    torch.cuda.synchronize()
    ry = oracle.forward_direct(xr["w"], xr["u"], xr["k"], xr["v"])
    rk, rv, rw, ru = oracle.backward_direct(xr["w"], xr["u"], xr["k"], xr["v"], xr["dy"])
    v = assert_io_close(y.float().cpu().numpy(), ry, fmt, fmt + " y")
    v = max(v, assert_io_close(dk.float().cpu().numpy(), rk, fmt, fmt + " dk"))
    v = max(v, assert_io_close(dv.float().cpu().numpy(), rv, fmt, fmt + " dv"))
    v = max(v, assert_wkv_close(dw.cpu().numpy(), rw, fmt + " dw"))
    v = max(v, assert_wkv_close(du.cpu().numpy(), ru, fmt + " du"))
    _log(fmt + " own forward, large keys", v)


@pytest.mark.parametrize("fmt", FORMATS)
def test_full_layer(wkv, dev, fmt):
    """The 3B-class layer shape in the format (linear-time oracle)."""
    import torch
    x = wkv_inputs.generate("l3b")
    t, xr = _dev_io(dev, x, fmt)
    B, T, C = x["k"].shape
    ws = wkv.forward_workspace(B, T, C, dev)
    y = wkv.forward(t["w"], t["u"], t["k"], t["v"], workspace=ws)
    dk, dv, dw, du = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=ws)
    torch.cuda.synchronize()
    ry = oracle.forward_recurrent(xr["w"], xr["u"], xr["k"], xr["v"])
    rk, rv, rw, ru = oracle.backward_recurrent(xr["w"], xr["u"], xr["k"], xr["v"], xr["dy"])
    v = assert_io_close(y.float().cpu().numpy(), ry, fmt, fmt + " l3b y")
    v = max(v, assert_io_close(dk.float().cpu().numpy(), rk, fmt, fmt + " l3b dk"))
    v = max(v, assert_io_close(dv.float().cpu().numpy(), rv, fmt, fmt + " l3b dv"))
    v = max(v, assert_wkv_close(dw.cpu().numpy(), rw, fmt + " l3b dw"))
    v = max(v, assert_wkv_close(du.cpu().numpy(), ru, fmt + " l3b du"))
    _log(fmt + " l3b", v)
