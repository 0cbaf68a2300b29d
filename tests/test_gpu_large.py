"""Parity at the largest sizes (marked gpu): past 2^31 elements per tensor, and the largest
channel counts accepted.

The [B, T, C] tensors here hold 2.15e9 elements (8.6 GB each in fp32), so every element
offset needs 64 bits; T and C are ragged (neither a multiple of the 64-token window nor of
the 64-channel group). The inputs follow the 3B-class layer's distributions but are drawn
on the device; outputs are checked on sampled channels, whose whole sequences the fp64
oracle recomputes (the recursive form of formula (8), "RWKV解读：在Transformer的时代的新
RNN", section 二.3, and its gradients), with the parity tolerance of the other tests.
"""
import numpy as np
import pytest

import oracle
from helpers import assert_wkv_close

pytestmark = pytest.mark.gpu


def test_beyond_2_31_elements(wkv, dev):
    import torch
    B, T, C = 2, 32805, 32800
    assert B * T * C > 2 ** 31
    g = torch.Generator(device=dev)
    g.manual_seed(2031)
    w = torch.exp(torch.rand(C, device=dev, generator=g) * 10 - 8)
    u = torch.rand(C, device=dev, generator=g) * 2 - 1
    k = torch.randn(B, T, C, device=dev, generator=g)
    v = torch.randn(B, T, C, device=dev, generator=g)
    fws = wkv.forward_workspace(B, T, C, dev)
    y = wkv.forward(w, u, k, v, workspace=fws)
    dy = torch.randn(B, T, C, device=dev, generator=g)
    dk, dv, dw, du = wkv.backward(w, u, k, v, dy, fwd_workspace=fws)
    torch.cuda.synchronize()
    idx = torch.tensor([0, 63, 64, 12345, 16447, C - 37, C - 1], device=dev)
    host = lambda t: t.index_select(-1, idx).double().cpu().numpy()
    wn, un = host(w), host(u)
    kn, vn, dyn = host(k), host(v), host(dy)
    del k, v, dy, fws
    yr, _ = oracle.forward_rescaled(wn, un, kn, vn)
    worst = {"y": assert_wkv_close(host(y), yr, "y")}
    ref = oracle.backward_recurrent(wn, un, kn, vn, dyn)
    for got, r, n in zip((host(dk), host(dv), host(dw), host(du)), ref, ("dk", "dv", "dw", "du")):
        worst[n] = assert_wkv_close(got, r, n)
    print("[large] B=%d T=%d C=%d max_violation %s" % (
        B, T, C, " ".join("%s %.3g" % kv for kv in worst.items())), flush=True)


@pytest.mark.parametrize("B,T,C", [(1, 3, 1 << 24), (2, 100, (1 << 22) + 37)])
def test_largest_channel_counts(wkv, dev, B, T, C):
    # C up to the largest accepted (2^24): the last channels' rows sit 2^26 bytes apart, the
    # largest row stride the 32-bit buffer offsets have to span
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(2032 + T)
    w = torch.exp(torch.rand(C, device=dev, generator=g) * 10 - 8)
    u = torch.rand(C, device=dev, generator=g) * 2 - 1
    k = torch.randn(B, T, C, device=dev, generator=g)
    v = torch.randn(B, T, C, device=dev, generator=g)
    dy = torch.randn(B, T, C, device=dev, generator=g)
    fws = wkv.forward_workspace(B, T, C, dev)
    y = wkv.forward(w, u, k, v, workspace=fws)
    dk, dv, dw, du = wkv.backward(w, u, k, v, dy, fwd_workspace=fws)
    torch.cuda.synchronize()
    idx = torch.tensor([0, 1, 63, 64, C // 2, C - 65, C - 64, C - 2, C - 1], device=dev)
    host = lambda t: t.index_select(-1, idx).double().cpu().numpy()
    wn, un, kn, vn, dyn = host(w), host(u), host(k), host(v), host(dy)
    assert_wkv_close(host(y), oracle.forward_direct(wn, un, kn, vn), "y")
    ref = oracle.backward_direct(wn, un, kn, vn, dyn)
    for got, r, n in zip((host(dk), host(dv), host(dw), host(du)), ref, ("dk", "dv", "dw", "du")):
        assert_wkv_close(got, r, n)
