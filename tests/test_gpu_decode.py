"""GPU parity of wkv_decode_step against the fp64 oracle (marked gpu).

The recursive form of formula (8) ("RWKV解读：在Transformer的时代的新RNN", section 二.3);
inference takes a token and a state and returns the new state ("RWKV についての調査記録",
section "RWKVとは？"). States are compared through what is unique about them: the ratio
a/b (a convex combination of past v) and the log-mass p + ln b; (a e^d, b e^d, p - d)
is the same state for any d.
"""
import numpy as np
import pytest

import oracle
import wkv_inputs
from helpers import assert_wkv_close

pytestmark = pytest.mark.gpu


def _t(dev, a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def test_decode_chain_equals_parallel_form(wkv, dev):
    import torch
    x = wkv_inputs.generate("l3b", seed=21, B=3, T=60, C=70, with_dy=False)
    ref = oracle.forward_direct(x["w"], x["u"], x["k"], x["v"])
    w, u = _t(dev, x["w"]), _t(dev, x["u"])
    a, b, p = (_t(dev, s) for s in wkv_inputs.empty_decode_state(3, 70))
    for t in range(60):
        y = wkv.decode_step(w, u, _t(dev, x["k"][:, t]), _t(dev, x["v"][:, t]), a, b, p)
        torch.cuda.synchronize()
        assert_wkv_close(y.cpu().numpy(), ref[:, t], "t=%d" % t)


@pytest.mark.parametrize("B", [1, 2, 3, 5, 6, 7, 9])
def test_decode_ragged_row_groups(wkv, dev, B):
    """A lane decodes a group of four sequences; a group cut short by B (remainders 1, 2 and 3,
    alone and after whole groups) repeats its first sequence in the missing rows, and that
    repeat must not apply the first sequence's update twice: several steps against the
    oracle's chain, then the state."""
    import torch
    C, steps, layer = 70, 6, 3
    wn, un = wkv_inputs.decode_layer_params(layer, C=C)
    w, u = _t(dev, wn), _t(dev, un)
    ost = wkv_inputs.empty_decode_state(B, C)
    a, b, p = (_t(dev, s) for s in ost)
    for s in range(steps):
        kn, vn = wkv_inputs.decode_step_inputs(s, layer, B=B, C=C)
        y = wkv.decode_step(w, u, _t(dev, kn), _t(dev, vn), a, b, p)
        yr, ost = oracle.decode_step(wn, un, kn, vn, ost)
        torch.cuda.synchronize()
        assert_wkv_close(y.cpu().numpy(), yr, "B=%d step %d" % (B, s))
    ga, gb, gp = (t.cpu().numpy().astype(np.float64) for t in (a, b, p))
    oa, ob, op = ost
    assert_wkv_close(ga / gb, oa / ob, "state ratio")
    np.testing.assert_allclose(gp + np.log(gb), op + np.log(ob), rtol=0, atol=1e-4)


@pytest.mark.parametrize("layer,B,steps", [(0, 256, 1000), (39, 256, 1000), (7, 8, 1000)])
def test_batched_decode_workload(wkv, dev, layer, B, steps):
    """The batched decode workload's full width (256 sequences x 5120 channels) over its whole
    horizon of 1000 steps, for the first and the last of its 40 layer states (and a narrow
    batch of a middle layer): every step's y against the oracle's chain, then the state."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    C = wkv_inputs.DECODE["C"]
    wn, un = wkv_inputs.decode_layer_params(layer)
    w, u = _t(dev, wn), _t(dev, un)
    st = wkv_inputs.empty_decode_state(B, C)
    a, b, p = (_t(dev, s) for s in st)
    ost = st
    worst = 0.0
    # the next step's inputs are drawn while this step runs (the draws are what they are,
    # whichever thread makes them)
    with ThreadPoolExecutor(max_workers=1) as pool:
        nxt = pool.submit(wkv_inputs.decode_step_inputs, 0, layer, None, B)
        for s in range(steps):
            kn, vn = nxt.result()
            if s + 1 < steps:
                nxt = pool.submit(wkv_inputs.decode_step_inputs, s + 1, layer, None, B)
            y = wkv.decode_step(w, u, _t(dev, kn), _t(dev, vn), a, b, p)
            yr, ost = oracle.decode_step(wn, un, kn, vn, ost)
            torch.cuda.synchronize()
            worst = max(worst, assert_wkv_close(y.cpu().numpy(), yr,
                                                "layer %d step %d" % (layer, s)))
    ga, gb, gp = (t.cpu().numpy().astype(np.float64) for t in (a, b, p))
    oa, ob, op = ost
    assert_wkv_close(ga / gb, oa / ob, "state ratio")
    np.testing.assert_allclose(gp + np.log(gb), op + np.log(ob), rtol=0, atol=1e-4)
    print("[decode] layer %d steps %d max_violation=%.3g" % (layer, steps, worst), flush=True)


def test_resume_through_host_is_bitwise(wkv, dev):
    import torch
    x = wkv_inputs.generate("l3b", seed=22, B=4, T=20, C=256, with_dy=False)
    w, u = _t(dev, x["w"]), _t(dev, x["u"])

    def run(a, b, p, t0, t1):
        ys = []
        for t in range(t0, t1):
            ys.append(wkv.decode_step(w, u, _t(dev, x["k"][:, t]), _t(dev, x["v"][:, t]), a, b, p))
        torch.cuda.synchronize()
        return [y.cpu().numpy() for y in ys]

    st = [_t(dev, s) for s in wkv_inputs.empty_decode_state(4, 256)]
    y_all = run(*st, 0, 20)
    st2 = [_t(dev, s) for s in wkv_inputs.empty_decode_state(4, 256)]
    y1 = run(*st2, 0, 9)
    host = [s.cpu().numpy() for s in st2]
    st3 = [_t(dev, s) for s in host]
    y2 = run(*st3, 9, 20)
    for g, r in zip(y1 + y2, y_all):
        assert np.array_equal(g, r)
    for s, r in zip(st3, st):
        assert np.array_equal(s.cpu().numpy(), r.cpu().numpy())


@pytest.mark.parametrize("kbig", [30.0, 1000.0])
def test_sentinels_and_large_keys(wkv, dev, kbig):
    """Both empty-state sentinels (p = -1e38 and -inf), with every seventh step's keys drawn
    with standard deviation kbig (30: the long-context workload's spikes; 1000: far beyond
    any workload), at the stated tolerance."""
    import torch
    B, C = 2, 64
    rng = np.random.default_rng(23)
    w = np.exp(rng.uniform(-8, 2, C)).astype(np.float32)
    u = rng.uniform(-1, 1, C).astype(np.float32)
    a = np.zeros((B, C), np.float32)
    b = np.zeros((B, C), np.float32)
    p = np.full((B, C), -np.inf, np.float32)
    p[0] = -1e38
    ta, tb, tp = _t(dev, a), _t(dev, b), _t(dev, p)
    st = (a.astype(np.float64), b.astype(np.float64), np.full((B, C), -1e38))
    for s in range(40):
        k = (rng.standard_normal((B, C)) * (kbig if s % 7 == 3 else 3.0)).astype(np.float32)
        v = rng.standard_normal((B, C)).astype(np.float32)
        y = wkv.decode_step(_t(dev, w), _t(dev, u), _t(dev, k), _t(dev, v), ta, tb, tp)
        yr, st = oracle.decode_step(w, u, k, v, st)
        torch.cuda.synchronize()
        yg = y.cpu().numpy()
        assert np.all(np.isfinite(yg))
        assert_wkv_close(yg, yr, "step %d" % s)


def test_decode_rejects_bad_output_tensor(wkv, dev):
    # a wrong `out` is refused before any launch (the kernel would write B*C floats to it)
    import torch
    B, C = 4, 96
    k = torch.zeros(B, C, device=dev)
    w = torch.ones(C, device=dev)
    st = [torch.zeros(B, C, device=dev) for _ in range(3)]
    for bad in (torch.zeros(B, C - 1, device=dev), torch.zeros(B * C, device=dev),
                torch.zeros(B, C, device=dev, dtype=torch.float64)):
        with pytest.raises((ValueError, TypeError)):
            wkv.decode_step(w, w, k, k, *st, out=bad)
    y = wkv.decode_step(w, w, k, k, *st, out=torch.empty(B, C, device=dev))
    torch.cuda.synchronize()
    assert y.shape == (B, C)


def _decode_inputs(torch, dev, B, C, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    w = torch.exp(torch.rand(C, device=dev, generator=g) * 10 - 8)
    u = torch.rand(C, device=dev, generator=g) * 2 - 1
    k = torch.randn(B, C, device=dev, generator=g) * 3
    v = torch.randn(B, C, device=dev, generator=g)
    b = torch.rand(B, C, device=dev, generator=g) * 4 + 1
    a = b * torch.randn(B, C, device=dev, generator=g)
    p = torch.randn(B, C, device=dev, generator=g) * 5
    return w, u, k, v, a, b, p


def test_decode_grid_stride_pass(wkv, dev):
    # more groups of four sequences than a grid's y extent (65535): the launch caps its grid
    # and each workgroup row loops over groups; the last group holds three sequences. The
    # result is bitwise that of the same rows decoded in two calls of one pass each.
    import torch
    B, C = 262203, 70
    assert (B + 3) // 4 > 65535 and (B // 2 + 3) // 4 <= 65535
    w, u, k, v, a, b, p = _decode_inputs(torch, dev, B, C, 32)
    st = [t.clone() for t in (a, b, p)]
    y = wkv.decode_step(w, u, k, v, *st)
    half = B // 2
    yh = torch.empty_like(y)
    for r0, r1 in ((0, half), (half, B)):
        wkv.decode_step(w, u, k[r0:r1], v[r0:r1], a[r0:r1], b[r0:r1], p[r0:r1], out=yh[r0:r1])
    torch.cuda.synchronize()
    assert torch.equal(y, yh)
    for x, z in zip(st, (a, b, p)):
        assert torch.equal(x, z)


def test_decode_graph_replays_match_eager(wkv, dev):
    # a serving loop captures its per-layer decode calls once and replays them: every replay
    # (with eager work and synchronizations in between) must equal the same calls made eagerly
    import torch
    B, C, L = 16, 320, 4
    per = [_decode_inputs(torch, dev, B, C, 40 + l) for l in range(L)]
    gst = [[t.clone() for t in x[4:]] for x in per]
    est = [[t.clone() for t in x[4:]] for x in per]
    kv = torch.empty(L, 2, B, C, device=dev)
    y = torch.empty(L, B, C, device=dev)

    def calls(st, out):
        for l in range(L):
            w, u = per[l][0], per[l][1]
            wkv.decode_step(w, u, kv[l, 0], kv[l, 1], *st[l], out=out[l])

    kv.normal_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(gst, y)  # warm-up outside the capture, as a real loop would
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ye = torch.empty_like(y)
    calls(est, ye)  # the eager twin takes the same first step
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(gst, y)
    torch.cuda.synchronize()
    for r in range(4):
        kv.normal_()
        torch.cuda.synchronize()
        g.replay()
        calls(est, ye)
        torch.cuda.synchronize()
        assert torch.equal(y, ye), "replay %d" % r
        for l in range(L):
            for x, z in zip(gst[l], est[l]):
                assert torch.equal(x, z), "replay %d layer %d" % (r, l)


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
def test_decode_16bit_storage(wkv, dev, dtype):
    """k, v, y stored in 16 bits, the state in fp32: y and the state are bitwise those of the
    fp32 decode on the same (exactly widened) k, v, with y rounded to the format to nearest
    even; and the chain follows the oracle on those inputs to the fp32 tolerance plus one
    unit in the format's last place."""
    import torch
    from helpers import assert_io_close
    tdt = getattr(torch, dtype)
    B, C, steps = 33, 200, 40
    layer = 5
    wn, un = wkv_inputs.decode_layer_params(layer, C=C)
    w, u = _t(dev, wn), _t(dev, un)
    s16 = [_t(dev, s) for s in wkv_inputs.empty_decode_state(B, C)]
    s32 = [t.clone() for t in s16]
    ost = wkv_inputs.empty_decode_state(B, C)
    worst = 0.0
    for s in range(steps):
        kn, vn = wkv_inputs.decode_step_inputs(s, layer, B=B, C=C)
        k16, v16 = _t(dev, kn).to(tdt), _t(dev, vn).to(tdt)
        y16 = wkv.decode_step(w, u, k16, v16, *s16)
        y32 = wkv.decode_step(w, u, k16.float(), v16.float(), *s32)
        torch.cuda.synchronize()
        assert y16.dtype == tdt
        assert torch.equal(y16, y32.to(tdt)), "step %d" % s
        for x, z in zip(s16, s32):
            assert torch.equal(x, z), "state, step %d" % s
        kw, vw = (t.float().cpu().numpy() for t in (k16, v16))
        yr, ost = oracle.decode_step(wn, un, kw, vw, ost)
        worst = max(worst, assert_io_close(y16.float().cpu().numpy(), yr, dtype,
                                           "%s step %d" % (dtype, s)))
    print("[decode %s] max allowance used %.3g" % (dtype, worst), flush=True)
