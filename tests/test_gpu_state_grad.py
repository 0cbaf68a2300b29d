"""GPU parity of wkv_backward_state against the fp64 oracle (marked gpu).

A sequence run in pieces, each resuming from the state the previous one left ("RWKV
についての調査記録", section "RWKVとは？": the state is what carries the past), is trained
through those states when the gradient reaches the state each piece started from. The
reference is the oracle's direct backward of the piece with the state's token prepended
(key p + ln b, value a / b), whose own dk, dv give da, db, dp by the chain rule
(tests/state_ref.py, pinned against finite differences and a closed form in
test_oracle_state.py). dk, dv, dw, du must be bitwise those of wkv_backward.
"""
import numpy as np
import pytest

import wkv_inputs
from helpers import assert_wkv_close
from state_ref import backward_state_grad, state_grad_scale

pytestmark = pytest.mark.gpu


def _t(dev, a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _forward_state(wkv, dev, t, state):
    B, T, C = t["k"].shape
    ws = wkv.forward_workspace(B, T, C, dev)
    st = [_t(dev, s) for s in state]
    wkv.forward_state(t["w"], t["u"], t["k"], t["v"], *st, workspace=ws)
    return ws


def _floors(scale):
    """The floor of |x - r| <= 1e-4 max(|r|, floor) per gradient: the operator's 0.1 for dk,
    dv, dr, dw, du; for da, db, dp, which scale with e^p over (b, c) and sum terms of either
    sign, each entry's own conditioning, the sum of the absolute values of its terms
    (state_grad_scale, pinned in test_oracle_state.py), so each is judged to 1e-4 of it."""
    sa, sb, sp = scale
    return {"dk": 0.1, "dv": 0.1, "dr": 0.1, "dw": 0.1, "du": 0.1, "da": sa, "db": sb,
            "dp": sp}


def _log(name, v):
    print("[backward_state] %s max_violation=%.3g" % (name, v), flush=True)


@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 37, 70), (1, 64, 64), (3, 129, 130),
                                   (2, 300, 65), (1, 1000, 256)])
@pytest.mark.parametrize("prange", [(-3.0, 3.0), (20.0, 30.0), (-30.0, -20.0)])
def test_state_gradient_parity(wkv, dev, B, T, C, prange):
    """States on the keys' scale, far above it (they dominate the first tokens) and far
    below it (their gradient is tiny but must still be right to the relative bar)."""
    import torch
    x = wkv_inputs.generate("l3b", seed=60 + B * T + C, B=B, T=T, C=C)
    st = wkv_inputs.random_state(B, C, seed=T + C, p_range=prange)
    t = {n: _t(dev, x[n]) for n in ("w", "u", "k", "v", "dy")}
    ws = _forward_state(wkv, dev, t, st)
    got = wkv.backward_state(t["w"], t["u"], t["k"], t["v"], t["dy"], ws)
    torch.cuda.synchronize()
    ref = backward_state_grad(x["w"], x["u"], x["k"], x["v"], x["dy"], st)
    floors = _floors(state_grad_scale(x["w"], x["u"], x["k"], x["v"], x["dy"], st))
    worst = 0.0
    for g, r, n in zip(got, ref, ("dk", "dv", "dw", "du", "da", "db", "dp")):
        r = np.asarray(r, np.float64)
        worst = max(worst, assert_wkv_close(g.cpu().numpy(), r, "%s B=%d T=%d C=%d p in %s"
                                            % (n, B, T, C, prange), floor=floors[n]))
    _log("B=%d T=%d C=%d p in %s" % (B, T, C, prange), worst)


@pytest.mark.parametrize("B,T,C", [(2, 37, 70), (3, 700, 200)])
def test_other_gradients_bitwise_equal_backward(wkv, dev, B, T, C):
    import torch
    x = wkv_inputs.generate("l3b", seed=80 + T, B=B, T=T, C=C)
    st = wkv_inputs.random_state(B, C, seed=81, p_range=(-3.0, 3.0))
    t = {n: _t(dev, x[n]) for n in ("w", "u", "k", "v", "dy")}
    ws = _forward_state(wkv, dev, t, st)
    got = wkv.backward_state(t["w"], t["u"], t["k"], t["v"], t["dy"], ws)
    base = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=ws)
    torch.cuda.synchronize()
    for g, r, n in zip(got[:4], base, ("dk", "dv", "dw", "du")):
        assert torch.equal(g, r), n


def test_empty_state_gives_zero_state_gradient(wkv, dev):
    """From the empty state (wkv_forward, or wkv_forward_state from a = b = 0, p = -1e38 or
    -inf) the state gradient is zero: A = a e^p has no slope in a, b or p there."""
    import torch
    B, T, C = 2, 90, 130
    x = wkv_inputs.generate("l3b", seed=90, B=B, T=T, C=C)
    t = {n: _t(dev, x[n]) for n in ("w", "u", "k", "v", "dy")}
    ws = wkv.forward_workspace(B, T, C, dev)
    wkv.forward(t["w"], t["u"], t["k"], t["v"], workspace=ws)
    outs = [wkv.backward_state(t["w"], t["u"], t["k"], t["v"], t["dy"], ws)]
    e = wkv_inputs.empty_decode_state(B, C)
    for p in (e[2], np.full_like(e[2], -np.inf)):
        ws2 = _forward_state(wkv, dev, t, (e[0], e[1], p))
        outs.append(wkv.backward_state(t["w"], t["u"], t["k"], t["v"], t["dy"], ws2))
    torch.cuda.synchronize()
    for o in outs:
        for g in o[4:]:
            assert torch.count_nonzero(g).item() == 0
        for g, r in zip(o[:4], outs[0][:4]):
            assert torch.equal(g, r)


def test_zero_length_writes_zeros(wkv, dev):
    import torch
    B, C = 3, 70
    w = torch.rand(C, device=dev)
    k = torch.zeros(B, 0, C, device=dev)
    ws = wkv.forward_workspace(B, 0, C, dev)
    out = [torch.full(s, 7.0, device=dev) for s in ((B, 0, C), (B, 0, C), (C,), (C,),
                                                    (B, C), (B, C), (B, C))]
    got = wkv.backward_state(w, w, k, k, k, ws, out=out)
    torch.cuda.synchronize()
    for g in got[2:]:
        assert torch.count_nonzero(g).item() == 0


def test_full_layer_state_gradient(wkv, dev):
    """The 3B-class layer shape (B=8, T=4096, C=2560) from a random state; da, db, dp in
    full and dk, dv on the first 96 tokens, where the state still counts (the oracle's
    direct form is O(T^2) per channel, so it runs on that prefix: the gradients of the
    prefix's loss only, with dy zero beyond it)."""
    import torch
    x = wkv_inputs.generate("l3b")
    B, T, C = x["k"].shape
    Tp = 96
    dy = x["dy"].copy()
    dy[:, Tp:] = 0
    st = wkv_inputs.random_state(B, C, seed=91)
    t = {n: _t(dev, x[n]) for n in ("w", "u", "k", "v")}
    t["dy"] = _t(dev, dy)
    ws = _forward_state(wkv, dev, t, st)
    got = wkv.backward_state(t["w"], t["u"], t["k"], t["v"], t["dy"], ws)
    torch.cuda.synchronize()
    ref = backward_state_grad(x["w"], x["u"], x["k"][:, :Tp], x["v"][:, :Tp], dy[:, :Tp], st)
    floors = _floors(state_grad_scale(x["w"], x["u"], x["k"][:, :Tp], x["v"][:, :Tp],
                                      dy[:, :Tp], st))
    worst = 0.0
    for g, r, n in ((got[0][:, :Tp], ref[0], "dk"), (got[1][:, :Tp], ref[1], "dv"),
                    (got[2], ref[2], "dw"), (got[3], ref[3], "du"), (got[4], ref[4], "da"),
                    (got[5], ref[5], "db"), (got[6], ref[6], "dp")):
        r = np.asarray(r, np.float64)
        worst = max(worst, assert_wkv_close(g.cpu().numpy(), r, "l3b " + n, floor=floors[n]))
    assert torch.count_nonzero(got[0][:, Tp:]).item() == 0
    _log("l3b (loss on the first %d tokens)" % Tp, worst)


def _cot_case(wkv, dev, x, st, seed):
    """GPU forward_state, then backward_state with a cotangent of the final state. The
    cotangent is drawn on (A_T, B_T) from the oracle's own final state (dA = r e^{-p_T}) and
    handed to the GPU in its decode convention (dfa = dA e^{p_T} with the GPU's p_T)."""
    import torch
    from oracle import forward_rescaled
    B, T, C = x["k"].shape
    t = {n: _t(dev, x[n]) for n in ("w", "u", "k", "v", "dy")}
    ws = wkv.forward_workspace(B, T, C, dev)
    sg = [_t(dev, s) for s in st]
    wkv.forward_state(t["w"], t["u"], t["k"], t["v"], *sg, workspace=ws)
    _, (_, _, po) = forward_rescaled(x["w"], x["u"], x["k"], x["v"], st)
    rng = np.random.default_rng(seed)
    ra = rng.standard_normal((B, C)) * 0.5
    rb = rng.standard_normal((B, C)) * 0.5
    dA, dB = ra * np.exp(-po), rb * np.exp(-po)
    pg = sg[2].cpu().numpy().astype(np.float64)
    dfa = _t(dev, (ra * np.exp(pg - po)).astype(np.float32))
    dfb = _t(dev, (rb * np.exp(pg - po)).astype(np.float32))
    got = wkv.backward_state(t["w"], t["u"], t["k"], t["v"], t["dy"], ws, dstate=(dfa, dfb))
    torch.cuda.synchronize()
    return got, dA, dB


@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 37, 70), (1, 64, 64), (3, 129, 130),
                                   (2, 300, 65), (1, 1000, 256)])
@pytest.mark.parametrize("prange", [(-3.0, 3.0), (20.0, 30.0)])
def test_final_state_cotangent_parity(wkv, dev, B, T, C, prange):
    """L = sum(dy * y) + sum(dA A_T + dB B_T): every gradient against the oracle's direct
    backward plus the final state's terms (tests/state_ref.py, pinned by finite differences
    of the oracle)."""
    from state_ref import backward_state_grad_cot
    x = wkv_inputs.generate("l3b", seed=100 + B * T + C, B=B, T=T, C=C)
    st = wkv_inputs.random_state(B, C, seed=T + 2 * C, p_range=prange)
    got, dA, dB = _cot_case(wkv, dev, x, st, seed=T + C)
    ref = backward_state_grad_cot(x["w"], x["u"], x["k"], x["v"], x["dy"], st, dA, dB)
    floors = _floors(state_grad_scale(x["w"], x["u"], x["k"], x["v"], x["dy"], st, dA, dB))
    worst = 0.0
    for g, r, n in zip(got, ref, ("dk", "dv", "dw", "du", "da", "db", "dp")):
        r = np.asarray(r, np.float64)
        worst = max(worst, assert_wkv_close(g.cpu().numpy(), r, "%s B=%d T=%d C=%d p in %s"
                                            % (n, B, T, C, prange), floor=floors[n]))
    _log("final-state cotangent B=%d T=%d C=%d p in %s" % (B, T, C, prange), worst)


@pytest.mark.parametrize("cuts", [(0, 97, 300), (0, 64, 128, 300), (0, 1, 2, 300)])
def test_pieces_chain_to_the_whole_sequence(wkv, dev, cuts):
    """A sequence run forward in pieces (each from the state the last one left) and then
    backward from the last piece to the first, each piece's da, db handed to the one before
    as its final state's cotangent: the gradients of the whole sequence, from its initial
    state, against the oracle's direct backward of the whole."""
    import torch
    B, C = 2, 130
    T = cuts[-1]
    x = wkv_inputs.generate("l3b", seed=110 + len(cuts), B=B, T=T, C=C)
    st = wkv_inputs.random_state(B, C, seed=111, p_range=(-3.0, 3.0))
    t = {n: _t(dev, x[n]) for n in ("w", "u", "k", "v", "dy")}
    sg = [_t(dev, s) for s in st]
    pieces = []
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        sl = {n: t[n][:, t0:t1].contiguous() for n in ("k", "v", "dy")}
        ws = wkv.forward_workspace(B, t1 - t0, C, dev)
        wkv.forward_state(t["w"], t["u"], sl["k"], sl["v"], *sg, workspace=ws)
        pieces.append((sl, ws))
    grads = [None] * len(pieces)
    dstate = None
    for i in range(len(pieces) - 1, -1, -1):
        sl, ws = pieces[i]
        grads[i] = wkv.backward_state(t["w"], t["u"], sl["k"], sl["v"], sl["dy"], ws,
                                      dstate=dstate)
        dstate = (grads[i][4], grads[i][5])
    torch.cuda.synchronize()
    ref = backward_state_grad(x["w"], x["u"], x["k"], x["v"], x["dy"], st)
    floors = _floors(state_grad_scale(x["w"], x["u"], x["k"], x["v"], x["dy"], st))
    got = [torch.cat([g[0] for g in grads], dim=1), torch.cat([g[1] for g in grads], dim=1),
           sum(g[2].double() for g in grads), sum(g[3].double() for g in grads),
           grads[0][4], grads[0][5], grads[0][6]]
    worst = 0.0
    for g, r, n in zip(got, ref, ("dk", "dv", "dw", "du", "da", "db", "dp")):
        r = np.asarray(r, np.float64)
        worst = max(worst, assert_wkv_close(g.cpu().numpy(), r, "%s cuts=%s" % (n, cuts),
                                            floor=floors[n]))
    _log("pieces %s" % (cuts,), worst)


def test_final_state_cotangent_extreme_decay(wkv, dev):
    """w up to 200 with 28 padded tokens after T: the cotangent, placed at the last window's
    end, carries a growth of up to e^{28 * 200} there, which only the per-token path can
    hold (and a few channels with w ~ 1e-7, where it does not decay at all)."""
    from state_ref import backward_state_grad_cot
    B, T, C = 2, 100, 70
    rng = np.random.default_rng(120)
    w = np.exp(rng.uniform(-8.0, np.log(200.0), C)).astype(np.float32)
    w[:3] = 1e-7
    x = {"w": w, "u": rng.uniform(-1, 1, C).astype(np.float32),
         "k": rng.standard_normal((B, T, C)).astype(np.float32),
         "v": rng.standard_normal((B, T, C)).astype(np.float32),
         "dy": rng.standard_normal((B, T, C)).astype(np.float32)}
    st = wkv_inputs.random_state(B, C, seed=121, p_range=(-3.0, 3.0))
    got, dA, dB = _cot_case(wkv, dev, x, st, seed=122)
    ref = backward_state_grad_cot(x["w"], x["u"], x["k"], x["v"], x["dy"], st, dA, dB)
    floors = _floors(state_grad_scale(x["w"], x["u"], x["k"], x["v"], x["dy"], st, dA, dB))
    worst = 0.0
    for g, r, n in zip(got, ref, ("dk", "dv", "dw", "du", "da", "db", "dp")):
        r = np.asarray(r, np.float64)
        worst = max(worst, assert_wkv_close(g.cpu().numpy(), r, "%s extreme w" % n,
                                            floor=floors[n]))
    _log("final-state cotangent, w up to 200", worst)


def _sig(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


@pytest.mark.parametrize("dtype,gated", [("bfloat16", False), ("float16", False),
                                         ("float32", True), ("bfloat16", True)])
def test_typed_and_gated_state_pair(wkv, dev, dtype, gated):
    """forward_state / backward_state with 16-bit k, v, dy, r, y, dk, dv, dr and/or the
    receptance gate, a cotangent of the final state included. The oracle runs on the same
    values widened exactly; the gated reference is the plain one with the cotangent
    dy = dout sigma(r), plus dr = dout sigma(r) (1 - sigma(r)) y. 16-bit outputs get one unit
    in the format's last place on top of the fp32 tolerance."""
    import torch
    from oracle import forward_rescaled
    from helpers import assert_io_close
    from state_ref import backward_state_grad_cot
    tdt = getattr(torch, dtype)
    B, T, C = 2, 150, 70
    x = wkv_inputs.generate("l3b", seed=130, B=B, T=T, C=C)
    rng = np.random.default_rng(131)
    rr = rng.standard_normal((B, T, C)).astype(np.float32) * 2
    t = {n: _t(dev, x[n]).to(tdt) for n in ("k", "v", "dy")}
    t["r"] = _t(dev, rr).to(tdt) if gated else None
    for n in ("w", "u"):
        t[n] = _t(dev, x[n])
    wide = {n: t[n].float().cpu().numpy().astype(np.float64) for n in ("k", "v", "dy")}
    rw = t["r"].float().cpu().numpy().astype(np.float64) if gated else None
    st = wkv_inputs.random_state(B, C, seed=132, p_range=(-3.0, 3.0))
    sg = [_t(dev, s) for s in st]
    ws = wkv.forward_workspace(B, T, C, dev)
    out = wkv.forward_state(t["w"], t["u"], t["k"], t["v"], *sg, workspace=ws, r=t["r"])
    yo, (_, _, po) = forward_rescaled(x["w"], x["u"], wide["k"], wide["v"], st)
    ra = rng.standard_normal((B, C)) * 0.5
    rb = rng.standard_normal((B, C)) * 0.5
    dA, dB = ra * np.exp(-po), rb * np.exp(-po)
    pg = sg[2].cpu().numpy().astype(np.float64)
    dfa = _t(dev, (ra * np.exp(pg - po)).astype(np.float32))
    dfb = _t(dev, (rb * np.exp(pg - po)).astype(np.float32))
    got = wkv.backward_state(t["w"], t["u"], t["k"], t["v"], t["dy"], ws, dstate=(dfa, dfb),
                             r=t["r"])
    torch.cuda.synchronize()
    dyeff = wide["dy"] * _sig(rw) if gated else wide["dy"]
    ref = list(backward_state_grad_cot(x["w"], x["u"], wide["k"], wide["v"], dyeff, st, dA, dB))
    floors = _floors(state_grad_scale(x["w"], x["u"], wide["k"], wide["v"], dyeff, st, dA, dB))
    names = ["dk", "dv", "dw", "du", "da", "db", "dp"]
    yref = yo * _sig(rw) if gated else yo
    if gated:
        ref.insert(2, wide["dy"] * _sig(rw) * (1 - _sig(rw)) * yo)
        names.insert(2, "dr")
    ofl = out.float().cpu().numpy()
    worst = (assert_io_close(ofl, yref, dtype, "out") if dtype != "float32"
             else assert_wkv_close(ofl, yref, "out"))
    for g, r, n in zip(got, ref, names):
        g = g.float().cpu().numpy()
        r = np.asarray(r, np.float64)
        what = "%s %s gated=%s" % (n, dtype, gated)
        if n in ("dk", "dv", "dr") and dtype != "float32":
            worst = max(worst, assert_io_close(g, r, dtype, what))
        else:
            worst = max(worst, assert_wkv_close(g, r, what, floor=floors[n]))
    _log("%s gated=%s with cotangent" % (dtype, gated), worst)
