"""GPU parity of wkv_forward_state against the fp64 oracle (marked gpu).

The prompt's tokens go through the layer one after another, each updating the state, and
generation continues from the state they leave ("RWKV についての調査記録", section
"コードを見ながらRWKVの構造を把握"). wkv_forward_state runs the prompt in parallel from a
given state and leaves the final state; the oracle is forward_rescaled from the same state
(pinned against the direct form in test_oracle_state.py). y is compared with the usual
tolerance; states through what is unique about them, the ratio a/b and the log-mass
p + ln b (decode's convention: (a e^d, b e^d, p - d) is the same state).
"""
import numpy as np
import pytest

import oracle
import wkv_inputs
from helpers import assert_wkv_close
from state_ref import backward_with_state

pytestmark = pytest.mark.gpu


def _t(dev, a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _run(wkv, dev, x, state, ws=None):
    """GPU forward_state: returns y and the final state (numpy), and the workspace."""
    import torch
    t = {n: _t(dev, x[n]) for n in ("w", "u", "k", "v")}
    st = [_t(dev, s) for s in state]
    B, T, C = x["k"].shape
    if ws is None:
        ws = wkv.forward_workspace(B, T, C, dev)
    y = wkv.forward_state(t["w"], t["u"], t["k"], t["v"], *st, workspace=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), tuple(s.cpu().numpy() for s in st), ws


def _check_state(got, ref, what):
    ga, gb, gp = (np.asarray(s, np.float64) for s in got)
    ra, rb, rp = (np.asarray(s, np.float64) for s in ref)
    assert np.all(np.isfinite(ga)) and np.all(gb > 0), what
    v = assert_wkv_close(ga / gb, ra / rb, what + " a/b")
    np.testing.assert_allclose(gp + np.log(gb), rp + np.log(rb), rtol=0, atol=1e-4,
                               err_msg=what + " log-mass")
    return v


def _log(name, v):
    print("[forward_state] %s max_violation=%.3g" % (name, v), flush=True)


@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 37, 70), (3, 300, 130), (1, 257, 64),
                                   (2, 513, 65), (4, 31, 200), (2, 1000, 256)])
@pytest.mark.parametrize("prange", [(-4.0, 4.0), (20.0, 30.0), (-30.0, -20.0)])
def test_parity_from_a_state(wkv, dev, B, T, C, prange):
    """States around the keys' scale, far above it (the state dominates for a while) and
    far below it (it hardly counts)."""
    x = wkv_inputs.generate("l3b", seed=31 + B * T + C, B=B, T=T, C=C, with_dy=False)
    st = wkv_inputs.random_state(B, C, seed=B + T + C, p_range=prange)
    y, fin, _ = _run(wkv, dev, x, st)
    ry, rfin = oracle.forward_rescaled(x["w"], x["u"], x["k"], x["v"], st)
    v = assert_wkv_close(y, ry, "y B=%d T=%d C=%d" % (B, T, C))
    v = max(v, _check_state(fin, rfin, "state B=%d T=%d C=%d" % (B, T, C)))
    _log("B=%d T=%d C=%d p in %s" % (B, T, C, prange), v)


def test_empty_state_matches_forward_bitwise(wkv, dev):
    import torch
    x = wkv_inputs.generate("l3b", seed=41, B=3, T=700, C=200, with_dy=False)
    y_state, fin, _ = _run(wkv, dev, x, wkv_inputs.empty_decode_state(3, 200))
    t = {n: _t(dev, x[n]) for n in ("w", "u", "k", "v")}
    y = wkv.forward(t["w"], t["u"], t["k"], t["v"])
    torch.cuda.synchronize()
    assert np.array_equal(y_state, y.cpu().numpy())
    _, rfin = oracle.forward_rescaled(x["w"], x["u"], x["k"], x["v"])
    _check_state(fin, rfin, "final state")
    # p = -inf is the empty state too
    st = wkv_inputs.empty_decode_state(3, 200)
    y_inf, _, _ = _run(wkv, dev, x, (st[0], st[1], np.full_like(st[2], -np.inf)))
    assert np.array_equal(y_inf, y_state)


def test_prompt_in_pieces_then_decode(wkv, dev):
    """Prefill in three calls of different lengths, then 20 decode steps: every output
    equals the direct form over the whole sequence."""
    import torch
    B, C, T = 2, 130, 400
    x = wkv_inputs.generate("l3b", seed=42, B=B, T=T, C=C, with_dy=False)
    ref = oracle.forward_direct(x["w"], x["u"], x["k"], x["v"])
    w, u = _t(dev, x["w"]), _t(dev, x["u"])
    a, b, p = (_t(dev, s) for s in wkv_inputs.empty_decode_state(B, C))
    cuts = [0, 1, 97, 380]
    worst = 0.0
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        y = wkv.forward_state(w, u, _t(dev, x["k"][:, t0:t1]), _t(dev, x["v"][:, t0:t1]), a, b, p)
        torch.cuda.synchronize()
        worst = max(worst, assert_wkv_close(y.cpu().numpy(), ref[:, t0:t1], "prefill %d:%d" % (t0, t1)))
    for t in range(cuts[-1], T):
        y = wkv.decode_step(w, u, _t(dev, x["k"][:, t]), _t(dev, x["v"][:, t]), a, b, p)
        torch.cuda.synchronize()
        worst = max(worst, assert_wkv_close(y.cpu().numpy(), ref[:, t], "decode t=%d" % t))
    _log("pieces then decode", worst)


def test_zero_length_keeps_the_state(wkv, dev):
    import torch
    x = wkv_inputs.generate("l3b", seed=43, B=2, T=0, C=65, with_dy=False)
    st = wkv_inputs.random_state(2, 65, seed=5)
    y, fin, _ = _run(wkv, dev, x, st)
    assert y.shape == (2, 0, 65)
    for g, r in zip(fin, st):
        assert np.array_equal(g, r)


@pytest.mark.parametrize("B,T,C", [(2, 37, 70), (1, 300, 64), (3, 129, 130)])
def test_backward_after_a_state_forward(wkv, dev, B, T, C):
    """wkv_backward given the workspace of a state forward: gradients with the initial
    state held constant (the direct backward with the state's token prepended)."""
    import torch
    x = wkv_inputs.generate("l3b", seed=44 + T, B=B, T=T, C=C)
    st = wkv_inputs.random_state(B, C, seed=T, p_range=(-3.0, 3.0))
    _, _, ws = _run(wkv, dev, x, st)
    t = {n: _t(dev, x[n]) for n in ("w", "u", "k", "v", "dy")}
    got = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=ws)
    torch.cuda.synchronize()
    ref = backward_with_state(x["w"], x["u"], x["k"], x["v"], x["dy"], st)
    worst = 0.0
    for g, r, n in zip(got, ref, ("dk", "dv", "dw", "du")):
        worst = max(worst, assert_wkv_close(g.cpu().numpy(), r, "%s B=%d T=%d C=%d" % (n, B, T, C)))
    _log("backward B=%d T=%d C=%d" % (B, T, C), worst)


def test_full_layer_from_a_state(wkv, dev):
    """The 3B-class layer shape, started from a random state."""
    x = wkv_inputs.generate("l3b", with_dy=False)
    B, T, C = x["k"].shape
    st = wkv_inputs.random_state(B, C, seed=45)
    y, fin, _ = _run(wkv, dev, x, st)
    ry, rfin = oracle.forward_rescaled(x["w"], x["u"], x["k"], x["v"], st)
    v = assert_wkv_close(y, ry, "l3b y")
    v = max(v, _check_state(fin, rfin, "l3b state"))
    _log("l3b", v)
