"""Pins for the oracle's forward routines (CPU only).

Each test fixes the oracle against something other than itself: hand-worked values,
closed forms, invariants of the definition, or a textbook routine. Together they are
chosen so that a plausible slip (a dropped bonus term, a decay offset of t-i instead of
t-1-i, a wrong sign of w, a transposed index) fails at least one of them.

Operator: "RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (8) and its
recursive form; "RWKV についての調査記録", section 【wkvとは】.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import wkv_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FORWARDS = {
    "direct": oracle.forward_direct,
    "recurrent": oracle.forward_recurrent,
    "rescaled": lambda w, u, k, v: oracle.forward_rescaled(w, u, k, v)[0],
}


def _rand(B, T, C, seed, kscale=1.0, d=(-6.0, 1.0), urange=(-1.0, 1.0)):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(*d, size=C))
    u = rng.uniform(*urange, size=C)
    k = kscale * rng.standard_normal((B, T, C))
    v = rng.standard_normal((B, T, C))
    return w, u, k, v


def _val(s):
    named = {"ln2": math.log(2.0), "ln4": math.log(4.0)}
    return named[s] if s in named else float(s)


@pytest.mark.parametrize("name", sorted(FORWARDS))
def test_hand_worked_cases(name):
    with open(os.path.join(GOLDEN, "hand_forward.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        T = len(case["v"])
        w = np.array([_val(case["w"])])
        u = np.array([_val(case["u"])])
        k = np.array([_val(s) for s in case["k"]]).reshape(1, T, 1)
        v = np.array(case["v"], float).reshape(1, T, 1)
        y = FORWARDS[name](w, u, k, v)[0, :, 0]
        np.testing.assert_allclose(y, case["y"], rtol=1e-13, atol=1e-14, err_msg=case["name"])


@pytest.mark.parametrize("name", sorted(FORWARDS))
def test_single_token_is_v(name):
    w, u, k, v = _rand(3, 1, 5, 1, kscale=5.0)
    np.testing.assert_allclose(FORWARDS[name](w, u, k, v), v, rtol=1e-14, atol=0)


@pytest.mark.parametrize("name", sorted(FORWARDS))
def test_first_two_positions_closed_form(name):
    # y_0 = v_0; y_1 = (e^{k0} v0 + e^{u+k1} v1) / (e^{k0} + e^{u+k1}), independent of w
    # (the most recent past token is not decayed).
    w, u, k, v = _rand(2, 7, 6, 2, kscale=2.0)
    y = FORWARDS[name](w, u, k, v)
    np.testing.assert_allclose(y[:, 0], v[:, 0], rtol=1e-14)
    a = np.exp(k[:, 0])
    b = np.exp(u + k[:, 1])
    np.testing.assert_allclose(y[:, 1], (a * v[:, 0] + b * v[:, 1]) / (a + b), rtol=1e-13)
    y2 = FORWARDS[name](w * 3.0 + 1.0, u, k, v)
    np.testing.assert_allclose(y2[:, 1], y[:, 1], rtol=1e-13)


@pytest.mark.parametrize("name", sorted(FORWARDS))
def test_zero_parameters_give_prefix_mean(name):
    # w = u = k = 0: every token has weight 1, y_t = mean(v_0..v_t).
    B, T, C = 2, 40, 3
    v = np.random.default_rng(3).standard_normal((B, T, C))
    y = FORWARDS[name](np.zeros(C), np.zeros(C), np.zeros((B, T, C)), v)
    ref = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("name", sorted(FORWARDS))
def test_geometric_denominator(name):
    # k = 0, v = (1, 0, 0, ...): the numerator is e^{-(t-1)w} and the denominator is the
    # geometric sum (1 - e^{-tw}) / (1 - e^{-w}) + e^u, for t >= 1.
    T, C = 30, 4
    w = np.array([0.05, 0.3, 1.0, 2.5])
    u = np.array([-0.5, 0.0, 0.7, 1.3])
    v = np.zeros((1, T, C))
    v[0, 0] = 1.0
    y = FORWARDS[name](w, u, np.zeros((1, T, C)), v)[0]
    t = np.arange(1, T)[:, None]
    ref = np.exp(-(t - 1) * w) / ((1 - np.exp(-t * w)) / (1 - np.exp(-w)) + np.exp(u))
    np.testing.assert_allclose(y[1:], ref, rtol=1e-12)
    assert np.all(y[0] == 1.0)


@pytest.mark.parametrize("name", sorted(FORWARDS))
def test_fast_decay_keeps_two_terms(name):
    # w = 200: tokens older than t-1 carry weight <= e^{-200}; y_t is the two-term average.
    w, u, k, v = _rand(2, 9, 5, 4)
    w = np.full(5, 200.0)
    y = FORWARDS[name](w, u, k, v)
    a = np.exp(k[:, :-1])
    b = np.exp(u + k[:, 1:])
    np.testing.assert_allclose(y[:, 1:], (a * v[:, :-1] + b * v[:, 1:]) / (a + b), rtol=1e-12)


@pytest.mark.parametrize("name", sorted(FORWARDS))
def test_large_bonus_limits(name):
    w, u, k, v = _rand(2, 12, 4, 5)
    y = FORWARDS[name](w, np.full(4, 200.0), k, v)
    np.testing.assert_allclose(y, v, rtol=1e-12, atol=1e-14)
    y = FORWARDS[name](w, np.full(4, -200.0), k, v)
    # u -> -inf: the current token drops out, y_t is the decayed average of the past.
    num = np.zeros_like(v[:, 0])
    den = np.zeros_like(v[:, 0])
    for t in range(1, 12):
        num = np.exp(-w) * num + np.exp(k[:, t - 1]) * v[:, t - 1]
        den = np.exp(-w) * den + np.exp(k[:, t - 1])
        np.testing.assert_allclose(y[:, t], num / den, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y[:, 0], v[:, 0], rtol=1e-14)


@pytest.mark.parametrize("name", sorted(FORWARDS))
def test_key_shift_invariance(name):
    # Adding a constant to every k (of one channel) scales all weights alike.
    w, u, k, v = _rand(2, 25, 4, 6, kscale=3.0)
    y0 = FORWARDS[name](w, u, k, v)
    y1 = FORWARDS[name](w, u, k + np.array([3.7, -11.0, 0.25, 40.0]), v)
    np.testing.assert_allclose(y1, y0, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("name", sorted(FORWARDS))
def test_affine_equivariance_and_convexity(name):
    w, u, k, v = _rand(2, 50, 5, 7, kscale=2.0)
    y = FORWARDS[name](w, u, k, v)
    alpha, beta = -2.5, 0.75
    np.testing.assert_allclose(FORWARDS[name](w, u, k, alpha * v + beta), alpha * y + beta,
                               rtol=1e-12, atol=1e-12)
    lo = np.minimum.accumulate(v, axis=1)
    hi = np.maximum.accumulate(v, axis=1)
    assert np.all(y >= lo - 1e-12) and np.all(y <= hi + 1e-12)


@pytest.mark.parametrize("name", sorted(FORWARDS))
def test_causality_and_independence(name):
    w, u, k, v = _rand(3, 20, 6, 8)
    y = FORWARDS[name](w, u, k, v)
    s = 11
    k2, v2 = k.copy(), v.copy()
    k2[:, s] += 5.0
    v2[:, s] -= 3.0
    y2 = FORWARDS[name](w, u, k2, v2)
    assert np.array_equal(y2[:, :s], y[:, :s])
    assert not np.allclose(y2[:, s:], y[:, s:])
    perm = np.array([3, 0, 5, 1, 4, 2])
    yp = FORWARDS[name](w[perm], u[perm], k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(yp, y[:, :, perm], rtol=1e-15, atol=0)
    y1 = FORWARDS[name](w, u, k[1:2], v[1:2])
    np.testing.assert_allclose(y1, y[1:2], rtol=1e-15, atol=0)


def test_three_forms_agree():
    w, u, k, v = _rand(2, 300, 8, 9, kscale=3.0, d=(-8.0, 2.0), urange=(-3, 3))
    yd = oracle.forward_direct(w, u, k, v)
    yr = oracle.forward_recurrent(w, u, k, v)
    ys, _ = oracle.forward_rescaled(w, u, k, v)
    np.testing.assert_allclose(yr, yd, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(ys, yd, rtol=1e-11, atol=1e-13)


def test_large_keys_stay_finite_and_agree():
    # |k| in the hundreds and thousands: the plain recursion refuses, the direct and
    # rescaled forms stay finite, agree, and keep the convex-combination bounds.
    w, u, k, v = _rand(2, 80, 5, 10)
    k = k * 400.0
    k[0, 5, 0] = 1000.0
    k[1, 7, 3] = -1000.0
    with pytest.raises(OverflowError):
        oracle.forward_recurrent(w, u, k, v)
    yd = oracle.forward_direct(w, u, k, v)
    ys, _ = oracle.forward_rescaled(w, u, k, v)
    assert np.all(np.isfinite(yd)) and np.all(np.isfinite(ys))
    np.testing.assert_allclose(ys, yd, rtol=1e-9, atol=1e-12)
    lo = np.minimum.accumulate(v, axis=1)
    hi = np.maximum.accumulate(v, axis=1)
    assert np.all(yd >= lo - 1e-12) and np.all(yd <= hi + 1e-12)


def test_softmax_library_routine():
    # The definition as a causal-masked softmax, evaluated with scipy's softmax.
    from scipy.special import softmax
    w, u, k, v = _rand(2, 17, 3, 11, kscale=2.0)
    y = oracle.forward_direct(w, u, k, v)
    B, T, C = k.shape
    t = np.arange(T)[:, None]
    i = np.arange(T)[None, :]
    for b in range(B):
        for c in range(C):
            logit = np.where(i < t, k[b, None, :, c] - (t - 1 - i) * w[c], -np.inf)
            logit[np.arange(T), np.arange(T)] = u[c] + k[b, :, c]
            P = softmax(logit, axis=1)
            np.testing.assert_allclose(y[b, :, c], P @ v[b, :, c], rtol=1e-12, atol=1e-14)


def test_generated_workload_small():
    x = wkv_inputs.generate("small")
    yd = oracle.forward_direct(x["w"], x["u"], x["k"], x["v"])
    yr = oracle.forward_recurrent(x["w"], x["u"], x["k"], x["v"])
    np.testing.assert_allclose(yr, yd, rtol=1e-11, atol=1e-13)
    assert np.all(np.isfinite(yd))
