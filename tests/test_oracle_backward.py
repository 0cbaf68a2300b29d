"""Pins for the oracle's backward routines (CPU only).

The backward of L = sum_t dy_t y_t is pinned against central finite differences of the
direct forward, against torch autograd through the causal softmax form (a library
derivative, independent of the hand-derived gradient formulas), against hand-worked
values, and against exact identities that follow from invariances of the definition:

  * shift of every k by a constant leaves y unchanged      => sum_t dk_t = 0
  * y(alpha v + beta) = alpha y(v) + beta                  => sum_t dv_t = sum_t dy_t
  * k_i -> k_i + gamma i together with w -> w + gamma,
    u -> u + gamma moves every logit of y_t by the same     => sum_t t dk_t = dw + du
    amount gamma (t-1)                                         (per sequence)

Operator: "RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (8);
"RWKV についての調査記録", section "Trainingについて" (all parameters get gradients).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import wkv_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BACKWARDS = {"direct": oracle.backward_direct, "recurrent": oracle.backward_recurrent}


def _rand(B, T, C, seed, kscale=1.0, d=(-6.0, 1.0), urange=(-1.0, 1.0)):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(*d, size=C))
    u = rng.uniform(*urange, size=C)
    k = kscale * rng.standard_normal((B, T, C))
    v = rng.standard_normal((B, T, C))
    g = rng.standard_normal((B, T, C))
    return w, u, k, v, g


def _val(s):
    named = {"ln2": math.log(2.0), "ln4": math.log(4.0)}
    return named[s] if s in named else float(s)


@pytest.mark.parametrize("name", sorted(BACKWARDS))
def test_hand_worked_cases(name):
    with open(os.path.join(GOLDEN, "hand_backward.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        T = len(case["v"])
        w = np.array([_val(case["w"])])
        u = np.array([_val(case["u"])])
        k = np.array([_val(s) for s in case["k"]]).reshape(1, T, 1)
        v = np.array(case["v"], float).reshape(1, T, 1)
        g = np.array(case["dy"], float).reshape(1, T, 1)
        dk, dv, dw, du = BACKWARDS[name](w, u, k, v, g)
        np.testing.assert_allclose(dk[0, :, 0], case["dk"], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dv[0, :, 0], case["dv"], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dw[0], case["dw"], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(du[0], case["du"], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("name", sorted(BACKWARDS))
def test_finite_differences(name):
    B, T, C = 2, 6, 3
    w, u, k, v, g = _rand(B, T, C, 21, kscale=1.5)
    dk, dv, dw, du = BACKWARDS[name](w, u, k, v, g)

    def loss(w_, u_, k_, v_):
        return float(np.sum(g * oracle.forward_direct(w_, u_, k_, v_)))

    def central(x, fn):
        out = np.empty_like(x)
        flat = x.reshape(-1)
        for idx in range(flat.size):
            h = 1e-6 * max(1.0, abs(flat[idx]))
            keep = flat[idx]
            flat[idx] = keep + h
            lp = fn()
            flat[idx] = keep - h
            lm = fn()
            flat[idx] = keep
            out.reshape(-1)[idx] = (lp - lm) / (2 * h)
        return out

    kk, vv, ww, uu = k.copy(), v.copy(), w.copy(), u.copy()
    fk = central(kk, lambda: loss(w, u, kk, v))
    fv = central(vv, lambda: loss(w, u, k, vv))
    fw = central(ww, lambda: loss(ww, u, k, v))
    fu = central(uu, lambda: loss(w, uu, k, v))
    for got, ref in ((dk, fk), (dv, fv), (dw, fw), (du, fu)):
        np.testing.assert_allclose(got, ref, rtol=2e-7, atol=2e-8)


@pytest.mark.parametrize("name", sorted(BACKWARDS))
def test_torch_autograd_of_softmax_form(name):
    torch = pytest.importorskip("torch")
    B, T, C = 2, 23, 4
    w, u, k, v, g = _rand(B, T, C, 22, kscale=2.0, d=(-8.0, 2.0), urange=(-3, 3))
    tw = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    tu = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    t = torch.arange(T, dtype=torch.float64)[:, None]
    i = torch.arange(T, dtype=torch.float64)[None, :]
    age = (t - 1 - i)  # [T, T]
    kk = tk.permute(0, 2, 1)  # [B, C, T]
    logit = kk[:, :, None, :] - age[None, None] * tw[None, :, None, None]
    diag = (tu[None, :, None] + kk)  # [B, C, T]
    eye = torch.eye(T, dtype=torch.bool)
    logit = torch.where(eye, diag[..., None].expand(B, C, T, T), logit)
    logit = logit.masked_fill(i > t, float("-inf"))
    P = torch.softmax(logit, dim=-1)
    y = (P @ tv.permute(0, 2, 1)[..., None])[..., 0].permute(0, 2, 1)
    (y * torch.tensor(g)).sum().backward()
    dk, dv, dw, du = BACKWARDS[name](w, u, k, v, g)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(du, tu.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("name", sorted(BACKWARDS))
def test_invariance_identities(name):
    B, T, C = 3, 60, 5
    w, u, k, v, g = _rand(B, T, C, 23, kscale=2.0, d=(-8.0, 2.0), urange=(-3, 3))
    dk, dv, dw, du = BACKWARDS[name](w, u, k, v, g)
    scale = np.abs(dk).sum(axis=1)
    assert np.all(np.abs(dk.sum(axis=1)) <= 1e-12 * (1 + scale))
    np.testing.assert_allclose(dv.sum(axis=1), g.sum(axis=1), rtol=1e-11, atol=1e-12)
    tdk = (np.arange(T)[None, :, None] * dk).sum(axis=(0, 1))
    np.testing.assert_allclose(tdk, dw + du, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("name", sorted(BACKWARDS))
def test_one_hot_cotangent_gives_weight_row(name):
    B, T, C = 1, 15, 3
    w, u, k, v, _ = _rand(B, T, C, 24, kscale=2.0)
    for t in (0, 7, T - 1):
        g = np.zeros((B, T, C))
        g[:, t] = 1.0
        dk, dv, dw, du = BACKWARDS[name](w, u, k, v, g)
        assert np.all(dv[:, t + 1:] == 0.0)
        assert np.all(dv >= 0.0)
        np.testing.assert_allclose(dv.sum(axis=1), 1.0, rtol=1e-13)
        # the weight row reproduces the forward output at t
        y = oracle.forward_direct(w, u, k, v)
        np.testing.assert_allclose((dv * v).sum(axis=1), y[:, t], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("name", sorted(BACKWARDS))
def test_short_sequences(name):
    w, u, k, v, g = _rand(2, 2, 4, 25, kscale=3.0)
    dk, dv, dw, du = BACKWARDS[name](w, u, k, v, g)
    assert np.all(np.abs(dw) < 1e-15)  # no token is older than age 0 when T <= 2
    w, u, k, v, g = _rand(2, 1, 4, 26, kscale=3.0)
    dk, dv, dw, du = BACKWARDS[name](w, u, k, v, g)
    np.testing.assert_allclose(dv, g, rtol=1e-15)
    # y_0 = v_0 exactly in the definition; the recurrent form rounds cur*v/cur.
    tol = 1e-15 * np.abs(g).max()
    assert np.all(np.abs(dk) <= tol) and np.all(np.abs(du) <= tol) and np.all(dw == 0.0)


def test_direct_and_recurrent_agree():
    w, u, k, v, g = _rand(2, 200, 6, 27, kscale=3.0, d=(-8.0, 2.0), urange=(-3, 3))
    a = oracle.backward_direct(w, u, k, v, g)
    b = oracle.backward_recurrent(w, u, k, v, g)
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, x, rtol=1e-9, atol=1e-11)


def test_generated_workload_small():
    x = wkv_inputs.generate("small")
    a = oracle.backward_direct(x["w"], x["u"], x["k"], x["v"], x["dy"])
    b = oracle.backward_recurrent(x["w"], x["u"], x["k"], x["v"], x["dy"])
    for p, q in zip(a, b):
        np.testing.assert_allclose(q, p, rtol=1e-9, atol=1e-11)
        assert np.all(np.isfinite(p))
