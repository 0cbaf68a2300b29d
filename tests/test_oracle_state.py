"""Pins for the oracle's forward from a given state (CPU only).

Prompt tokens pass through the layer one after another, each updating the state, and the
next token is then predicted from that state ("RWKV についての調査記録", section
"コードを見ながらRWKVの構造を把握"; the state is what inference carries from token to
token, same page, section "RWKVとは？"). The oracle's forward_rescaled with a given state is
that computation. It is pinned here against the direct O(T^2) definition through a
construction the definition itself fixes: the state (a, b, p) before token 0 holds
A = a e^p and B = b e^p, which decay by e^{-t w} by token t, exactly as the contribution
of one extra token placed just before the sequence with key p + ln b and value a / b
(its weight e^{-(t-1-(-1)) w + k} = e^{-t w} b e^p). So the state-in forward equals the
direct forward of the sequence with that token prepended, dropping its output.
"""
import numpy as np
import pytest

import oracle
from state_ref import (backward_state_grad, backward_state_grad_cot, backward_with_state,
                       prepend_state_token as _prepend)


def _rand(B, T, C, seed, kscale=1.0):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-6.0, 1.5, size=C))
    u = rng.uniform(-1.0, 1.0, size=C)
    k = kscale * rng.standard_normal((B, T, C))
    v = rng.standard_normal((B, T, C))
    return rng, w, u, k, v


def _state(rng, B, C):
    b = rng.uniform(0.5, 8.0, size=(B, C))
    a = b * rng.standard_normal((B, C))
    p = rng.uniform(-4.0, 4.0, size=(B, C))
    return a, b, p


@pytest.mark.parametrize("T", [1, 2, 17])
def test_state_forward_equals_direct_with_prepended_token(T):
    rng, w, u, k, v = _rand(3, T, 5, 40 + T, kscale=2.0)
    st = _state(rng, 3, 5)
    y, _ = oracle.forward_rescaled(w, u, k, v, st)
    kk, vv = _prepend(st, k, v)
    ref = oracle.forward_direct(w, u, kk, vv)[:, 1:]
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-13)


def test_first_output_from_a_state_closed_form():
    # y_0 = (a e^p + e^{u+k_0} v_0) / (b e^p + e^{u+k_0}), whatever w is
    rng, w, u, k, v = _rand(2, 1, 4, 45)
    a, b, p = _state(rng, 2, 4)
    y, _ = oracle.forward_rescaled(w, u, k, v, (a, b, p))
    e = np.exp(u + k[:, 0] - p)
    np.testing.assert_allclose(y[:, 0], (a + e * v[:, 0]) / (b + e), rtol=1e-13)


def test_final_state_predicts_the_next_token():
    # the state after the last token, advanced by one more token, gives that token's output
    # of the direct form over the whole sequence (prepended state token included)
    rng, w, u, k, v = _rand(2, 23, 6, 46, kscale=2.0)
    st = _state(rng, 2, 6)
    _, fin = oracle.forward_rescaled(w, u, k[:, :22], v[:, :22], st)
    y_next, _ = oracle.decode_step(w, u, k[:, 22], v[:, 22], fin)
    kk, vv = _prepend(st, k, v)
    ref = oracle.forward_direct(w, u, kk, vv)[:, -1]
    np.testing.assert_allclose(y_next, ref, rtol=1e-11, atol=1e-13)


def test_empty_state_is_the_plain_forward():
    _, w, u, k, v = _rand(2, 30, 4, 47, kscale=3.0)
    empty = (np.zeros((2, 4)), np.zeros((2, 4)), np.full((2, 4), -1e38))
    y, _ = oracle.forward_rescaled(w, u, k, v, empty)
    np.testing.assert_allclose(y, oracle.forward_direct(w, u, k, v), rtol=1e-11, atol=1e-13)


def test_backward_with_state_finite_differences():
    rng, w, u, k, v = _rand(2, 5, 3, 48, kscale=1.5)
    st = _state(rng, 2, 3)
    dy = rng.standard_normal(k.shape)
    got = backward_with_state(w, u, k, v, dy, st)

    def loss(w_, u_, k_, v_):
        return float(np.sum(dy * oracle.forward_rescaled(w_, u_, k_, v_, st)[0]))

    args = [w, u, k, v]
    names = ["w", "u", "k", "v"]
    grads = {"k": got[0], "v": got[1], "w": got[2], "u": got[3]}
    for i, name in enumerate(names):
        x = args[i]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-6 * max(1.0, abs(x[idx]))
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = list(args)
            am = list(args)
            ap[i], am[i] = xp, xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        np.testing.assert_allclose(grads[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("T", [1, 6])
def test_state_gradient_finite_differences(T):
    # da, db, dp of L = sum(dy * y) against central differences of the state-in forward
    rng, w, u, k, v = _rand(2, T, 3, 50 + T, kscale=1.5)
    st = _state(rng, 2, 3)
    dy = rng.standard_normal(k.shape)
    got = backward_state_grad(w, u, k, v, dy, st)
    base = backward_with_state(w, u, k, v, dy, st)
    for g, r in zip(got[:4], base):
        np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-14)

    def loss(s_):
        return float(np.sum(dy * oracle.forward_rescaled(w, u, k, v, s_)[0]))

    for i, name in enumerate(("a", "b", "p")):
        x = st[i]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-6 * max(1.0, abs(x[idx]))
            sp, sm = [s_.copy() for s_ in st], [s_.copy() for s_ in st]
            sp[i][idx] += h
            sm[i][idx] -= h
            fd[idx] = (loss(sp) - loss(sm)) / (2 * h)
        np.testing.assert_allclose(got[4 + i], fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_state_gradient_closed_form_single_token():
    # T = 1: y_0 = (A + e^{u+k} v) / (B + e^{u+k}) with A = a e^p, B = b e^p, so
    # dL/dA = dy / D and dL/dB = -dy y / D, D = B + e^{u+k}
    rng, w, u, k, v = _rand(2, 1, 4, 55)
    a, b, p = _state(rng, 2, 4)
    dy = rng.standard_normal(k.shape)
    got = backward_state_grad(w, u, k, v, dy, (a, b, p))
    ep = np.exp(p)
    e = np.exp(u + k[:, 0])
    D = b * ep + e
    y = (a * ep + e * v[:, 0]) / D
    g, hh = dy[:, 0] / D, dy[:, 0] * y / D
    np.testing.assert_allclose(got[4], g * ep, rtol=1e-12)
    np.testing.assert_allclose(got[5], -hh * ep, rtol=1e-12)
    np.testing.assert_allclose(got[6], (a * g - b * hh) * ep, rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("T", [1, 5])
def test_final_state_cotangent_finite_differences(T):
    # L = sum(dy * y) + sum(dA A_T + dB B_T), (A_T, B_T) = (a_T e^{p_T}, b_T e^{p_T}) the
    # oracle's final state: every gradient against central differences of the oracle
    rng, w, u, k, v = _rand(2, T, 3, 60 + T, kscale=1.5)
    st = _state(rng, 2, 3)
    dy = rng.standard_normal(k.shape)
    dA = rng.standard_normal((2, 3)) * 0.3
    dB = rng.standard_normal((2, 3)) * 0.3
    got = backward_state_grad_cot(w, u, k, v, dy, st, dA, dB)

    def loss(w_, u_, k_, v_, s_):
        y, (a, b, p) = oracle.forward_rescaled(w_, u_, k_, v_, s_)
        return float(np.sum(dy * y) + np.sum(dA * a * np.exp(p) + dB * b * np.exp(p)))

    args = [w, u, k, v, list(st)]
    # (argument, state field, index in got): w, u, k, v, then a, b, p
    flat = [(0, None, 2), (1, None, 3), (2, None, 0), (3, None, 1), (4, 0, 4), (4, 1, 5),
            (4, 2, 6)]
    for i, j, slot in flat:
        x = args[i] if j is None else args[4][j]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-6 * max(1.0, abs(x[idx]))
            vals = []
            for sgn in (1.0, -1.0):
                xx = x.copy()
                xx[idx] += sgn * h
                aa = [a_ if not isinstance(a_, list) else list(a_) for a_ in args]
                if j is None:
                    aa[i] = xx
                else:
                    aa[4][j] = xx
                vals.append(loss(aa[0], aa[1], aa[2], aa[3], tuple(aa[4])))
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        np.testing.assert_allclose(got[slot], fd, rtol=1e-6, atol=1e-8,
                                   err_msg="slot %d" % slot)


def test_final_state_cotangent_chains_two_pieces():
    # the gradient of a sequence run in two pieces: the second piece's state gradient
    # (da, db at its start) is the cotangent of the first piece's final state
    rng, w, u, k, v = _rand(2, 11, 3, 70, kscale=1.5)
    st = _state(rng, 2, 3)
    dy = rng.standard_normal(k.shape)
    whole = backward_state_grad(w, u, k, v, dy, st)
    T1 = 4
    _, mid = oracle.forward_rescaled(w, u, k[:, :T1], v[:, :T1], st)
    g2 = backward_state_grad(w, u, k[:, T1:], v[:, T1:], dy[:, T1:], mid)
    a1, b1, p1 = mid
    dA, dB = g2[4] * np.exp(-p1), g2[5] * np.exp(-p1)
    g1 = backward_state_grad_cot(w, u, k[:, :T1], v[:, :T1], dy[:, :T1], st, dA, dB)
    np.testing.assert_allclose(np.concatenate([g1[0], g2[0]], axis=1), whole[0], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([g1[1], g2[1]], axis=1), whole[1], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(g1[2] + g2[2], whole[2], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(g1[3] + g2[3], whole[3], rtol=1e-9, atol=1e-12)
    for i in (4, 5, 6):
        np.testing.assert_allclose(g1[i], whole[i], rtol=1e-9, atol=1e-12)


def _explicit_state_token_terms(w, u, k, v, dy, state):
    """Brute force in numpy for tiny shapes: the softmax weight P_t0 of the prepended state
    token in every later output t, and sum_t |g_t| P_t0, sum_t |g_t| P_t0 |v0 - y_t|."""
    kk, vv = _prepend(state, k, v)
    B, T1, C = kk.shape
    dv_abs = np.zeros((B, C))
    dk_abs = np.zeros((B, C))
    for b in range(B):
        for c in range(C):
            for t in range(1, T1):
                logit = np.array([-(t - 1 - i) * w[c] + kk[b, i, c] for i in range(t)]
                                 + [u[c] + kk[b, t, c]])
                P = np.exp(logit - logit.max())
                P /= P.sum()
                y = float(P @ vv[b, :t + 1, c])
                g = abs(dy[b, t - 1, c])
                dv_abs[b, c] += g * P[0]
                dk_abs[b, c] += g * P[0] * abs(vv[b, 0, c] - y)
    return dv_abs, dk_abs


@pytest.mark.parametrize("T", [1, 3, 12])
def test_state_token_abs_terms_by_brute_force(T):
    """The conditioning the GPU state-gradient tests are judged against is the sum of the
    absolute terms of dv0 and dk0; it is checked here against the terms written out."""
    from state_ref import state_token_abs_terms
    rng, w, u, k, v = _rand(2, T, 4, 70 + T, kscale=1.5)
    st = _state(rng, 2, 4)
    dy = rng.standard_normal((2, T, 4))
    got = state_token_abs_terms(w, u, k, v, dy, st)
    want = _explicit_state_token_terms(w, u, k, v, dy, st)
    for g, r in zip(got, want):
        np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("T", [1, 9, 40])
def test_state_grad_scale_bounds_the_gradients(T):
    """Each of |da|, |db|, |dp| is at most its scale (a sum of absolute terms), with and
    without a cotangent of the final state, and the scale is not needlessly loose: for a
    one-signed cotangent dy > 0, dv0 has no cancellation and |da| equals its scale."""
    from state_ref import state_grad_scale
    rng, w, u, k, v = _rand(3, T, 5, 80 + T)
    st = _state(rng, 3, 5)
    dy = rng.standard_normal((3, T, 5))
    dA = rng.standard_normal((3, 5))
    dB = rng.standard_normal((3, 5))
    for cot in (False, True):
        ref = (backward_state_grad_cot(w, u, k, v, dy, st, dA, dB) if cot
               else backward_state_grad(w, u, k, v, dy, st))
        sc = state_grad_scale(w, u, k, v, dy, st, *((dA, dB) if cot else ()))
        for r, s in zip(ref[4:], sc):
            assert np.all(np.abs(r) <= s * (1 + 1e-12))
    dyp = np.abs(dy)
    ref = backward_state_grad(w, u, k, v, dyp, st)
    sc = state_grad_scale(w, u, k, v, dyp, st)
    np.testing.assert_allclose(np.abs(ref[4]), sc[0], rtol=1e-12)
