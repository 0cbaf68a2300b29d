"""References for the forward from a given state, built from oracle routines only.

A state (a, b, p) before token 0 holds A = a e^p and B = b e^p, which decay by e^{-t w}
by token t: exactly the contribution of one extra token placed just before the sequence
with key p + ln b and value a / b. tests/test_oracle_state.py pins this construction
against the oracle's recurrence and against finite differences.
"""
import numpy as np

import oracle


def prepend_state_token(state, k, v):
    """k, v [B, T, C] with the state's token (key p + ln b, value a / b) in front."""
    a, b, p = (np.asarray(s, np.float64) for s in state)
    k0 = (p + np.log(b))[:, None, :]
    v0 = (a / b)[:, None, :]
    return (np.concatenate([k0, np.asarray(k, np.float64)], axis=1),
            np.concatenate([v0, np.asarray(v, np.float64)], axis=1))


def backward_with_state(w, u, k, v, dy, state):
    """(dk, dv, dw, du) of L = sum(dy * y) for the forward from `state`, the state held
    constant: the direct backward of the sequence with the state's token prepended, that
    token's output given no weight and its own dk, dv dropped."""
    kk, vv = prepend_state_token(state, k, v)
    dy = np.asarray(dy, np.float64)
    g = np.concatenate([np.zeros_like(dy[:, :1]), dy], axis=1)
    dk, dv, dw, du = oracle.backward_direct(w, u, kk, vv, g)
    return dk[:, 1:], dv[:, 1:], dw, du


def backward_state_grad(w, u, k, v, dy, state):
    """backward_with_state plus (da, db, dp), the gradient of L with respect to the state
    (b > 0): through the prepended token, k0 = p + ln b and v0 = a / b, so with that token's
    own dk0, dv0: da = dv0 / b, db = dk0 / b - dv0 a / b^2, dp = dk0."""
    a, b, p = (np.asarray(s, np.float64) for s in state)
    kk, vv = prepend_state_token(state, k, v)
    dy = np.asarray(dy, np.float64)
    g = np.concatenate([np.zeros_like(dy[:, :1]), dy], axis=1)
    dk, dv, dw, du = oracle.backward_direct(w, u, kk, vv, g)
    dk0, dv0 = dk[:, 0], dv[:, 0]
    return (dk[:, 1:], dv[:, 1:], dw, du, dv0 / b, dk0 / b - dv0 * a / (b * b), dk0)


def state_token_abs_terms(w, u, k, v, dy, state):
    """The sums of the absolute values of the terms of the prepended state token's dv0 and
    dk0: dv0 = sum_t g_t P_t0 with P_t0 >= 0, so |g| in place of g gives sum_t |g_t| P_t0;
    dk0 = sum_t g_t P_t0 (v0 - y_t), so g_t sign(v0 - y_t) in place of g gives
    sum_t |g_t| P_t0 |v0 - y_t| (y of the sequence with the token prepended)."""
    kk, vv = prepend_state_token(state, k, v)
    dy = np.asarray(dy, np.float64)
    g = np.abs(np.concatenate([np.zeros_like(dy[:, :1]), dy], axis=1))
    y = oracle.forward_direct(w, u, kk, vv)
    _, dv_abs, _, _ = oracle.backward_direct(w, u, kk, vv, g)
    dk_abs, _, _, _ = oracle.backward_direct(w, u, kk, vv, g * np.sign(vv[:, :1] - y))
    return dv_abs[:, 0], dk_abs[:, 0]


def state_grad_scale(w, u, k, v, dy, state, dA=None, dB=None):
    """The conditioning of (da, db, dp): for da and db the sum of the absolute values of the
    terms that make them up (through da = dv0 / b, db = dk0 / b - dv0 a / b^2, and with a
    cotangent (dA, dB) of the final state the terms final_state_terms adds); for dp, which
    is a da + b db (the state's gradient along its own scale), |a| times da's plus |b| times
    db's. An entry is computed to 1e-4 of its scale when its error is below 1e-4 of it; |entry|
    never exceeds it."""
    a, b, p = (np.asarray(s, np.float64) for s in state)
    dv0, dk0 = state_token_abs_terms(w, u, k, v, dy, state)
    sa = dv0 / b
    sb = dk0 / b + dv0 * np.abs(a) / (b * b)
    if dA is not None:
        *_, xa, xb, _ = final_state_terms(w, u, k, v, state, dA, dB)
        sa = sa + np.abs(xa)
        sb = sb + np.abs(xb)
    return sa, sb, np.abs(a) * sa + np.abs(b) * sb


def final_state_terms(w, u, k, v, state, dA, dB):
    """The gradients of sum_{b,c} (dA A_T + dB B_T), (A_T, B_T) the state after the last
    token, in the order (dk, dv, dw, du, da, db, dp). From the recursion unrolled: A_T =
    sum_i e^{k_i - (T-1-i) w} v_i + e^{-T w} A_0 with A_0 = a e^p (B alike, without v).
    dA, dB [B, C] may be tiny and k large: every product is formed as one exponential of a
    sum of logs."""
    w = np.asarray(w, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    a, b, p = (np.asarray(s, np.float64) for s in state)
    dA = np.asarray(dA, np.float64)
    dB = np.asarray(dB, np.float64)
    T = k.shape[1]
    age = (T - 1 - np.arange(T, dtype=np.float64))[None, :, None]
    x = k - age * w[None, None, :]
    lA = np.log(np.abs(dA))[:, None, :]
    lB = np.log(np.abs(dB))[:, None, :]
    cA = np.sign(dA)[:, None, :] * np.exp(x + lA)   # e^{k_i - age w} dA
    cB = np.sign(dB)[:, None, :] * np.exp(x + lB)
    dv = cA
    dk = cA * v + cB
    dw = -np.sum(age * dk, axis=(0, 1))
    f = np.exp(-T * w[None, :] + p)                  # e^{-T w} e^p
    xa, xb = dA * f, dB * f                          # into da, db
    dw = dw - T * np.sum(xa * a + xb * b, axis=0)
    return dk, dv, dw, np.zeros_like(w), xa, xb, a * xa + b * xb


def backward_state_grad_cot(w, u, k, v, dy, state, dA, dB):
    """backward_state_grad for L = sum(dy * y) + sum(dA A_T + dB B_T)."""
    base = backward_state_grad(w, u, k, v, dy, state)
    extra = final_state_terms(w, u, k, v, state, dA, dB)
    return tuple(x + y for x, y in zip(base, extra))
