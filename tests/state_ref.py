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
