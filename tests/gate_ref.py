"""References for the receptance-gated WKV (out = sigma(r) * y), built from oracle routines
and the logistic function only. tests/test_oracle_gate.py pins them against central finite
differences of L = sum(dout * sigma(r) * y)."""
import numpy as np

import oracle


def sigmoid(x):
    """1 / (1 + e^{-x}) in fp64, without overflow for either sign."""
    x = np.asarray(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _forward(w, u, k, v, direct):
    return (oracle.forward_direct if direct else oracle.forward_recurrent)(w, u, k, v)


def forward_gated(w, u, k, v, r, direct=True):
    """sigma(r) * y; the O(T^2) definition for y (or the plain recursion for long inputs)."""
    return sigmoid(r) * _forward(w, u, k, v, direct)


def backward_gated(w, u, k, v, r, dout, direct=True):
    """(dk, dv, dr, dw, du) of L = sum(dout * sigma(r) * y): the cotangent of y is
    dout * sigma(r), and dL/dr = dout * y * sigma(r) (1 - sigma(r))."""
    s = sigmoid(r)
    dout = np.asarray(dout, np.float64)
    y = _forward(w, u, k, v, direct)
    back = oracle.backward_direct if direct else oracle.backward_recurrent
    dk, dv, dw, du = back(w, u, k, v, dout * s)
    return dk, dv, dout * y * s * (1.0 - s), dw, du
