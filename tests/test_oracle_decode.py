"""Pins for the oracle's recurrent state and decode step (CPU only).

The pages describe inference as an RNN that takes a token and a state and returns the
new state ("RWKV についての調査記録", section "RWKVとは？"; "介绍RWKV – 具有Transformer优势的RNN",
section "RWKV作为RNN和transformer的结合体"), and say formula (8) has a recursive form
("RWKV解读：在Transformer的时代的新RNN", section 二.3). These tests pin the state (a, b, p),
meaning A = a e^p and B = b e^p, against the direct definition and closed forms.
"""
import numpy as np

import oracle
import wkv_inputs


def _rand(B, T, C, seed, kscale=1.0):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-8.0, 2.0, size=C))
    u = rng.uniform(-1.0, 1.0, size=C)
    k = kscale * rng.standard_normal((B, T, C))
    v = rng.standard_normal((B, T, C))
    return w, u, k, v


def test_decode_chain_equals_parallel_form():
    w, u, k, v = _rand(4, 40, 6, 31, kscale=2.0)
    ref = oracle.forward_direct(w, u, k, v)
    st = wkv_inputs.empty_decode_state(4, 6)
    for t in range(40):
        y, st = oracle.decode_step(w, u, k[:, t], v[:, t], st)
        np.testing.assert_allclose(y, ref[:, t], rtol=1e-11, atol=1e-13)


def test_state_meaning_geometric():
    # k = 0 and v = 1: after t tokens A = B = sum_{j<t} e^{-jw} = (1 - e^{-tw}) / (1 - e^{-w}).
    C, T = 5, 25
    w = np.array([0.01, 0.2, 1.0, 3.0, 7.0])
    u = np.zeros(C)
    _, (a, b, p) = oracle.forward_rescaled(w, u, np.zeros((1, T, C)), np.ones((1, T, C)))
    ref = (1 - np.exp(-T * w)) / (1 - np.exp(-w))
    np.testing.assert_allclose(b[0] * np.exp(p[0]), ref, rtol=1e-13)
    np.testing.assert_allclose(a[0] * np.exp(p[0]), ref, rtol=1e-13)


def test_resume_is_bitwise():
    w, u, k, v = _rand(3, 30, 4, 32, kscale=3.0)
    y_all, st_all = oracle.forward_rescaled(w, u, k, v)
    y1, st = oracle.forward_rescaled(w, u, k[:, :13], v[:, :13])
    y2, st2 = oracle.forward_rescaled(w, u, k[:, 13:], v[:, 13:], st)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y_all)
    for x, y in zip(st2, st_all):
        assert np.array_equal(x, y)


def test_state_rescaling_is_equivalent():
    # (a e^d, b e^d, p - d) is the same state: the next outputs agree.
    w, u, k, v = _rand(2, 20, 3, 33, kscale=2.0)
    _, (a, b, p) = oracle.forward_rescaled(w, u, k[:, :10], v[:, :10])
    d = np.array([[5.0, -3.0, 0.5], [-40.0, 12.0, 1.0]])
    y1, _ = oracle.forward_rescaled(w, u, k[:, 10:], v[:, 10:], (a, b, p))
    y2, _ = oracle.forward_rescaled(w, u, k[:, 10:], v[:, 10:], (a * np.exp(d), b * np.exp(d), p - d))
    np.testing.assert_allclose(y2, y1, rtol=1e-12, atol=1e-14)


def test_empty_state_first_output_is_v():
    w, u, k, v = _rand(3, 1, 7, 34, kscale=10.0)
    y, st = oracle.decode_step(w, u, k[:, 0], v[:, 0], wkv_inputs.empty_decode_state(3, 7))
    np.testing.assert_allclose(y, v[:, 0], rtol=1e-14)
    np.testing.assert_allclose(st[0] / st[1], v[:, 0], rtol=1e-14)  # a / b = v after one token
