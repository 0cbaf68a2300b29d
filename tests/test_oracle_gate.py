"""Pins for the receptance-gated references (CPU only).

The time-mixing block gates the WKV result elementwise by the sigmoid of the receptance r
("RWKV解读：在Transformer的时代的新RNN", section 二.3: R is sigmoid-activated, formula (9);
"RWKV についての調査記録", section "コードを見ながらRWKVの構造を把握": wkv is computed,
then gated by sigma). The gradients of L = sum(dout * sigma(r) * y) are checked against
central finite differences on every input element of tiny cases.
"""
import numpy as np
import pytest

from gate_ref import backward_gated, forward_gated, sigmoid
import oracle


def test_sigmoid_values():
    assert sigmoid(0.0) == 0.5
    np.testing.assert_allclose(sigmoid([1.0, -1.0]), [0.7310585786300049, 0.2689414213699951],
                               rtol=1e-15)
    assert sigmoid(800.0) == 1.0 and sigmoid(-800.0) == 0.0


def test_forward_gated_is_the_gate_times_y():
    rng = np.random.default_rng(50)
    w = np.exp(rng.uniform(-4, 1, 3))
    u = rng.uniform(-1, 1, 3)
    k, v, r = (rng.standard_normal((2, 6, 3)) for _ in range(3))
    y = oracle.forward_direct(w, u, k, v)
    np.testing.assert_allclose(forward_gated(w, u, k, v, np.zeros_like(r)), 0.5 * y, rtol=1e-15)
    np.testing.assert_allclose(forward_gated(w, u, k, v, np.full_like(r, 60.0)), y, rtol=1e-15)


@pytest.mark.parametrize("seed", [51, 52])
def test_backward_gated_finite_differences(seed):
    rng = np.random.default_rng(seed)
    B, T, C = 2, 5, 3
    w = np.exp(rng.uniform(-4, 1, C))
    u = rng.uniform(-1, 1, C)
    k = 1.5 * rng.standard_normal((B, T, C))
    v, r, dout = (rng.standard_normal((B, T, C)) for _ in range(3))
    got = dict(zip(("k", "v", "r", "w", "u"), backward_gated(w, u, k, v, r, dout)))
    args = dict(w=w, u=u, k=k, v=v, r=r)

    def loss(a):
        return float(np.sum(dout * forward_gated(a["w"], a["u"], a["k"], a["v"], a["r"])))

    for name in ("k", "v", "r", "w", "u"):
        x = args[name]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-6 * max(1.0, abs(x[idx]))
            ap, am = dict(args), dict(args)
            ap[name], am[name] = x.copy(), x.copy()
            ap[name][idx] += h
            am[name][idx] -= h
            fd[idx] = (loss(ap) - loss(am)) / (2 * h)
        np.testing.assert_allclose(got[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)
