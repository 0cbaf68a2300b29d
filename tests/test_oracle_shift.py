"""Pins for the token-shift oracle (CPU only).

"RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (7): R, K, V are computed from a
weighted sum of the current and the previous token's input. Pinned by the cases the
weights fix (mu = 1 is the current token, mu = 0 the previous one, mu = 1/2 their mean),
by chaining calls through the carried last token, and by finite differences.
"""
import numpy as np

import oracle


def _rand(B, T, C, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, T, C)), rng.uniform(0, 1, (3, C)), rng.standard_normal((B, C))


def test_closed_forms():
    x, _, prev = _rand(2, 5, 4, 80)
    mu = np.stack([np.ones(4), np.zeros(4), np.full(4, 0.5)])
    (o_r, o_k, o_v), last = oracle.token_shift(x, mu, prev)
    np.testing.assert_array_equal(o_r, x)
    np.testing.assert_array_equal(o_k[:, 0], prev)
    np.testing.assert_array_equal(o_k[:, 1:], x[:, :-1])
    np.testing.assert_allclose(o_v[:, 2], 0.5 * (x[:, 2] + x[:, 1]), rtol=1e-15)
    np.testing.assert_array_equal(last, x[:, -1])
    (_, o_k0, _), _ = oracle.token_shift(x, mu)  # a fresh sequence: the previous input is 0
    np.testing.assert_array_equal(o_k0[:, 0], 0.0)


def test_chained_calls_equal_one_call():
    x, mu, prev = _rand(3, 11, 5, 81)
    whole, last = oracle.token_shift(x, mu, prev)
    a, mid = oracle.token_shift(x[:, :4], mu, prev)
    b, last2 = oracle.token_shift(x[:, 4:], mu, mid)
    for m in range(3):
        np.testing.assert_array_equal(np.concatenate([a[m], b[m]], axis=1), whole[m])
    np.testing.assert_array_equal(last2, last)


def test_backward_finite_differences():
    x, mu, prev = _rand(2, 4, 3, 82)
    rng = np.random.default_rng(83)
    dout = [rng.standard_normal(x.shape) for _ in range(3)]
    dx, dprev, dmu = oracle.token_shift_backward(x, mu, dout, prev)
    args = {"x": x, "mu": mu, "prev": prev}

    def loss(a):
        outs, _ = oracle.token_shift(a["x"], a["mu"], a["prev"])
        return float(sum(np.sum(d * o) for d, o in zip(dout, outs)))

    for name, got in (("x", dx), ("mu", dmu), ("prev", dprev)):
        v = args[name]
        fd = np.empty_like(v)
        for idx in np.ndindex(v.shape):
            h = 1e-6 * max(1.0, abs(v[idx]))
            ap, am = dict(args), dict(args)
            ap[name], am[name] = v.copy(), v.copy()
            ap[name][idx] += h
            am[name][idx] -= h
            fd[idx] = (loss(ap) - loss(am)) / (2 * h)
        np.testing.assert_allclose(got, fd, rtol=1e-7, atol=1e-9, err_msg=name)
