"""Plain fp64 CPU oracle for the token-shift mix (TEST INFRASTRUCTURE ONLY, like the rest of
this package: only tests/, the smoke check and the benchmark's CPU leg call it).

"RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (7): the input from which R, K
and V are computed is not the current token's embedding alone but a weighted sum of the
current and the previous token's, with a trained per-channel weight for each of the three.
Here, for one batch row and channel (0-based t, x_{-1} the previous token's input carried
over from an earlier call, 0 for a fresh sequence):

    out_m[t] = mu_m x[t] + (1 - mu_m) x[t-1],   m = r, k, v

The projections that follow are matrix products and not part of this. The backward of
L = sum_m sum dout_m * out_m follows from the same line by the product rule.
"""
import numpy as np


def _shifted(x, x_prev):
    x = np.asarray(x, np.float64)
    B, T, C = x.shape
    prev = np.zeros((B, C)) if x_prev is None else np.asarray(x_prev, np.float64)
    return x, np.concatenate([prev[:, None, :], x[:, :-1, :]], axis=1)


def token_shift(x, mu, x_prev=None):
    """(out_r, out_k, out_v) [B, T, C] and the last token's x [B, C] (the next call's x_prev).
    mu is [3, C] (rows r, k, v)."""
    x, xs = _shifted(x, x_prev)
    mu = np.asarray(mu, np.float64)
    outs = tuple(mu[m] * x + (1.0 - mu[m]) * xs for m in range(3))
    return outs, x[:, -1, :].copy()


def token_shift_backward(x, mu, dout, x_prev=None):
    """(dx [B, T, C], dx_prev [B, C], dmu [3, C]) of L = sum_m sum(dout[m] * out_m)."""
    x, xs = _shifted(x, x_prev)
    mu = np.asarray(mu, np.float64)
    d = [np.asarray(g, np.float64) for g in dout]
    dx = np.zeros_like(x)
    dxs = np.zeros_like(x)  # gradient with respect to the shifted input x[t-1]
    dmu = np.zeros((3, x.shape[2]))
    for m in range(3):
        dx += mu[m] * d[m]
        dxs += (1.0 - mu[m]) * d[m]
        dmu[m] = np.sum((x - xs) * d[m], axis=(0, 1))
    dx[:, :-1, :] += dxs[:, 1:, :]  # x[t] is the shifted input of token t + 1
    return dx, dxs[:, 0, :].copy(), dmu
