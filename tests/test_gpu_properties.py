"""Properties of the operator checked on the GPU path itself (marked gpu).

Beside the element-by-element parity against the fp64 oracle, the library's own outputs
must show what the pages say the operator is:

- a weighted average of the values, with the current token's bonus and a decay that grows
  with distance ("RWKV についての調査記録", section 【wkvとは】): every y_t lies between the
  smallest and largest v_i, i <= t, and y(alpha v + beta) = alpha y(v) + beta;
- channel by channel, with no mixing between channels (the same section), and sequence
  by sequence: a permutation of the channels permutes the outputs, and a sequence run alone
  gives its row of the batched run;
- causal, over the past and the current token only ("RWKV解读：在Transformer的时代的新RNN",
  section 二.3, formula (8)): changing token s leaves every output before it unchanged, and
  in the backward changing the cotangent at s leaves every gradient after it unchanged;
- a softmax over the logits, so adding one constant to every key changes nothing.

Outputs computed from the same inputs in a different arrangement are compared bitwise
where the arithmetic is the same (a sequence alone, tokens in windows the change does not
reach) and within the operator's tolerance |x - r| <= 1e-4 max(|r|, 0.1) elsewhere.
"""
import numpy as np
import pytest

import wkv_inputs
from helpers import assert_wkv_close

pytestmark = pytest.mark.gpu

B, T, C = 3, 300, 130  # windows of 64 tokens and channel groups of 64, both ragged


def _inputs(seed):
    return wkv_inputs.generate("l3b", seed=seed, B=B, T=T, C=C)


def _dev(dev, x):
    import torch
    return {n: torch.from_numpy(np.ascontiguousarray(a)).to(dev) for n, a in x.items()}


def _fwd(wkv, t):
    import torch
    y = wkv.forward(t["w"], t["u"], t["k"], t["v"])
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def test_outputs_are_weighted_averages_of_the_values(wkv, dev):
    x = _inputs(201)
    y = _fwd(wkv, _dev(dev, x))
    v = x["v"].astype(np.float64)
    lo = np.minimum.accumulate(v, axis=1)
    hi = np.maximum.accumulate(v, axis=1)
    slack = 1e-4 * np.maximum(np.abs(v).max(), 0.1)
    assert np.all(y >= lo - slack) and np.all(y <= hi + slack)


def test_affine_in_the_values(wkv, dev):
    x = _inputs(202)
    y = _fwd(wkv, _dev(dev, x))
    alpha, beta = np.float32(-2.5), np.float32(0.75)
    x2 = dict(x, v=(alpha * x["v"] + beta).astype(np.float32))
    y2 = _fwd(wkv, _dev(dev, x2))
    assert_wkv_close(y2, alpha * y + beta, "y(alpha v + beta)")


def test_channel_permutation_permutes_outputs(wkv, dev):
    x = _inputs(203)
    y = _fwd(wkv, _dev(dev, x))
    perm = np.random.default_rng(203).permutation(C)
    xp = {n: a[..., perm] for n, a in x.items()}  # w, u along with k, v
    yp = _fwd(wkv, _dev(dev, xp))
    assert_wkv_close(yp, y[..., perm], "permuted channels")


def test_a_sequence_alone_gives_its_row(wkv, dev):
    import torch
    x = _inputs(204)
    t = _dev(dev, x)
    y = _fwd(wkv, t)
    g = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"])
    torch.cuda.synchronize()
    for b in range(B):
        xb = {n: (a[b:b + 1] if a.ndim == 3 else a) for n, a in x.items()}
        tb = _dev(dev, xb)
        yb = _fwd(wkv, tb)
        assert np.array_equal(yb[0], y[b]), "y of sequence %d" % b
        gb = wkv.backward(tb["w"], tb["u"], tb["k"], tb["v"], tb["dy"])
        torch.cuda.synchronize()
        assert torch.equal(gb[0][0], g[0][b]) and torch.equal(gb[1][0], g[1][b]), \
            "dk, dv of sequence %d" % b


@pytest.mark.parametrize("s", [0, 31, 64, 130, 299])
def test_forward_is_causal(wkv, dev, s):
    x = _inputs(205)
    y = _fwd(wkv, _dev(dev, x))
    x2 = {n: a.copy() for n, a in x.items()}
    x2["k"][:, s] += np.float32(3.0)
    x2["v"][:, s] = -x2["v"][:, s] + np.float32(1.0)
    y2 = _fwd(wkv, _dev(dev, x2))
    start = (s // 32) * 32  # the 32-token chunk holding s shares one frame
    assert np.array_equal(y2[:, :start], y[:, :start])
    if s > start:
        assert_wkv_close(y2[:, start:s], y[:, start:s], "outputs before the changed token")
    assert not np.array_equal(y2[:, s], y[:, s])


@pytest.mark.parametrize("s", [0, 63, 100, 299])
def test_backward_is_anticausal(wkv, dev, s):
    import torch
    x = _inputs(206)
    t = _dev(dev, x)
    g = wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"])
    dy2 = t["dy"].clone()
    dy2[:, s] = -dy2[:, s] + 0.5
    g2 = wkv.backward(t["w"], t["u"], t["k"], t["v"], dy2)
    torch.cuda.synchronize()
    end = min((s // 32 + 1) * 32, T)  # the chunk holding s
    for a, b_, n in zip(g2[:2], g[:2], ("dk", "dv")):
        a, b_ = a.cpu().numpy().astype(np.float64), b_.cpu().numpy().astype(np.float64)
        assert np.array_equal(a[:, end:], b_[:, end:]), n + " after the changed token"
        if end > s + 1:
            assert_wkv_close(a[:, s + 1:end], b_[:, s + 1:end], n + " in the changed chunk")


def test_a_common_key_offset_changes_nothing(wkv, dev):
    x = _inputs(207)
    # keys on a grid of 1/64, so that k + 16 is exact in fp32
    x["k"] = (np.round(x["k"] * 64.0) / 64.0).astype(np.float32)
    y = _fwd(wkv, _dev(dev, x))
    x2 = dict(x, k=(x["k"] + np.float32(16.0)).astype(np.float32))
    y2 = _fwd(wkv, _dev(dev, x2))
    assert_wkv_close(y2, y, "y(k + 16)")
