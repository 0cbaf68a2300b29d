"""GPU parity of the token-shift mix against the fp64 oracle (marked gpu).

"RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (7): the inputs of the R, K, V
projections are weighted sums of the current and the previous token's input. Oracle:
oracle.token_shift / token_shift_backward (pinned in test_oracle_shift.py). Tolerance as
everywhere: |x - r| <= 1e-4 max(|r|, 0.1).
"""
import numpy as np
import pytest

import oracle
from helpers import assert_wkv_close

pytestmark = pytest.mark.gpu


def _t(dev, a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def _inputs(B, T, C, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, C)).astype(np.float32)
    mu = rng.uniform(0, 1, (3, C)).astype(np.float32)
    prev = rng.standard_normal((B, C)).astype(np.float32)
    dout = [rng.standard_normal((B, T, C)).astype(np.float32) for _ in range(3)]
    return x, mu, prev, dout


@pytest.mark.parametrize("with_prev", [False, True])
@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 37, 70), (3, 65, 130), (1, 300, 64),
                                   (2, 129, 200)])
def test_parity(wkv, dev, B, T, C, with_prev):
    import torch
    x, mu, prev, dout = _inputs(B, T, C, seed=90 + B * T + C)
    xp = prev if with_prev else None
    outs = wkv.token_shift(_t(dev, x), _t(dev, mu), _t(dev, xp) if with_prev else None)
    dx, dprev, dmu = wkv.token_shift_backward(_t(dev, x), _t(dev, mu),
                                              [_t(dev, d) for d in dout],
                                              _t(dev, xp) if with_prev else None)
    torch.cuda.synchronize()
    ref, last = oracle.token_shift(x, mu, xp)
    rdx, rdprev, rdmu = oracle.token_shift_backward(x, mu, dout, xp)
    worst = 0.0
    for g, r, n in zip(outs[:3], ref, ("out_r", "out_k", "out_v")):
        worst = max(worst, assert_wkv_close(g.cpu().numpy(), r, n))
    assert np.array_equal(outs[3].cpu().numpy(), x[:, -1])
    worst = max(worst, assert_wkv_close(dx.cpu().numpy(), rdx, "dx"))
    worst = max(worst, assert_wkv_close(dmu.cpu().numpy(), rdmu, "dmu"))
    if with_prev:
        worst = max(worst, assert_wkv_close(dprev.cpu().numpy(), rdprev, "dx_prev"))
    print("[shift] B=%d T=%d C=%d prev=%s max_violation=%.3g" % (B, T, C, with_prev, worst),
          flush=True)


def test_chained_calls_equal_one_call(wkv, dev):
    import torch
    x, mu, prev, _ = _inputs(2, 200, 96, seed=95)
    xt, mt = _t(dev, x), _t(dev, mu)
    whole = wkv.token_shift(xt, mt, _t(dev, prev))
    a = wkv.token_shift(xt[:, :77].contiguous(), mt, _t(dev, prev))
    b = wkv.token_shift(xt[:, 77:].contiguous(), mt, a[3])
    torch.cuda.synchronize()
    for m in range(3):
        assert torch.equal(torch.cat([a[m], b[m]], dim=1), whole[m])
    assert torch.equal(b[3], whole[3])


def test_empty_sequence_backward(wkv, dev):
    import torch
    x = torch.zeros(2, 0, 40, device=dev)
    mu = _t(dev, np.full((3, 40), 0.3))
    dx, dprev, dmu = wkv.token_shift_backward(x, mu, [x, x, x], torch.ones(2, 40, device=dev))
    torch.cuda.synchronize()
    assert torch.all(dmu == 0) and torch.all(dprev == 0) and dx.numel() == 0


def test_full_layer(wkv, dev):
    import torch
    x, mu, prev, dout = _inputs(8, 4096, 2560, seed=96)
    outs = wkv.token_shift(_t(dev, x), _t(dev, mu), _t(dev, prev))
    dx, dprev, dmu = wkv.token_shift_backward(_t(dev, x), _t(dev, mu),
                                              [_t(dev, d) for d in dout], _t(dev, prev))
    torch.cuda.synchronize()
    ref, _ = oracle.token_shift(x, mu, prev)
    rdx, rdprev, rdmu = oracle.token_shift_backward(x, mu, dout, prev)
    worst = max(assert_wkv_close(g.cpu().numpy(), r, "out") for g, r in zip(outs[:3], ref))
    worst = max(worst, assert_wkv_close(dx.cpu().numpy(), rdx, "dx"))
    worst = max(worst, assert_wkv_close(dprev.cpu().numpy(), rdprev, "dx_prev"))
    worst = max(worst, assert_wkv_close(dmu.cpu().numpy(), rdmu, "dmu"))
    print("[shift] l3b max_violation=%.3g" % worst, flush=True)
