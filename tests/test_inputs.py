"""The seeded generators are deterministic and draw the stated distributions (CPU only)."""
import numpy as np

import wkv_inputs


def test_deterministic_and_shapes():
    a = wkv_inputs.generate("small")
    b = wkv_inputs.generate("small")
    for n in ("w", "u", "k", "v", "dy"):
        assert a[n].dtype == np.float32
        assert np.array_equal(a[n], b[n])
    assert a["k"].shape == (1, 64, 64) and a["w"].shape == (64,)
    c = wkv_inputs.generate("small", seed=7)
    assert not np.array_equal(a["k"], c["k"])


def test_distributions():
    x = wkv_inputs.generate("longctx", T=2048, C=512)
    d = np.log(x["w"].astype(np.float64))
    assert d.min() >= -8.0 - 1e-5 and d.max() <= 2.0 + 1e-5
    assert np.abs(x["u"]).max() <= 3.0
    spikes = np.abs(x["k"]) == 30.0
    frac = spikes.mean()
    assert 0.008 < frac < 0.012
    assert abs((x["k"][spikes] > 0).mean() - 0.5) < 0.05
    body = x["k"][~spikes]
    assert abs(body.std() - 4.0) < 0.05
    y = wkv_inputs.generate("l169m", T=64)
    assert abs(y["k"].std() - 1.0) < 0.01 and abs(y["v"].mean()) < 0.01


def test_decode_draws():
    w, u = wkv_inputs.decode_layer_params(3, C=128)
    w2, _ = wkv_inputs.decode_layer_params(3, C=128)
    assert np.array_equal(w, w2) and w.dtype == np.float32
    k0, v0 = wkv_inputs.decode_step_inputs(0, 3, B=4, C=128)
    k1, _ = wkv_inputs.decode_step_inputs(1, 3, B=4, C=128)
    assert not np.array_equal(k0, k1)
    a, b, p = wkv_inputs.empty_decode_state(2, 5)
    assert np.all(a == 0) and np.all(b == 0) and np.all(p == np.float32(-1e38))
