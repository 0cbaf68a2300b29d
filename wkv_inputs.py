"""Seeded synthetic inputs for the WKV operator.

Shared by the tests (oracle and GPU sides alike) and by bench.py. This module holds
no WKV arithmetic: it only draws arrays. Draws use numpy's PCG64 (``default_rng``),
in fp32, in the fixed order d, u, k, [spike mask, spike sign], v, dy, with the decay
rate w = exp(d) taken in fp32. The same fp32 arrays go to the GPU and to the oracle.

Workloads (B = sequences, T = tokens, C = channels; k, v, dy are [B][T][C]):

  small      B=1  T=64   C=64    d~U(-6,1) u~U(-1,1) k,v,dy~N(0,1)           fwd+bwd
  l169m      B=8  T=1024 C=768   d~U(-6,1) u~U(-1,1) k,v~N(0,1)              fwd
  l3b        B=8  T=4096 C=2560  d~U(-8,2) u~U(-1,1) k,v,dy~N(0,1)           fwd+bwd
  longctx    B=1  T=8192 C=4096  d~U(-8,2) u~U(-3,3) k~N(0,4^2), 1% of k set
                                 to +-30 (Bernoulli(0.01), sign +-1 w.p. 1/2),
                                 v,dy~N(0,1)                                  fwd+bwd
  decode     B=256 C=5120, 40 layer states, per layer d~U(-8,2) u~U(-1,1),
             per step and layer k,v~N(0,1) [B][C]                             decode

Shapes follow the model sizes the pages mention (a 169M-parameter model,
3B-class layers, long contexts); no public dataset is involved.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "small": dict(index=1, B=1, T=64, C=64, d=(-6.0, 1.0), u=(-1.0, 1.0), k_std=1.0,
                  spike_p=0.0, ops="fwd+bwd"),
    "l169m": dict(index=2, B=8, T=1024, C=768, d=(-6.0, 1.0), u=(-1.0, 1.0), k_std=1.0,
                  spike_p=0.0, ops="fwd"),
    "l3b": dict(index=3, B=8, T=4096, C=2560, d=(-8.0, 2.0), u=(-1.0, 1.0), k_std=1.0,
                spike_p=0.0, ops="fwd+bwd"),
    "longctx": dict(index=4, B=1, T=8192, C=4096, d=(-8.0, 2.0), u=(-3.0, 3.0), k_std=4.0,
                    spike_p=0.01, spike_val=30.0, ops="fwd+bwd"),
}

DECODE = dict(index=5, B=256, C=5120, layers=40, steps=1000, d=(-8.0, 2.0), u=(-1.0, 1.0))


def default_seed(name: str) -> int:
    if name == "decode":
        return 1000 + DECODE["index"]
    return 1000 + WORKLOADS[name]["index"]


def generate(name: str, seed: int | None = None, B: int | None = None, T: int | None = None,
             C: int | None = None, with_dy: bool = True) -> dict:
    """Draw (w, u, k, v[, dy]) for a named workload; B/T/C override its shape.

    Returns fp32 numpy arrays: w, u of shape [C]; k, v, dy of shape [B, T, C].
    """
    cfg = WORKLOADS[name]
    B = cfg["B"] if B is None else B
    T = cfg["T"] if T is None else T
    C = cfg["C"] if C is None else C
    rng = np.random.default_rng(default_seed(name) if seed is None else seed)
    d = rng.uniform(cfg["d"][0], cfg["d"][1], size=C).astype(np.float32)
    u = rng.uniform(cfg["u"][0], cfg["u"][1], size=C).astype(np.float32)
    k = rng.standard_normal(size=(B, T, C), dtype=np.float32)
    if cfg["k_std"] != 1.0:
        k *= np.float32(cfg["k_std"])
    if cfg["spike_p"] > 0.0:
        mask = rng.random(size=(B, T, C), dtype=np.float32) < cfg["spike_p"]
        sign = np.where(rng.random(size=(B, T, C), dtype=np.float32) < 0.5,
                        np.float32(-1.0), np.float32(1.0))
        k = np.where(mask, sign * np.float32(cfg["spike_val"]), k).astype(np.float32)
    v = rng.standard_normal(size=(B, T, C), dtype=np.float32)
    out = dict(w=np.exp(d).astype(np.float32), u=u, k=k, v=v)
    if with_dy:
        out["dy"] = rng.standard_normal(size=(B, T, C), dtype=np.float32)
    return out


def random_state(B: int, C: int, seed: int, p_range=(-4.0, 4.0)):
    """A decode-convention state (a, b, p) [B, C] fp32 to start a forward from: b ~ U(0.5, 8),
    a = b * N(0, 1) (so a / b, the state's mean value, is ~ N(0, 1)), p ~ U(p_range)."""
    rng = np.random.default_rng(seed)
    b = rng.uniform(0.5, 8.0, size=(B, C)).astype(np.float32)
    a = (b * rng.standard_normal(size=(B, C))).astype(np.float32)
    p = rng.uniform(p_range[0], p_range[1], size=(B, C)).astype(np.float32)
    return a, b, p


def decode_layer_params(layer: int, seed: int | None = None, C: int | None = None):
    """Per-layer (w, u) [C] fp32 for the batched-decode workload."""
    C = DECODE["C"] if C is None else C
    base = default_seed("decode") if seed is None else seed
    rng = np.random.default_rng([base, 0, layer])
    d = rng.uniform(DECODE["d"][0], DECODE["d"][1], size=C).astype(np.float32)
    u = rng.uniform(DECODE["u"][0], DECODE["u"][1], size=C).astype(np.float32)
    return np.exp(d).astype(np.float32), u


def decode_step_inputs(step: int, layer: int, seed: int | None = None, B: int | None = None,
                       C: int | None = None):
    """Per-(step, layer) (k, v) [B, C] fp32 for the batched-decode workload."""
    B = DECODE["B"] if B is None else B
    C = DECODE["C"] if C is None else C
    base = default_seed("decode") if seed is None else seed
    rng = np.random.default_rng([base, 1 + step, layer])
    k = rng.standard_normal(size=(B, C), dtype=np.float32)
    v = rng.standard_normal(size=(B, C), dtype=np.float32)
    return k, v


def empty_decode_state(B: int, C: int):
    """The initial decode state: a = b = 0, p = -1e38 (fp32, [B, C] each)."""
    return (np.zeros((B, C), np.float32), np.zeros((B, C), np.float32),
            np.full((B, C), -1e38, np.float32))
