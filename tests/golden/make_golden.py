"""Write tests/golden/oracle_small.json from the oracle alone.

The fixture freezes the oracle's fp64 output on a slice of the "small" workload
(first 2 channels, first 12 tokens) so that an accidental change to the oracle's
arithmetic shows up as a test failure. It calls nothing but oracle/ and wkv_inputs.
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import wkv_inputs  # noqa: E402


def main():
    x = wkv_inputs.generate("small")
    sl = (slice(None), slice(0, 12), slice(0, 2))
    w, u = x["w"][:2], x["u"][:2]
    k, v, dy = x["k"][sl], x["v"][sl], x["dy"][sl]
    y = oracle.forward_direct(w, u, k, v)
    dk, dv, dw, du = oracle.backward_direct(w, u, k, v, dy)
    out = {
        "source": "oracle.forward_direct / oracle.backward_direct on wkv_inputs.generate('small')"
                  "[:, :12, :2]; written by tests/golden/make_golden.py",
        "inputs_fp32_hex": {n: [float(z).hex() for z in np.ravel(a).astype(np.float64)]
                            for n, a in (("w", w), ("u", u), ("k", k), ("v", v), ("dy", dy))},
        "shape": list(k.shape),
        "y": np.ravel(y).tolist(),
        "dk": np.ravel(dk).tolist(),
        "dv": np.ravel(dv).tolist(),
        "dw": np.ravel(dw).tolist(),
        "du": np.ravel(du).tolist(),
    }
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
