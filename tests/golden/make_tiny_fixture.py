"""Write tests/golden/tiny_oracle.json: the oracle's outputs on the tiny workload (one layer, d_model
64, 2 key heads x 16, 4 value heads x 16, 8 tokens, seed 0, zero initial state).

The fixture locks the oracle's numbers: a later change to its arithmetic shows up as a failure of
tests/test_golden.py and has to be justified by the passage it follows. Every value is computed
here by the oracle alone, on inputs from the seeded generator; nothing comes from the GPU path.

    python tests/golden/make_tiny_fixture.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import dn_inputs as gi  # noqa: E402
import oracle as orc  # noqa: E402


def compute():
    cfg = gi.CONFIGS["tiny"]
    layers, stream = gi.generate(cfg)
    out, S, hist = orc.run(cfg, layers, stream)
    o = out[:, 0, 0, :]  # [T][D]
    return {
        "workload": "tiny: one layer, d_model 64, 2 key heads x 16, 4 value heads x 16, conv 4, 8 tokens, seed 0, S0 = 0",
        "out_first8_per_token": [[float(v) for v in row[:8]] for row in o],
        "out_rms_per_token": [float(np.sqrt(np.mean(row * row))) for row in o],
        "state_sum_per_head": [float(v) for v in S[0, 0].sum(axis=(1, 2))],
        "state_frobenius": float(np.linalg.norm(S)),
        "ring_sum": float(hist.sum()),
    }


if __name__ == "__main__":
    path = os.path.join(HERE, "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=1)
        f.write("\n")
    print("wrote", path)
