"""The oracle against the fixture its own generator script wrote (tests/golden/): a change to the
oracle's arithmetic fails here. The pages print no values of the step, so this is a regression lock
on the oracle, not an external pin; the pins are in test_oracle_pins.py."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_tiny_fixture as fx  # noqa: E402


def test_tiny_fixture_unchanged():
    with open(os.path.join(HERE, "golden", "tiny_oracle.json")) as f:
        want = json.load(f)
    got = fx.compute()
    for key in ("out_first8_per_token", "out_rms_per_token", "state_sum_per_head"):
        np.testing.assert_allclose(np.array(got[key]), np.array(want[key]), rtol=1e-12, atol=1e-14, err_msg=key)
    for key in ("state_frobenius", "ring_sum"):
        assert abs(got[key] - want[key]) <= 1e-12 * max(1.0, abs(want[key])), key
