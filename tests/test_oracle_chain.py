"""Why the 30-layer stack is compared layer by layer: the chain of layers itself amplifies a
perturbation of its input (CPU, the oracle alone).

Both runs are the fp64 oracle on the 30-layer stack workload (d_model 2048, 16 x 128 key and 32 x 128
value heads, the stack pre-norm), four tokens. The second run's layer-0 inputs are moved by one fp32
ulp each, a change of the size of one fp32 rounding. Layer 0's output moves by about 1e-6 of its rms,
but the map compounds the change by about 1.4x per layer, so layer 29's output moves by more than the
2e-3 output bar of the decode step. Hence no fp32 implementation can be held to 2e-3 against the fp64
chain at full depth: the benchmarked chain is checked with each layer compared with the oracle's step
fed that layer's input from the card, and the free-running comparison stops where the amplification
alone stays inside the bar."""
import numpy as np

import dn_inputs as gi
import oracle as orc


def _rel(a, b):
    """max over tokens of max|a - b| / rms(b)."""
    g = a.reshape(a.shape[0], -1)
    r = b.reshape(b.shape[0], -1)
    return float(np.max(np.max(np.abs(g - r), axis=1) / np.sqrt(np.mean(r * r, axis=1))))


def _drift():
    cfg = gi.CONFIGS["stack"]
    layers, stream = gi.generate(cfg, n_tokens=4)
    o0, _, _ = orc.run(cfg, layers, stream)
    x1 = np.nextafter(stream.x, np.float32(np.inf)).astype(np.float32)
    assert np.all(x1 != stream.x)
    o1, _, _ = orc.run(cfg, layers, gi.Stream(x1, stream.alpha, stream.beta))
    return [_rel(o1[:, l], o0[:, l]) for l in range(cfg.n_layers)]


def test_one_ulp_at_the_input_grows_past_the_output_bar_by_layer_30():
    d = _drift()
    print("drift per layer: " + " ".join(f"{v:.1e}" for v in d))
    assert d[0] < 1e-5              # one layer: of the order of the perturbation itself
    assert d[-1] > 2e-3             # thirty layers: past the decode step's output bar
    assert d[-1] / d[0] > 1e3       # compounded through the chain
    # the growth is steady, not one outlier layer: every stretch of 5 layers at least doubles it
    assert all(d[l + 5] > 2 * d[l] for l in range(0, 25, 5))
    # the depth to which the free-running chain is compared end to end stays inside the bar
    assert max(d[:12]) < 2e-4
