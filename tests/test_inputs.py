"""The seeded input generator: determinism, value ranges and layouts."""
import numpy as np

import dn_inputs as gi


def test_same_seed_same_bytes():
    cfg = gi.CONFIGS["tiny"]
    a, sa = gi.generate(cfg)
    b, sb = gi.generate(cfg)
    for f in ["w_in", "s_in", "conv_w", "norm_w", "w_out", "s_out", "S0", "ring0"]:
        assert np.array_equal(getattr(a[0], f), getattr(b[0], f))
    for f in ["x", "alpha", "beta"]:
        assert np.array_equal(getattr(sa, f), getattr(sb, f))


def test_shapes_and_ranges_tiny():
    cfg = gi.CONFIGS["tiny"]
    (lay,), st = gi.generate(cfg)
    assert cfg.conv_channels == 128 and cfg.in_rows == 192
    assert lay.w_in.shape == (192, 64) and lay.w_in.dtype == np.int8
    assert lay.w_out.shape == (64, 64)
    assert lay.w_in.min() >= -127 and lay.w_in.max() <= 127
    assert lay.s_in.min() >= 0.005 and lay.s_in.max() <= 0.02
    assert np.all(lay.S0 == 0) and np.all(lay.ring0 == 0)
    assert st.x.shape == (8, 1, 64) and st.alpha.shape == (8, 1, 1, 4)
    assert st.alpha.min() >= np.float32(np.exp(-0.1)) and st.alpha.max() <= 1.0
    assert st.beta.min() > 0 and st.beta.max() < 1


def test_int4_packing_layout():
    cfg = gi.custom("i4", d_model=64, n_k_heads=2, d_k=16, n_v_heads=4, d_v=16, weight_bits=4)
    (lay,), _ = gi.generate(cfg)
    assert lay.w_in.dtype == np.uint8 and lay.w_in.shape == (192, 32)
    v = lay.w_in_vals
    assert v.min() >= -7 and v.max() <= 7
    lo = (lay.w_in & 15).astype(np.int16); hi = (lay.w_in >> 4).astype(np.int16)
    lo[lo >= 8] -= 16; hi[hi >= 8] -= 16
    assert np.array_equal(lo, v[:, 0::2]) and np.array_equal(hi, v[:, 1::2])


def test_metric_bytes_match_the_stated_budget():
    assert gi.CONFIGS["layer"].metric_bytes_per_step() == 37_937_664
    assert gi.CONFIGS["stack"].metric_bytes_per_step() == 1_138_129_920
    assert gi.CONFIGS["batched"].metric_bytes_per_step() == 302_178_816
    assert gi.CONFIGS["stack_int4"].metric_bytes_per_step() == 634_813_440
