"""The ABI's size limits on the card: a stack of 256 layers (the most a handle takes) on the
whole-stack kernel, the layer limits of its per-key and two-wave (48-head) forms, and a batch of 1024
sequences (the most a handle takes) on the batched and per-layer paths.

The 256-layer stack cannot be compared free-running with the oracle: the chain amplifies rounding
by about 1.44x per layer. Each layer is instead checked against the oracle's step of that layer fed
the card's own input to it (out[l-1] from the card), with the oracle's state for that layer carried
over the two tokens; so every layer's weights, gates, state, history and hand-off tags are
exercised at the limit."""
import numpy as np
import pytest
import torch

import dn_inputs as gi
import oracle as orc

from gpu_util import OUT_TOL, STATE_TOL, check_layers_fed_from_the_card, make_stack, out_err, run_gpu, state_err

pytestmark = pytest.mark.gpu


def _path(cfg, layers, capfd, monkeypatch, env=None):
    monkeypatch.setenv("DN_VERBOSE", "1")
    if env:
        monkeypatch.setenv(env, "1")
    st = make_stack(cfg, layers)
    monkeypatch.delenv("DN_VERBOSE")
    if env:
        monkeypatch.delenv(env)
    return st, capfd.readouterr().err


def _check_layers_fed_from_the_card(cfg, capfd, monkeypatch, path):
    layers, stream = gi.generate(cfg)
    print(f"[limits] {cfg.name}: {cfg.n_layers} layers generated", flush=True)
    st, err = _path(cfg, layers, capfd, monkeypatch)
    try:
        assert path in err, err
        gout = run_gpu(st, stream)  # [T][L][1][D]
        gS, gH = st.get_state()
        gS, gH = gS.cpu().numpy(), gH.cpu().numpy()
    finally:
        st.close()
    assert np.all(np.isfinite(gout))
    worst = check_layers_fed_from_the_card(cfg, layers, stream, gout, gS, gH)
    print(f"[limits] {cfg.name} ({path}): worst layer out {worst[0]:.2e} state {worst[1]:.2e} ring {worst[2]:.2e}",
          flush=True)
    assert worst[0] <= OUT_TOL and worst[1] <= STATE_TOL and worst[2] <= STATE_TOL


def test_whole_stack_at_the_layer_limit(capfd, monkeypatch):
    cfg = gi.custom("lim_L", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=256, n_tokens=2,
                    flags=gi.DN_X_RMSNORM, ring_std=1.0)
    _check_layers_fed_from_the_card(cfg, capfd, monkeypatch, "whole-stack kernel")


@pytest.mark.parametrize("L,path", [(32, "whole-stack kernel"), (33, "per-layer kernels")])
def test_per_key_decay_at_the_whole_stack_layer_limit(L, path, capfd, monkeypatch):
    """The whole-stack kernel keeps the per-key decays of up to 32 layers in LDS; one more layer
    takes the per-layer kernels."""
    cfg = gi.custom(f"lim_pk{L}", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=L, n_tokens=2,
                    flags=gi.DN_X_RMSNORM | gi.DN_ALPHA_PER_KEY, ring_std=1.0)
    _check_layers_fed_from_the_card(cfg, capfd, monkeypatch, path)


@pytest.mark.parametrize("L,path", [(64, "whole-stack kernel"), (65, "per-layer kernels")])
def test_48_heads_at_the_two_wave_layer_limit(L, path, capfd, monkeypatch):
    """The whole-stack kernel's two-wave form (48 value heads over d_model 2048) keeps the per-layer
    gate and norm tables of up to 64 layers in LDS; one more layer takes the per-layer kernels."""
    cfg = gi.custom(f"lim_h48_{L}", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=48, d_v=128, n_layers=L,
                    n_tokens=2, flags=gi.DN_X_RMSNORM, ring_std=1.0)
    _check_layers_fed_from_the_card(cfg, capfd, monkeypatch, path)


@pytest.mark.parametrize("env,path", [(None, "batched kernels"), ("DN_LAYER_KERNELS", "per-layer kernels")])
def test_batch_at_the_sequence_limit(env, path, capfd, monkeypatch):
    cfg = gi.custom("lim_B", d_model=512, n_k_heads=2, d_k=128, n_v_heads=4, d_v=128, batch=1024, n_tokens=2,
                    ring_std=1.0)
    layers, stream = gi.generate(cfg)
    st, err = _path(cfg, layers, capfd, monkeypatch, env)
    try:
        assert path in err, err
        gout = run_gpu(st, stream)
        gS, gH = st.get_state()
    finally:
        st.close()
    ref_out, ref_S, ref_H = orc.run(cfg, layers, stream)
    # per sequence: the output error relative to that sequence's output rms
    e = max(out_err(gout[:, 0, b], ref_out[:, 0, b]) for b in range(cfg.batch))
    es = state_err(gS.cpu().numpy(), ref_S)
    eh = state_err(gH.cpu().numpy(), ref_H)
    print(f"[limits] {cfg.name} ({path}): out {e:.2e} state {es:.2e} ring {eh:.2e}", flush=True)
    assert e <= OUT_TOL and es <= STATE_TOL and eh <= STATE_TOL


@pytest.mark.parametrize("name,kw", [
    # the widest model (16384 columns): in_proj rows and gate rows of 16 KiB, out_proj of 16384 rows
    ("lim_D", dict(d_model=16384, n_k_heads=1, d_k=16, n_v_heads=1, d_v=16)),
    # the widest readout: 64 value heads of 256 columns (out_proj rows of 16384 columns)
    ("lim_V", dict(d_model=256, n_k_heads=1, d_k=16, n_v_heads=64, d_v=256)),
])
def test_widths_at_the_limit(name, kw):
    """The per-layer kernels at the largest widths a handle takes, with the pre-norm and the gates
    computed on the card, two sequences, against the oracle."""
    cfg = gi.custom(name, batch=2, n_tokens=3, flags=gi.DN_X_RMSNORM | gi.DN_GATES_ON_DEVICE, ring_std=1.0, **kw)
    layers, stream = gi.generate(cfg)
    print(f"[limits] {name}: D={cfg.d_model} V={cfg.n_v_heads * cfg.d_v}", flush=True)
    ref_out, ref_S, ref_H = orc.run(cfg, layers, stream)
    st = make_stack(cfg, layers)
    try:
        gout = run_gpu(st, stream)
        gS, gH = st.get_state()
    finally:
        st.close()
    e, es, eh = out_err(gout, ref_out), state_err(gS.cpu().numpy(), ref_S), state_err(gH.cpu().numpy(), ref_H)
    print(f"[limits] {name}: out {e:.2e} state {es:.2e} ring {eh:.2e}", flush=True)
    assert e <= OUT_TOL and es <= STATE_TOL and eh <= STATE_TOL
