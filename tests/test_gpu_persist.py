"""The whole-stack decode kernel (one launch per token for single-sequence stacks with 128 x 128
state tiles): parity with the oracle on small compatible shapes, agreement with the per-layer
kernels, bitwise reruns, resume and the failed-step latch on this path."""
import numpy as np
import pytest
import torch

import dn_inputs as gi
import gated_deltanet_layer_dn_amd as dn
import oracle as orc

from gpu_util import OUT_TOL, STATE_TOL, make_stack, out_err, run_gpu, state_err, upload_stream

pytestmark = pytest.mark.gpu

PERSIST = {
    # 1024-wide model, 8 value heads (1024 value columns): 64 recurrence blocks on 256 workgroups
    "p_small": gi.custom("p_small", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=3,
                         n_tokens=8, flags=gi.DN_X_RMSNORM, ring_std=1.0),
    "p_int4": gi.custom("p_int4", d_model=2048, n_k_heads=2, d_k=128, n_v_heads=16, d_v=128, n_layers=2,
                        n_tokens=6, flags=gi.DN_X_RMSNORM, ring_std=1.0, weight_bits=4),
    "p_conv1": gi.custom("p_conv1", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, conv_k=1,
                         n_tokens=5),
    "p_conv2": gi.custom("p_conv2", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, conv_k=2,
                         n_tokens=5, ring_std=1.0),
    "p_nogqa": gi.custom("p_nogqa", d_model=1024, n_k_heads=8, d_k=128, n_v_heads=8, d_v=128, n_tokens=5,
                         q_scale=0.0883883),
    "p_full_shape": gi.custom("p_full", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128,
                              n_layers=2, n_tokens=6, flags=gi.DN_X_RMSNORM, ring_std=1.0),
    # one decay per key channel (alpha [L][Hv][128]), int8 and int4
    "p_perkey": gi.custom("p_pk", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=3,
                          n_tokens=7, flags=gi.DN_X_RMSNORM | gi.DN_ALPHA_PER_KEY, ring_std=1.0),
    "p_perkey_full_int4": gi.custom("p_pk4", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128,
                                    n_layers=2, n_tokens=5, weight_bits=4,
                                    flags=gi.DN_X_RMSNORM | gi.DN_ALPHA_PER_KEY, ring_std=1.0),
    # 48 value heads over 16 key heads at d_model 2048: the two-wave form (128 x 32 state slices on
    # 192 workgroups, 8 in_proj rows per compute wave, out_proj rows staged in LDS)
    "p_heads48": gi.custom("p_h48", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=48, d_v=128, n_layers=3,
                           n_tokens=6, flags=gi.DN_X_RMSNORM, ring_std=1.0),
    "p_heads48_conv2": gi.custom("p_h48c2", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=48, d_v=128,
                                 n_layers=2, conv_k=2, n_tokens=5, ring_std=1.0),
    # heads of 256 (8 key and 16 value heads) at d_model 2048: 256 x 16 state slices, 64 key rows per lane
    "p_dim256": gi.custom("p_d256", d_model=2048, n_k_heads=8, d_k=256, n_v_heads=16, d_v=256, n_layers=3,
                          n_tokens=6, flags=gi.DN_X_RMSNORM, ring_std=1.0),
    "p_dim256_conv3": gi.custom("p_d256c3", d_model=2048, n_k_heads=8, d_k=256, n_v_heads=16, d_v=256,
                                n_layers=2, conv_k=3, n_tokens=5, ring_std=1.0, q_scale=0.0625),
}


def _path_of(cfg, layers, capfd, monkeypatch):
    monkeypatch.setenv("DN_VERBOSE", "1")
    st = make_stack(cfg, layers)
    monkeypatch.delenv("DN_VERBOSE")
    err = capfd.readouterr().err
    return st, err


@pytest.mark.parametrize("name", list(PERSIST))
def test_persist_parity(name, capfd, monkeypatch):
    cfg = PERSIST[name]
    layers, stream = gi.generate(cfg)
    print(f"[persist] {name}", flush=True)
    st, err = _path_of(cfg, layers, capfd, monkeypatch)
    try:
        assert "whole-stack kernel" in err, err
        gout = run_gpu(st, stream)
        gS, gH = st.get_state()
    finally:
        st.close()
    ref_out, ref_S, ref_H = orc.run(cfg, layers, stream)
    e = max(out_err(gout[:, l], ref_out[:, l]) for l in range(cfg.n_layers))
    es = state_err(gS.cpu().numpy(), ref_S)
    eh = state_err(gH.cpu().numpy(), ref_H) if cfg.conv_k > 1 else 0.0
    print(f"[persist] {name}: out {e:.2e} state {es:.2e} ring {eh:.2e}", flush=True)
    assert e <= OUT_TOL and es <= STATE_TOL and eh <= STATE_TOL


@pytest.mark.parametrize("name", ["p_small", "p_heads48", "p_dim256"])
def test_persist_agrees_with_layer_kernels(name, monkeypatch):
    cfg = PERSIST[name]
    layers, stream = gi.generate(cfg)
    a = make_stack(cfg, layers)
    out_a = run_gpu(a, stream)
    Sa, Ra = a.get_state()
    a.close()
    monkeypatch.setenv("DN_LAYER_KERNELS", "1")
    b = make_stack(cfg, layers)
    monkeypatch.delenv("DN_LAYER_KERNELS")
    out_b = run_gpu(b, stream)
    Sb, Rb = b.get_state()
    b.close()
    for l in range(cfg.n_layers):
        assert out_err(out_a[:, l], out_b[:, l].astype(np.float64)) <= 1e-4
    assert state_err(Sa.cpu().numpy(), Sb.cpu().numpy()) <= 1e-5
    assert state_err(Ra.cpu().numpy(), Rb.cpu().numpy()) <= 1e-5


def test_persist_rerun_bitwise_and_resume():
    cfg = PERSIST["p_full_shape"]
    layers, stream = gi.generate(cfg)
    a = make_stack(cfg, layers)
    full = run_gpu(a, stream)
    Sfull = a.get_state()[0].cpu().numpy()
    a.close()
    b = make_stack(cfg, layers)
    first = run_gpu(b, stream, T=2)
    S, R = b.get_state()
    b.close()
    c = make_stack(cfg, layers)
    c.set_state(S, R)
    rest = run_gpu(c, stream, t0=2)
    Sc = c.get_state()[0].cpu().numpy()
    c.close()
    assert np.array_equal(np.concatenate([first, rest]), full)
    assert np.array_equal(Sc, Sfull)


def test_persist_failed_step_latch(monkeypatch):
    cfg = PERSIST["p_small"]
    layers, stream = gi.generate(cfg)
    monkeypatch.setenv("DN_FAULT_STEP", "3")
    st = make_stack(cfg, layers)
    monkeypatch.delenv("DN_FAULT_STEP")
    try:
        x, al, be = upload_stream(stream)
        for t in range(2):
            st.step(x[t], al[t], be[t])
        assert st.step(x[2], al[2], be[2], check=False) == dn.DN_E_FAULT
        assert st.step(x[2], al[2], be[2], check=False) == dn.DN_E_DISABLED
        gS, gR = st.get_state()
        _, ref_S, ref_H = orc.run(cfg, layers, stream, n_tokens=2)
        assert state_err(gS.cpu().numpy(), ref_S) <= STATE_TOL
        assert state_err(gR.cpu().numpy(), ref_H) <= STATE_TOL
        st.set_state(gS, gR)
        o = st.step(x[2], al[2], be[2])
        torch.cuda.synchronize()
        ref3, _, _ = orc.run(cfg, layers, stream, n_tokens=3)
        assert out_err(o.cpu().numpy()[None, -1], ref3[2:3, -1]) <= OUT_TOL
    finally:
        st.close()
