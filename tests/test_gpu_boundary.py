"""The C-ABI boundary on the GPU: validation, state movement, resume, the failed-step latch
(page "qwen36: run the DeltaNet layer end to end on the card", sections "What the PR does"
(Tier and Engine paragraphs) and "Verified": get_state works after a failed step and the
CPU continues from the card's state), and that destroy returns device memory."""
import ctypes
import os

import numpy as np
import pytest
import torch

import dn_inputs as gi
import gated_deltanet_layer_dn_amd as dn
import oracle as orc

from gpu_util import OUT_TOL, STATE_TOL, make_stack, out_err, run_gpu, state_err, upload_stream

pytestmark = pytest.mark.gpu

CFG = gi.custom("bnd", d_model=128, n_k_heads=2, d_k=32, n_v_heads=4, d_v=32, n_layers=2, n_tokens=8,
                flags=gi.DN_X_RMSNORM, ring_std=1.0)


def _weights_for(cfg, layers):
    st = dn.DeltaNetStack.from_config(cfg, layers)
    return st


@pytest.mark.parametrize("bad", [
    dict(n_v_heads=65, n_k_heads=1, d_v=16),   # more than 64 value heads
    dict(d_k=257),                              # key dim above 256
    dict(d_v=272),                              # value dim above 256
    dict(n_k_heads=3),                          # Hv not a multiple of Hk
    dict(d_model=100),                          # width not a multiple of 16
    dict(conv_k=5),
    dict(conv_k=0),
    dict(weight_bits=6),
    dict(batch=0),
    dict(flags=8),                              # an undefined flag bit
])
def test_invalid_configs_are_rejected(bad):
    base = dict(d_model=128, n_k_heads=2, d_k=32, n_v_heads=4, d_v=32, conv_k=4, batch=1, n_layers=1,
                weight_bits=8, flags=0, eps_l2=1e-6, eps_rms=1e-6, q_scale=1.0)
    base.update(bad)
    cfg = dn.dn_config(*[base[f] for f, _ in dn.dn_config._fields_])
    good = gi.custom("ok", d_model=128, n_k_heads=2, d_k=32, n_v_heads=4, d_v=32)
    layers, _ = gi.generate(good)
    st = dn.DeltaNetStack.from_config(good, layers)  # valid device weights to point at
    try:
        w = [dn.dn_weights(*[t.data_ptr() for t in st._keep[0]])]
        with pytest.raises(dn.DNError) as ei:
            dn.dn_create(cfg, w)
        assert ei.value.rc == dn.DN_E_INVAL
    finally:
        st.close()


def test_null_and_overlap_are_rejected():
    layers, stream = gi.generate(CFG)
    st = make_stack(CFG, layers)
    try:
        x, a, b = upload_stream(stream)
        out = st.new_out()
        assert dn.dn_step(st.h, None, a[0], b[0], out) == dn.DN_E_INVAL
        # out overlapping x
        buf = torch.zeros((CFG.n_layers + 1) * CFG.d_model, device="cuda:0")
        assert dn.dn_step(st.h, buf[:CFG.d_model], a[0], b[0], buf[CFG.d_model // 2:]) == dn.DN_E_INVAL
        # misaligned weights
        w = [dn.dn_weights(*[t.data_ptr() for t in st._keep[0]]) for _ in range(CFG.n_layers)]
        w[0].w_in += 4
        with pytest.raises(dn.DNError):
            dn.dn_create(st.cfg, w)
    finally:
        st.close()


def test_state_round_trip_is_bitwise():
    layers, _ = gi.generate(CFG)
    st = make_stack(CFG, layers)
    try:
        ss, rs = st.state_shapes()
        rng = np.random.default_rng(5)
        S = rng.standard_normal(ss).astype(np.float32)
        R = rng.standard_normal(rs).astype(np.float32)
        st.set_state(S, R)
        gS, gR = st.get_state()
        assert np.array_equal(gS.cpu().numpy(), S) and np.array_equal(gR.cpu().numpy(), R)
        # host pointers work too
        hS = np.zeros(ss, np.float32); hR = np.zeros(rs, np.float32)
        dn.dn_get_state(st.h, hS.ctypes.data, hR.ctypes.data)
        assert np.array_equal(hS, S) and np.array_equal(hR, R)
    finally:
        st.close()


def test_resume_from_state_is_bitwise():
    """Run 3 tokens, move the state to a fresh handle, run the rest: identical to one run."""
    layers, stream = gi.generate(CFG)
    a = make_stack(CFG, layers)
    full = run_gpu(a, stream)
    a.close()
    b = make_stack(CFG, layers)
    first = run_gpu(b, stream, T=3)
    S, R = b.get_state()
    b.close()
    c = make_stack(CFG, layers)
    c.set_state(S, R)
    rest = run_gpu(c, stream, t0=3)
    c.close()
    assert np.array_equal(np.concatenate([first, rest]), full)


def test_failed_step_latches_and_state_continues_on_cpu(monkeypatch):
    """DN_FAULT_STEP=4 fails the 4th step before any launch. The handle latches off, get_state
    returns the state after 3 tokens, the oracle continues from it, set_state re-arms."""
    layers, stream = gi.generate(CFG)
    monkeypatch.setenv("DN_FAULT_STEP", "4")
    st = make_stack(CFG, layers)
    monkeypatch.delenv("DN_FAULT_STEP")
    try:
        x, al, be = upload_stream(stream)
        outs = [st.step(x[t], al[t], be[t]).cpu().numpy() for t in range(3)]
        assert st.step(x[3], al[3], be[3], check=False) == dn.DN_E_FAULT
        assert st.step(x[3], al[3], be[3], check=False) == dn.DN_E_DISABLED
        gS, gR = st.get_state()
        ref_out, ref_S, ref_H = orc.run(CFG, layers, stream, n_tokens=3)
        assert state_err(gS.cpu().numpy(), ref_S) <= STATE_TOL
        # the CPU continues from what the card holds
        S2, H2 = gS.cpu().numpy().astype(np.float64), gR.cpu().numpy().astype(np.float64)
        tail = gi.Stream(stream.x[3:], stream.alpha[3:], stream.beta[3:])
        cpu_out, _, _ = orc.run(CFG, layers, tail, S=S2, hist=H2)
        ref_full, _, _ = orc.run(CFG, layers, stream)
        assert out_err(cpu_out[:, -1], ref_full[3:, -1]) <= OUT_TOL
        # set_state re-arms the handle
        st.set_state(gS, gR)
        o = st.step(x[3], al[3], be[3])
        torch.cuda.synchronize()
        assert out_err(o.cpu().numpy()[None, -1], ref_full[3:4, -1]) <= OUT_TOL
    finally:
        st.close()


def test_destroy_returns_device_memory():
    cfg = gi.CONFIGS["layer"].replace(batch=64)  # 128 MiB of state
    layers, _ = gi.generate(cfg.replace(batch=1), n_tokens=1)
    torch.cuda.synchronize()
    wts = dn.DeltaNetStack.from_config(cfg.replace(batch=1), layers)
    free0 = torch.cuda.mem_get_info()[0]
    ws = [dn.dn_weights(*[t.data_ptr() for t in wts._keep[0]])]
    c = dn.dn_config(cfg.d_model, cfg.n_k_heads, cfg.d_k, cfg.n_v_heads, cfg.d_v, cfg.conv_k, cfg.batch, 1,
                     8, 0, 1e-6, 1e-6, 1.0)
    for _ in range(3):
        h = dn.dn_create(c, ws)
        assert torch.cuda.mem_get_info()[0] <= free0 - 128 * 2**20
        dn.dn_destroy(h)
        assert torch.cuda.mem_get_info()[0] >= free0 - 4 * 2**20
    wts.close()


def test_stalled_hand_off_aborts_and_the_handle_recovers(capfd, monkeypatch):
    """A whole-stack launch whose exchanges between workgroups get a single poll round
    (DN_FAULT_STALL=2) ends through the kernel's own abort path. It writes into the second state
    buffer, which it does not make current, and the launch enqueued after it does nothing, so the
    card keeps the state after token 1. The status form of dn_get_state reports the failure and
    latches the handle; dn_get_state returns the state after token 1, from which the CPU continues
    exactly; and once dn_set_state has re-armed the handle a run from the initial state matches the
    oracle (no word left by the aborted launch is taken for a fresh one)."""
    cfg = gi.custom("stall", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=6, n_tokens=5,
                    flags=gi.DN_X_RMSNORM, ring_std=1.0)
    layers, stream = gi.generate(cfg)
    monkeypatch.setenv("DN_FAULT_STALL", "2")
    monkeypatch.setenv("DN_VERBOSE", "1")
    st = make_stack(cfg, layers)
    monkeypatch.delenv("DN_FAULT_STALL")
    monkeypatch.delenv("DN_VERBOSE")
    assert "whole-stack kernel" in capfd.readouterr().err
    ref_out, ref_S, ref_H = orc.run(cfg, layers, stream)
    _, ref_S1, ref_H1 = orc.run(cfg, layers, stream, n_tokens=1)
    try:
        x, a, b = upload_stream(stream)
        out = st.new_out()
        print("[stall] step 1, the stalled step 2, and step 3 behind it", flush=True)
        assert st.step(x[0], a[0], b[0], out, check=False) == dn.DN_OK
        assert st.step(x[1], a[1], b[1], out, check=False) == dn.DN_OK  # enqueued; aborts on the card
        rc3 = st.step(x[2], a[2], b[2], out, check=False)  # launched unless the abort was already seen
        assert rc3 in (dn.DN_OK, dn.DN_E_DEVICE)
        assert st.status() == dn.DN_E_DEVICE
        assert st.step(x[2], a[2], b[2], out, check=False) == dn.DN_E_DISABLED
        gS, gH = st.get_state()
        gS, gH = gS.cpu().numpy(), gH.cpu().numpy()
        es1, eh1 = state_err(gS, ref_S1), state_err(gH, ref_H1)
        print(f"[stall] the card holds the state after token 1: state {es1:.2e} ring {eh1:.2e}", flush=True)
        assert es1 <= STATE_TOL and eh1 <= STATE_TOL
        # the CPU continues exactly from what the card holds
        tail = gi.Stream(stream.x[1:], stream.alpha[1:], stream.beta[1:])
        cpu_out, _, _ = orc.run(cfg, layers, tail, S=gS.astype(np.float64), hist=gH.astype(np.float64))
        assert out_err(cpu_out[:, -1], ref_out[1:, -1]) <= OUT_TOL
        print("[stall] abort reported; re-arming from the initial state", flush=True)
        S0 = np.ascontiguousarray(np.stack([l.S0 for l in layers]), np.float32)
        R0 = np.ascontiguousarray(np.stack([l.ring0 for l in layers]), np.float32)
        st.set_state(S0, R0)
        assert st.status() == dn.DN_OK
        gout = run_gpu(st, stream)
        gS, _ = st.get_state()
    finally:
        st.close()
    e, es = out_err(gout, ref_out), state_err(gS.cpu().numpy(), ref_S)
    print(f"[stall] after recovery: out {e:.2e} state {es:.2e}", flush=True)
    assert e <= OUT_TOL and es <= STATE_TOL


def test_status_reports_every_completed_step():
    """dn_get_state with no buffers waits for the device and reports DN_OK while every step
    completed; it copies nothing and leaves the handle usable."""
    layers, stream = gi.generate(CFG)
    st = make_stack(CFG, layers)
    try:
        x, a, b = upload_stream(stream)
        out = st.new_out()
        for t in range(3):
            st.step(x[t], a[t], b[t], out)
        assert st.status() == dn.DN_OK
        hS = np.zeros(st.state_shapes()[1], np.float32)
        assert dn.lib().dn_get_state(st.h, None, hS.ctypes.data) == dn.DN_E_INVAL  # ring without S
        st.step(x[3], a[3], b[3], out)
        assert st.status() == dn.DN_OK
    finally:
        st.close()


@pytest.mark.parametrize("launch", ["ordinary", "cooperative"])
def test_whole_stack_step_shares_the_device_with_other_work(launch, capfd, monkeypatch):
    """The whole-stack kernel needs all of its workgroups resident at once. Launched while another
    stream's kernels occupy the compute units, an ordinary launch's first workgroups wait (within
    their bounded waits) for the rest to be placed as the other kernels drain, and a cooperative
    launch is started by the runtime only when the whole grid fits. Either way each step gives bit
    for bit the result of the same steps on an idle device."""
    cfg = gi.custom("shared", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=2, n_tokens=4,
                    flags=gi.DN_X_RMSNORM, ring_std=1.0)
    layers, stream = gi.generate(cfg)
    monkeypatch.setenv("DN_VERBOSE", "1")
    if launch == "cooperative":
        monkeypatch.setenv("DN_PERSIST_LAUNCH", "cooperative")
    st = make_stack(cfg, layers)
    monkeypatch.delenv("DN_VERBOSE")
    monkeypatch.delenv("DN_PERSIST_LAUNCH", raising=False)
    err = capfd.readouterr().err
    assert f"whole-stack kernel, {launch} launch" in err, err
    try:
        idle = run_gpu(st, stream)
        S0 = np.ascontiguousarray(np.stack([l.S0 for l in layers]), np.float32)
        R0 = np.ascontiguousarray(np.stack([l.ring0 for l in layers]), np.float32)
        st.set_state(S0, R0)
        x, a, b = upload_stream(stream)
        outs = torch.empty((cfg.n_tokens, cfg.n_layers, 1, cfg.d_model), device="cuda:0")
        busy = torch.cuda.Stream()
        A = torch.randn(4096, 4096, device="cuda:0")
        torch.cuda.synchronize()
        print("[shared] steps launched behind another stream's matrix products", flush=True)
        for t in range(cfg.n_tokens):
            with torch.cuda.stream(busy):
                for _ in range(3):
                    A = torch.tanh(A @ A * (1.0 / 64.0))
            st.step(x[t], a[t], b[t], outs[t])
        torch.cuda.synchronize()
        assert st.status() == dn.DN_OK
    finally:
        st.close()
    assert np.array_equal(outs.cpu().numpy(), idle)
