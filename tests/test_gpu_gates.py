"""Gates computed on the card (DN_GATES_ON_DEVICE): alpha and beta of every value head come from
two more in_proj rows, so dn_step and dn_prefill take no gate arrays (NULL is passed). Parity with
the oracle on each execution path (per-layer kernels, batched kernels, whole-stack kernel, prefill
then decode), and the boundary cases of the flag."""
import numpy as np
import pytest
import torch

import dn_inputs as gi
import gated_deltanet_layer_dn_amd as dn
import oracle as orc

from gpu_util import OUT_TOL, STATE_TOL, make_stack, out_err, state_err

pytestmark = pytest.mark.gpu

G = gi.DN_GATES_ON_DEVICE
PRE = gi.DN_X_RMSNORM
CASES = {
    # (config, execution path the handle must take)
    "g_layer_dk64": (gi.custom("g_l64", d_model=512, n_k_heads=4, d_k=64, n_v_heads=8, d_v=64, n_tokens=6,
                               flags=G, ring_std=1.0), "per-layer kernels"),
    "g_layer_b3_int4": (gi.custom("g_l4", d_model=512, n_k_heads=2, d_k=64, n_v_heads=4, d_v=64, batch=3,
                                  n_layers=2, n_tokens=5, weight_bits=4, flags=G | PRE, ring_std=1.0),
                        "per-layer kernels"),
    "g_batched": (gi.custom("g_b", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, batch=8,
                            n_tokens=5, flags=G, ring_std=1.0), "batched kernels"),
    "g_stack": (gi.custom("g_st", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=3,
                          n_tokens=8, flags=G | PRE, ring_std=1.0), "whole-stack kernel"),
    "g_stack_full": (gi.custom("g_full", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128,
                               n_layers=2, n_tokens=5, flags=G | PRE, ring_std=1.0), "whole-stack kernel"),
    "g_stack_full_int4": (gi.custom("g_full4", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128,
                                    n_layers=2, n_tokens=5, weight_bits=4, flags=G | PRE, ring_std=1.0),
                          "whole-stack kernel"),
}


def _make(cfg, layers, capfd, monkeypatch):
    monkeypatch.setenv("DN_VERBOSE", "1")
    st = make_stack(cfg, layers)
    monkeypatch.delenv("DN_VERBOSE")
    return st, capfd.readouterr().err


def _run_no_gates(st, x, t0, T):
    outs = torch.empty((T, st.L, st.B, st.D), dtype=torch.float32, device=st.device)
    for t in range(T):
        st.step(x[t0 + t], None, None, outs[t])
    torch.cuda.synchronize()
    return outs.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_gates_parity(name, capfd, monkeypatch):
    cfg, path = CASES[name]
    layers, stream = gi.generate(cfg)
    print(f"[gates] {name}", flush=True)
    st, err = _make(cfg, layers, capfd, monkeypatch)
    try:
        assert path in err, err
        x = torch.from_numpy(np.ascontiguousarray(stream.x)).cuda()
        gout = _run_no_gates(st, x, 0, x.shape[0])
        gS, gH = st.get_state()
    finally:
        st.close()
    ref_out, ref_S, ref_H = orc.run(cfg, layers, stream)
    e = max(out_err(gout[:, l], ref_out[:, l]) for l in range(cfg.n_layers))
    es = state_err(gS.cpu().numpy(), ref_S)
    eh = state_err(gH.cpu().numpy(), ref_H) if cfg.conv_k > 1 else 0.0
    print(f"[gates] {name}: out {e:.2e} state {es:.2e} ring {eh:.2e}", flush=True)
    assert np.all(np.isfinite(gout))
    assert e <= OUT_TOL and es <= STATE_TOL and eh <= STATE_TOL


def test_gates_prefill_then_decode():
    cfg = gi.custom("g_pf", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=2, n_tokens=104,
                    flags=G | PRE, ring_std=1.0)
    T = 100
    layers, stream = gi.generate(cfg)
    sub = gi.Stream(np.ascontiguousarray(stream.x[:T]), np.ascontiguousarray(stream.alpha[:T]),
                    np.ascontiguousarray(stream.beta[:T]))
    ref_pre, ref_S_pre, _ = orc.run(cfg, layers, sub)
    ref_all, ref_S, _ = orc.run(cfg, layers, stream)
    st = make_stack(cfg, layers)
    try:
        x = torch.from_numpy(np.ascontiguousarray(stream.x[:, 0])).cuda()
        out = st.prefill(x[:T].contiguous())
        torch.cuda.synchronize()
        gS_pre = st.get_state()[0].cpu().numpy()
        xs = torch.from_numpy(np.ascontiguousarray(stream.x)).cuda()
        gdec = _run_no_gates(st, xs, T, stream.x.shape[0] - T)
        gS = st.get_state()[0].cpu().numpy()
    finally:
        st.close()
    gpre = out.cpu().numpy().transpose(1, 0, 2)[:, :, None, :]
    e_pre = max(out_err(gpre[:, l], ref_pre[:, l]) for l in range(cfg.n_layers))
    es_pre = state_err(gS_pre, ref_S_pre)
    e_dec = max(out_err(gdec[:, l], ref_all[T:, l]) for l in range(cfg.n_layers))
    es = state_err(gS, ref_S)
    print(f"[gates] prefill out {e_pre:.2e} state {es_pre:.2e} | decode out {e_dec:.2e} state {es:.2e}", flush=True)
    assert e_pre <= OUT_TOL and es_pre <= STATE_TOL and e_dec <= OUT_TOL and es <= STATE_TOL


def test_gates_boundary():
    base = gi.custom("g_bd", d_model=512, n_k_heads=4, d_k=64, n_v_heads=8, d_v=64, flags=G)
    layers, stream = gi.generate(base)
    # the flag needs the gate parameters
    bare = [gi.Layer(l.w_in, l.s_in, l.conv_w, l.norm_w, l.w_out, l.s_out, l.S0, l.ring0) for l in layers]
    with pytest.raises(dn.DNError) as ei:
        dn.DeltaNetStack.from_config(base, bare)
    assert ei.value.rc == dn.DN_E_INVAL
    # not with a decay per key channel
    with pytest.raises(dn.DNError) as ei:
        dn.DeltaNetStack.from_config(base.replace(flags=G | gi.DN_ALPHA_PER_KEY), layers)
    assert ei.value.rc == dn.DN_E_INVAL
    # without the flag the gate arrays are required
    plain = base.replace(flags=0)
    pl, _ = gi.generate(plain)
    st = make_stack(plain, pl)
    try:
        x = torch.zeros((1, plain.d_model), device="cuda:0")
        assert st.step(x, None, None, check=False) == dn.DN_E_INVAL
        assert st.prefill(x, None, None, check=False) == dn.DN_E_INVAL
    finally:
        st.close()
