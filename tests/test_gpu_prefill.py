"""Prefill (dn_prefill): a prompt of T tokens through the handle on the card, compared element by
element with the oracle run token by token on the same inputs (the chunked recurrence is the
per-token step rewritten, so the bars are the decode step's), then decode continuing from the
prefilled state. Covers prompts of 1 token, shorter than the conv history, ragged chunks, several
chunks, conv widths 1 and 2, int4 weights, no grouped heads, a pre-normed stack, both state layouts
(whole-stack and per-layer handles) and the full layer shape; the 30-layer stack is checked
teacher-forced (each layer fed the oracle's input for that layer)."""
import numpy as np
import pytest
import torch

import dn_inputs as gi
import oracle as orc

from gpu_util import OUT_TOL, STATE_TOL, make_stack, out_err, run_gpu, state_err

pytestmark = pytest.mark.gpu

PF = {
    # (config, prompt length); the config's n_tokens covers the prompt and the decode after it
    "one_token": (gi.custom("pf_one", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_tokens=4,
                            ring_std=1.0), 1),
    "shorter_than_history": (gi.custom("pf_short", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128,
                                       n_tokens=6, ring_std=1.0), 2),
    "ragged_chunks": (gi.custom("pf_rag", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_tokens=104,
                                ring_std=1.0), 100),
    "conv1": (gi.custom("pf_c1", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, conv_k=1, n_tokens=75),
              70),
    "conv2": (gi.custom("pf_c2", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, conv_k=2, n_tokens=75,
                        ring_std=1.0), 70),
    "int4": (gi.custom("pf_i4", d_model=2048, n_k_heads=2, d_k=128, n_v_heads=16, d_v=128, weight_bits=4,
                       n_tokens=84, ring_std=1.0), 80),
    "no_gqa_qscale": (gi.custom("pf_ng", d_model=1024, n_k_heads=8, d_k=128, n_v_heads=8, d_v=128, n_tokens=68,
                                q_scale=0.0883883, ring_std=1.0), 64),
    "stack3_prenorm": (gi.custom("pf_st", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=3,
                                 n_tokens=135, flags=gi.DN_X_RMSNORM, ring_std=1.0), 130),
    # 768-wide model: not a whole-stack shape, so the handle keeps the canonical state layout
    "layer_kernels_handle": (gi.custom("pf_lk", d_model=768, n_k_heads=2, d_k=128, n_v_heads=4, d_v=128,
                                       n_tokens=70, ring_std=1.0), 66),
    # the widest readout (64 value heads x 128 = 8192 columns), normalised and split in one pass
    "widest_values": (gi.custom("pf_wv", d_model=256, n_k_heads=8, d_k=128, n_v_heads=64, d_v=128, n_tokens=70,
                                ring_std=1.0), 66),
    # three sequences, each with its own 70-token prompt, then decode on the batched kernels
    "batch3": (gi.custom("pf_b3", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, batch=3, n_layers=2,
                         n_tokens=74, flags=gi.DN_X_RMSNORM, ring_std=1.0), 70),
}


def _sub(stream, t0, t1):
    return gi.Stream(np.ascontiguousarray(stream.x[t0:t1]), np.ascontiguousarray(stream.alpha[t0:t1]),
                     np.ascontiguousarray(stream.beta[t0:t1]))


def _prompt(stream, T, dev="cuda:0"):
    """x [B][T][D] (one sequence after the other), alpha / beta [T][L][B][Hv]; for one sequence x is
    [T][D] and the gates [T][L][Hv]."""
    B = stream.x.shape[1]
    if B == 1:
        x = np.ascontiguousarray(stream.x[:T, 0])
        a, b = np.ascontiguousarray(stream.alpha[:T, :, 0]), np.ascontiguousarray(stream.beta[:T, :, 0])
    else:
        x = np.ascontiguousarray(stream.x[:T].transpose(1, 0, 2))
        a, b = np.ascontiguousarray(stream.alpha[:T]), np.ascontiguousarray(stream.beta[:T])
    return tuple(torch.from_numpy(v).to(dev) for v in (x, a, b))


def _check_prefill(cfg, T):
    layers, stream = gi.generate(cfg)
    Tall = stream.x.shape[0]
    print(f"[prefill] {cfg.name} L={cfg.n_layers} T={T} then {Tall - T} decode tokens", flush=True)
    ref_pre, ref_S_pre, ref_H_pre = orc.run(cfg, layers, _sub(stream, 0, T))
    ref_all, ref_S, ref_H = orc.run(cfg, layers, stream)
    st = make_stack(cfg, layers)
    try:
        x, a, b = _prompt(stream, T)
        out = torch.empty((cfg.n_layers, cfg.batch, T, cfg.d_model), device="cuda:0")
        st.prefill(x, a, b, out)  # [L][B][T][D]
        torch.cuda.synchronize()
        gS, gH = st.get_state()
        gS_pre, gH_pre = gS.cpu().numpy(), gH.cpu().numpy()
        gdec = run_gpu(st, stream, t0=T) if Tall > T else None
        gS, gH = st.get_state()
    finally:
        st.close()
    gpre = out.cpu().numpy().transpose(2, 0, 1, 3)  # [T][L][B][D]
    assert np.all(np.isfinite(gpre))
    e_pre = max(out_err(gpre[:, l], ref_pre[:, l]) for l in range(cfg.n_layers))
    es = state_err(gS_pre, ref_S_pre)
    eh = state_err(gH_pre, ref_H_pre) if cfg.conv_k > 1 else 0.0
    msg = f"[prefill] {cfg.name}: prompt out {e_pre:.2e} state {es:.2e} ring {eh:.2e}"
    if gdec is not None:
        e_dec = max(out_err(gdec[:, l], ref_all[T:, l]) for l in range(cfg.n_layers))
        es2 = state_err(gS.cpu().numpy(), ref_S)
        msg += f" | decode after it: out {e_dec:.2e} state {es2:.2e}"
    print(msg, flush=True)
    assert e_pre <= OUT_TOL and es <= STATE_TOL and eh <= STATE_TOL
    if gdec is not None:
        assert e_dec <= OUT_TOL and es2 <= STATE_TOL


FUSED_PATH = "in_proj fused int8 GEMM, out_proj fused int8 GEMM after the fused norm-and-split"
LIB_PATH = "in_proj library int8 GEMM, out_proj library int8 GEMM after the fused norm-and-split"
SPLITK_PATH = "in_proj split-K int8 GEMM, out_proj split-K int8 GEMM"


def _check_path(capfd, want):
    err = capfd.readouterr().err
    assert want in err, err


@pytest.mark.parametrize("name", list(PF))
def test_prefill_parity(name, capfd, monkeypatch):
    cfg, T = PF[name]
    monkeypatch.setenv("DN_VERBOSE", "1")
    _check_prefill(cfg, T)
    if cfg.weight_bits == 8:
        # 8-bit weights take the fused int8 GEMMs, with the gated RMSNorm fused into out_proj's split
        _check_path(capfd, FUSED_PATH)


def test_prefill_full_layer(capfd, monkeypatch):
    """The hybrid-35B layer shape: a 320-token prompt (five chunks), then 16 decode tokens."""
    base = gi.CONFIGS["layer"]
    monkeypatch.setenv("DN_VERBOSE", "1")
    _check_prefill(base.replace(name="pf_full", n_tokens=336), 320)
    _check_path(capfd, FUSED_PATH)


def test_prefill_full_stack_teacher_forced():
    """The 30-layer stack, a 200-token prompt: each layer prefilled in its own handle from the
    oracle's input to that layer (the chained stack amplifies rounding by about 1.44x per layer)."""
    cfg = gi.CONFIGS["stack"]
    layers, stream = gi.generate(cfg)
    T, L, D = cfg.n_tokens, cfg.n_layers, cfg.d_model
    ref_out, ref_S, ref_H = orc.run(cfg, layers, stream)
    xin = np.empty((L, T, D), np.float32)
    xin[0] = stream.x[:, 0]
    xin[1:] = ref_out[:, :-1, 0].transpose(1, 0, 2).astype(np.float32)
    a_all = torch.from_numpy(np.ascontiguousarray(stream.alpha[:, :, 0])).cuda()
    b_all = torch.from_numpy(np.ascontiguousarray(stream.beta[:, :, 0])).cuda()
    c1 = cfg.replace(n_layers=1)
    worst = [0.0, 0.0, 0.0]
    for l in range(L):
        st = make_stack(c1, [layers[l]])
        try:
            out = st.prefill(torch.from_numpy(xin[l]).cuda(), a_all[:, l:l + 1].contiguous(), b_all[:, l:l + 1].contiguous())
            torch.cuda.synchronize()
            gS, gH = st.get_state()
        finally:
            st.close()
        e = out_err(out.cpu().numpy()[0][:, None, None, :], ref_out[:, l:l + 1])
        es = state_err(gS.cpu().numpy(), ref_S[l:l + 1])
        eh = state_err(gH.cpu().numpy(), ref_H[l:l + 1])
        worst = [max(worst[0], e), max(worst[1], es), max(worst[2], eh)]
        assert e <= OUT_TOL and es <= STATE_TOL and eh <= STATE_TOL, (l, e, es, eh)
    print(f"[prefill] stack teacher-forced worst over layers: out {worst[0]:.2e} state {worst[1]:.2e} "
          f"ring {worst[2]:.2e}", flush=True)


def test_prefill_rerun_is_bitwise_identical():
    cfg, T = PF["stack3_prenorm"]
    layers, stream = gi.generate(cfg)
    outs, states = [], []
    for _ in range(2):
        st = make_stack(cfg, layers)
        x, a, b = _prompt(stream, T)
        outs.append(st.prefill(x, a, b).cpu().numpy())
        states.append(st.get_state()[0].cpu().numpy())
        st.close()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(states[0], states[1])


def test_prefill_rejects_unsupported_shapes():
    import gated_deltanet_layer_dn_amd as dn
    # a 64-wide head and the per-key decay are not prefill shapes
    for cfg in (gi.custom("pf_d64", d_model=1024, n_k_heads=4, d_k=64, n_v_heads=8, d_v=64),
                gi.custom("pf_pk", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128,
                          flags=gi.DN_ALPHA_PER_KEY)):
        layers, stream = gi.generate(cfg)
        st = make_stack(cfg, layers)
        try:
            T = 4
            x = torch.zeros((T, cfg.d_model), device="cuda:0")
            a = torch.ones((T, 1, cfg.batch * cfg.n_v_heads), device="cuda:0")
            rc = st.prefill(x, a, a, check=False)
            assert rc == dn.DN_E_INVAL, (cfg.name, rc)
            # the handle is still usable
            run_gpu(st, stream, T=1)
        finally:
            st.close()


def test_prefill_arguments_are_checked():
    """An empty or over-long prompt, a NULL input or gate array, and an output overlapping the input are refused
    before anything is launched; the handle then still prefills and matches the oracle."""
    import gated_deltanet_layer_dn_amd as dn
    cfg = gi.custom("pf_args", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=2, n_tokens=4,
                    flags=gi.DN_X_RMSNORM, ring_std=1.0)
    layers, stream = gi.generate(cfg)
    st = make_stack(cfg, layers)
    try:
        T, D, L = 4, cfg.d_model, cfg.n_layers
        x, a, b = _prompt(stream, T)
        out = torch.empty((L, T, D), device="cuda:0")
        for n in (0, -3, dn.DN_PREFILL_MAX_TOKENS + 1):
            assert dn.dn_prefill(st.h, x, n, a, b, out) == dn.DN_E_INVAL
        assert dn.dn_prefill(st.h, None, T, a, b, out) == dn.DN_E_INVAL
        assert dn.dn_prefill(st.h, x, T, None, b, out) == dn.DN_E_INVAL
        assert dn.dn_prefill(st.h, x, T, a, None, out) == dn.DN_E_INVAL
        assert dn.dn_prefill(st.h, x, T, a, b, None) == dn.DN_E_INVAL
        buf = torch.zeros((L + 1) * T * D, device="cuda:0")
        assert dn.dn_prefill(st.h, buf[:T * D], T, a, b, buf[T * D // 2:]) == dn.DN_E_INVAL
        assert dn.dn_prefill(st.h, x, T, a, b, out) == dn.DN_OK
        torch.cuda.synchronize()
        gS, _ = st.get_state()
    finally:
        st.close()
    ref_out, ref_S, _ = orc.run(cfg, layers, stream)
    gpre = out.cpu().numpy().transpose(1, 0, 2)[:, :, None, :]
    assert max(out_err(gpre[:, l], ref_out[:, l]) for l in range(L)) <= OUT_TOL
    assert state_err(gS.cpu().numpy(), ref_S) <= STATE_TOL


@pytest.mark.parametrize("name", ["stack3_prenorm", "ragged_chunks"])
def test_prefill_split_k_gemm(name, capfd, monkeypatch):
    """8-bit weights with the hand-written split-K GEMM (the path of a shape that neither the fused
    GEMM nor the library takes)."""
    monkeypatch.setenv("DN_PREFILL_GEMM", "splitk")
    monkeypatch.setenv("DN_VERBOSE", "1")
    cfg, T = PF[name]
    _check_prefill(cfg, T)
    _check_path(capfd, SPLITK_PATH)


@pytest.mark.parametrize("name", ["stack3_prenorm", "ragged_chunks"])
def test_prefill_library_gemm(name, capfd, monkeypatch):
    """8-bit weights with the library's int8 GEMM over the three terms, folded by the next kernel."""
    monkeypatch.setenv("DN_PREFILL_GEMM", "library")
    monkeypatch.setenv("DN_VERBOSE", "1")
    cfg, T = PF[name]
    _check_prefill(cfg, T)
    _check_path(capfd, LIB_PATH)


def _prefill_outputs(cfg, T, gemm, monkeypatch):
    layers, stream = gi.generate(cfg)
    monkeypatch.setenv("DN_PREFILL_GEMM", gemm)
    st = make_stack(cfg, layers)
    try:
        x, a, b = _prompt(stream, T)
        out = torch.empty((cfg.n_layers, cfg.batch, T, cfg.d_model), device="cuda:0")
        st.prefill(x, a, b, out)
        torch.cuda.synchronize()
        S, H = (v.cpu().numpy() for v in st.get_state())
    finally:
        st.close()
    monkeypatch.delenv("DN_PREFILL_GEMM")
    return out.cpu().numpy(), S, H


@pytest.mark.parametrize("name", ["ragged_chunks", "stack3_prenorm", "layer_kernels_handle", "widest_values",
                                  "batch3", "one_token"])
def test_fused_gemm_equals_library_gemm(name, capfd, monkeypatch):
    """The fused int8 GEMM and the library's sum the same int8 products exactly (int32) and fold the
    three terms with the same double expression, so every output, state and history agree bit for
    bit; ragged token counts, a 768-row out_proj and the 8192-column readout included."""
    cfg, T = PF[name]
    monkeypatch.setenv("DN_VERBOSE", "1")
    fo, fS, fH = _prefill_outputs(cfg, T, "fused", monkeypatch)
    _check_path(capfd, FUSED_PATH)
    lo, lS, lH = _prefill_outputs(cfg, T, "library", monkeypatch)
    _check_path(capfd, LIB_PATH)
    print(f"[prefill] {name}: fused vs library GEMM, max |diff| out {np.abs(fo - lo).max():.3e} "
          f"state {np.abs(fS - lS).max():.3e}", flush=True)
    assert np.array_equal(fo, lo) and np.array_equal(fS, lS) and np.array_equal(fH, lH)
