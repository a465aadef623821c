"""The method's degenerate cases on the card, on every execution path of dn_step and on dn_prefill,
compared element by element with the oracle on the same inputs.

The step (page "qwen36: run the DeltaNet layer end to end on the card", section "What the PR does",
Backend paragraph) decays the state, then applies the delta rule against the decayed state. Its
special cases:
  * alpha = 1, beta = 0: the state does not change at all (compared bit for bit);
  * alpha = 0, beta = 1: the state becomes the outer product of the normalised key and the value;
  * beta = 1: a just-written key reads back its value (the retrieval identity the oracle is pinned on);
  * an all-zero input (the activation split's zero-scale case), a zero state, and both with a zero
    history, where every output and the whole state stay exactly zero;
and for the chunked prompt path, whose recurrence runs on running sums of log decays: strong decays
(alpha in [1e-4, 1e-2] per token) and exact zeros of alpha inside a chunk and on a chunk boundary.
Bars: output max-abs error <= 2e-3 of each token's output rms, state and history <= 1e-3 relative
Frobenius error."""
import numpy as np
import pytest
import torch

import dn_inputs as gi
import oracle as orc

from gpu_util import OUT_TOL, STATE_TOL, make_stack, out_err, run_gpu, state_err

pytestmark = pytest.mark.gpu

# one shape per execution path: 8 value heads of 128 over 4 key heads, d_model 1024, two layers with
# the stack pre-norm; the batched path with three sequences
BASE = dict(d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=2, n_tokens=5,
            flags=gi.DN_X_RMSNORM, ring_std=1.0)
PATHS = {
    "whole-stack kernel": (dict(), None),
    "per-layer kernels": (dict(), "DN_LAYER_KERNELS"),
    "batched kernels": (dict(batch=3), None),
}


def _gates(cfg, case, rng):
    T, L, B, Hv = cfg.n_tokens, cfg.n_layers, cfg.batch, cfg.n_v_heads
    shp = (T, L, B, Hv)
    a = np.exp(-rng.uniform(0.0, 0.1, size=shp))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal(shp)))
    if case == "hold":
        a, b = np.ones(shp), np.zeros(shp)
    elif case == "erase":
        a, b = np.zeros(shp), np.ones(shp)
    elif case == "beta1":
        b = np.ones(shp)
    return a.astype(np.float32), b.astype(np.float32)


def _inputs(cfg, case):
    layers, stream = gi.generate(cfg)
    rng = np.random.default_rng(77)
    a, b = _gates(cfg, case, rng)
    x = stream.x.copy()
    if case in ("zero_input", "all_zero"):
        x[:] = 0.0
    if case in ("zero_state", "all_zero"):
        for lay in layers:
            lay.S0 = np.zeros_like(lay.S0)
    if case == "all_zero":
        for lay in layers:
            lay.ring0 = np.zeros_like(lay.ring0)
    return layers, gi.Stream(x, a, b)


def _err(gpu, ref):
    """out_err over the tokens whose reference output is not zero; where the reference output is
    exactly zero (an all-zero input with a zero history: zero q, k, v and z), the card's output
    must be exactly zero too."""
    g = gpu.reshape(gpu.shape[0], -1)
    r = ref.reshape(ref.shape[0], -1)
    zero = ~np.any(r, axis=1)
    assert not np.any(g[zero]), "non-zero output where the reference output is zero"
    return out_err(gpu[~zero], ref[~zero]) if np.any(~zero) else 0.0


def _open(cfg, layers, env, capfd, monkeypatch):
    monkeypatch.setenv("DN_VERBOSE", "1")
    if env:
        monkeypatch.setenv(env, "1")
    st = make_stack(cfg, layers)
    monkeypatch.delenv("DN_VERBOSE")
    if env:
        monkeypatch.delenv(env)
    return st, capfd.readouterr().err


CASES = ["hold", "erase", "beta1", "zero_input", "zero_state", "all_zero"]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("path", list(PATHS))
def test_step_edge_cases(path, case, capfd, monkeypatch):
    kw, env = PATHS[path]
    cfg = gi.custom("edge_" + case, **{**BASE, **kw})
    layers, stream = _inputs(cfg, case)
    print(f"[edges] {path} / {case}", flush=True)
    st, err = _open(cfg, layers, env, capfd, monkeypatch)
    try:
        assert path in err, err
        gout = run_gpu(st, stream)
        gS, gH = st.get_state()
        gS, gH = gS.cpu().numpy(), gH.cpu().numpy()
    finally:
        st.close()
    S0 = np.stack([l.S0 for l in layers])
    H0 = np.stack([l.ring0 for l in layers])
    if case == "all_zero":
        assert not np.any(gout) and not np.any(gS) and not np.any(gH)
        return
    ref_out, ref_S, ref_H = orc.run(cfg, layers, stream)
    e = max(_err(gout[:, l], ref_out[:, l]) for l in range(cfg.n_layers))
    es, eh = state_err(gS, ref_S), state_err(gH, ref_H)
    print(f"[edges] {path} / {case}: out {e:.2e} state {es:.2e} ring {eh:.2e}", flush=True)
    assert np.all(np.isfinite(gout))
    assert e <= OUT_TOL and es <= STATE_TOL and eh <= STATE_TOL
    if case == "hold":
        assert np.array_equal(gS, S0)  # bit for bit: decay by 1, no delta
        assert np.array_equal(ref_S, S0.astype(np.float64))


# --- prompts ---------------------------------------------------------------------------------

PF_BASE = dict(d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=2, n_tokens=100,
               flags=gi.DN_X_RMSNORM, ring_std=1.0)
PF_CASES = ["hold", "erase", "beta1", "strong_decay", "zero_decay_in_chunk", "zero_input"]


def _pf_gates(cfg, case):
    rng = np.random.default_rng(5)
    a, b = _gates(cfg, case if case in ("hold", "erase", "beta1") else "", rng)
    if case == "strong_decay":
        a = rng.uniform(1e-4, 1e-2, size=a.shape).astype(np.float32)
    elif case == "zero_decay_in_chunk":
        # inside the first chunk, on the first token of the second, and near the prompt's end
        a[[10, 37, 64, 90]] = 0.0
    return a, b


@pytest.mark.parametrize("case", PF_CASES)
@pytest.mark.parametrize("gemm", [None, "library", "splitk"])
def test_prefill_edge_cases(case, gemm, monkeypatch):
    """A 100-token prompt (two chunks, the second ragged), then two decode tokens."""
    cfg = gi.custom("pfedge_" + case, **PF_BASE)
    layers, stream = gi.generate(cfg)
    a, b = _pf_gates(cfg, case)
    x = stream.x.copy()
    if case == "zero_input":
        x[:] = 0.0
    stream = gi.Stream(x, a, b)
    T = 98
    print(f"[edges] prefill ({gemm or 'default'} GEMM) / {case}", flush=True)
    ref_all, ref_S, ref_H = orc.run(cfg, layers, stream)
    _, ref_S_pre, ref_H_pre = orc.run(cfg, layers, stream, n_tokens=T)
    if gemm:
        monkeypatch.setenv("DN_PREFILL_GEMM", gemm)
    st = make_stack(cfg, layers)
    try:
        xp = torch.from_numpy(np.ascontiguousarray(x[:T, 0])).cuda()
        ap = torch.from_numpy(np.ascontiguousarray(a[:T, :, 0])).cuda()
        bp = torch.from_numpy(np.ascontiguousarray(b[:T, :, 0])).cuda()
        out = torch.empty((cfg.n_layers, T, cfg.d_model), device="cuda:0")
        st.prefill(xp, ap, bp, out)
        torch.cuda.synchronize()
        gS_pre, gH_pre = (v.cpu().numpy() for v in st.get_state())
        gdec = run_gpu(st, stream, t0=T)
        gS, gH = (v.cpu().numpy() for v in st.get_state())
    finally:
        st.close()
    gpre = out.cpu().numpy().transpose(1, 0, 2)[:, :, None]  # [T][L][1][D]
    assert np.all(np.isfinite(gpre)) and np.all(np.isfinite(gdec))
    e_pre = max(_err(gpre[:, l], ref_all[:T, l]) for l in range(cfg.n_layers))
    e_dec = max(_err(gdec[:, l], ref_all[T:, l]) for l in range(cfg.n_layers))
    es_pre, eh_pre = state_err(gS_pre, ref_S_pre), state_err(gH_pre, ref_H_pre)
    es, eh = state_err(gS, ref_S), state_err(gH, ref_H)
    print(f"[edges] prefill / {case}: prompt out {e_pre:.2e} state {es_pre:.2e} ring {eh_pre:.2e}; "
          f"decode out {e_dec:.2e} state {es:.2e} ring {eh:.2e}", flush=True)
    assert max(e_pre, e_dec) <= OUT_TOL
    assert max(es_pre, eh_pre, es, eh) <= STATE_TOL
    if case == "hold":
        assert np.array_equal(gS_pre, np.stack([l.S0 for l in layers]))
