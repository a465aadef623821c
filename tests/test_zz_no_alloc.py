"""dn_prefill_noalloc (include/dn_prefill.h), the prompt call that allocates nothing, through the C
ABI on the card: two calls in a row, the second with fewer tokens, each compared with the existing
entry point dn_prefill on a twin handle (same weights, same starting state): bit for bit against
dn_prefill on its default kernels, and within the decode step's bars (output 2e-3 of each token's
rms, state 1e-3 relative Frobenius) against dn_prefill on the library GEMMs. A call whose scratch
would not fit the static array is refused before anything runs."""
import numpy as np
import pytest
import torch

import dn_inputs as gi
import gated_deltanet_layer_dn_amd as dn

from gpu_util import OUT_TOL, STATE_TOL, make_stack, out_err, state_err

pytestmark = pytest.mark.gpu

CASES = {
    # a whole-stack handle of three layers with the stack pre-norm: 150 tokens (three chunks, ragged),
    # then 40
    "stack3": (gi.custom("na_st", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=3,
                         n_tokens=190, flags=gi.DN_X_RMSNORM, ring_std=1.0), (150, 40)),
    # the hybrid-35B layer shape near the scratch's limit: 200 tokens, then 17
    "layer": (gi.custom("na_layer", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128, n_tokens=217,
                        ring_std=1.0), (200, 17)),
}


def _run(cfg, layers, stream, sizes, call):
    st = make_stack(cfg, layers)
    outs, states = [], []
    t0 = 0
    try:
        for T in sizes:
            x = torch.from_numpy(np.ascontiguousarray(stream.x[t0:t0 + T, 0])).cuda()
            a = torch.from_numpy(np.ascontiguousarray(stream.alpha[t0:t0 + T, :, 0])).cuda()
            b = torch.from_numpy(np.ascontiguousarray(stream.beta[t0:t0 + T, :, 0])).cuda()
            out = torch.empty((cfg.n_layers, T, cfg.d_model), device="cuda:0")
            assert call(st.h, x, T, a, b, out) == dn.DN_OK
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
            S, H = st.get_state()
            states.append((S.cpu().numpy(), H.cpu().numpy()))
            t0 += T
    finally:
        st.close()
    return outs, states


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_prefill_matches_dn_prefill(name, monkeypatch):
    cfg, sizes = CASES[name]
    layers, stream = gi.generate(cfg)
    print(f"[noalloc] {name}: calls of {sizes} tokens", flush=True)
    got = _run(cfg, layers, stream, sizes, dn.dn_prefill_noalloc)
    own_gemm = _run(cfg, layers, stream, sizes, dn.dn_prefill)
    monkeypatch.setenv("DN_PREFILL_GEMM", "library")
    lib_gemm = _run(cfg, layers, stream, sizes, dn.dn_prefill)
    monkeypatch.delenv("DN_PREFILL_GEMM")
    for i, T in enumerate(sizes):
        g, r, o = got[0][i], lib_gemm[0][i], own_gemm[0][i]
        assert np.array_equal(g, o), f"call {i}: output differs from dn_prefill on the same kernels"
        assert np.array_equal(got[1][i][0], own_gemm[1][i][0]) and np.array_equal(got[1][i][1], own_gemm[1][i][1])
        e = max(out_err(g[l][:, None, :], r[l][:, None, :].astype(np.float64)) for l in range(cfg.n_layers))
        es = state_err(got[1][i][0], lib_gemm[1][i][0].astype(np.float64))
        eh = state_err(got[1][i][1], lib_gemm[1][i][1].astype(np.float64))
        print(f"[noalloc] {name} call {i} ({T} tokens): against dn_prefill with the library GEMMs: out {e:.2e} "
              f"state {es:.2e} ring {eh:.2e}; bit for bit against dn_prefill", flush=True)
        assert e <= OUT_TOL and es <= STATE_TOL and eh <= STATE_TOL


def test_noalloc_prefill_refuses_a_prompt_beyond_its_scratch(capfd, monkeypatch):
    cfg = gi.custom("na_big", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128, n_tokens=256, ring_std=1.0)
    layers, stream = gi.generate(cfg)
    monkeypatch.setenv("DN_VERBOSE", "1")
    st = make_stack(cfg, layers)
    monkeypatch.delenv("DN_VERBOSE")
    try:
        S0, H0 = (v.cpu().numpy() for v in st.get_state())
        T = 256  # about 73 MiB of scratch at this shape
        x = torch.from_numpy(np.ascontiguousarray(stream.x[:T, 0])).cuda()
        a = torch.from_numpy(np.ascontiguousarray(stream.alpha[:T, :, 0])).cuda()
        b = torch.from_numpy(np.ascontiguousarray(stream.beta[:T, :, 0])).cuda()
        out = torch.empty((1, T, cfg.d_model), device="cuda:0")
        capfd.readouterr()
        assert dn.dn_prefill_noalloc(st.h, x, T, a, b, out) == dn.DN_E_INVAL
        assert "bytes of scratch" in capfd.readouterr().err
        S1, H1 = (v.cpu().numpy() for v in st.get_state())
        assert np.array_equal(S0, S1) and np.array_equal(H0, H1)
        # the handle is still usable, for a prompt that fits
        assert dn.dn_prefill_noalloc(st.h, x[:100], 100, a[:100], b[:100], out[:, :100]) == dn.DN_OK
        torch.cuda.synchronize()
        assert st.status() == dn.DN_OK
    finally:
        st.close()
