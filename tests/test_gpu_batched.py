"""The batched path (B >= 2 sequences with 128 x 128 state tiles: int8-MFMA projections, streaming
state kernel): parity with the oracle per sequence, ragged batches (a partial block of 64
sequences), int4 weights, conv widths, a pre-normed stack, K ranges of 1024 / 512 / 256 columns,
agreement with the per-layer kernels and bitwise reruns. The in_proj runs as the split-K GEMM with a
separate epilogue, or (shapes with at least 48 x 256 rows, or every supported shape under
DN_BPROJ=1) as one whole-K kernel that ends in the epilogue; both are checked."""
import numpy as np
import pytest

import dn_inputs as gi
import oracle as orc

from gpu_util import OUT_TOL, STATE_TOL, make_stack, out_err, run_gpu, state_err

pytestmark = pytest.mark.gpu

BATCHED = {
    # d_model 1024: in_proj K range 1024 (one split), out_proj 512
    "b_small": gi.custom("b_small", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, batch=8,
                         n_tokens=6, ring_std=1.0),
    # 70 sequences: a full block of 64 and a ragged block of 6
    "b_ragged": gi.custom("b_ragged", d_model=512, n_k_heads=2, d_k=128, n_v_heads=4, d_v=128, batch=70,
                          n_tokens=4, ring_std=1.0),
    "b_int4": gi.custom("b_int4", d_model=2048, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, batch=16,
                        n_tokens=5, weight_bits=4, ring_std=1.0),
    "b_conv1": gi.custom("b_conv1", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, batch=4,
                         conv_k=1, n_tokens=4),
    "b_conv2": gi.custom("b_conv2", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, batch=3,
                         conv_k=2, n_tokens=4, ring_std=1.0),
    # 768-wide model and 768 value columns: 256-column K ranges; in_proj rows 2304 (18 blocks of 128)
    "b_odd": gi.custom("b_odd", d_model=768, n_k_heads=3, d_k=128, n_v_heads=6, d_v=128, batch=5,
                       n_tokens=4, q_scale=0.0883883),
    # three pre-normed layers, each output feeding the next layer
    "b_stack": gi.custom("b_stack", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, batch=6,
                         n_layers=3, n_tokens=5, flags=gi.DN_X_RMSNORM, ring_std=1.0),
    # one decay per key channel, alpha [B][Hv][128]
    "b_perkey": gi.custom("b_perkey", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, batch=5,
                          n_tokens=5, flags=gi.DN_ALPHA_PER_KEY, ring_std=1.0),
    # 48 value heads of 128 over 16 key heads: in_proj 16384 rows, out_proj K = 6144
    "b_heads48": gi.custom("b_heads48", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=48, d_v=128, batch=4,
                           n_tokens=3, ring_std=1.0),
    # the stack's layer shape (in_proj 12288 rows: the whole-K kernel by default), pre-normed, 70
    # sequences (a full block of 64 and a ragged block of 6)
    "b_wide": gi.custom("b_wide", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128, batch=70,
                        n_tokens=2, flags=gi.DN_X_RMSNORM, ring_std=1.0),
}
# shapes whose in_proj also runs through the whole-K kernel when forced (8-bit weights, K of 1024 or
# 2048); b_int4 stays on the split-K GEMM
WHOLE_K = ["b_small", "b_int4", "b_conv1", "b_conv2", "b_stack", "b_perkey"]


def _in_rows(cfg):
    return 2 * cfg.n_k_heads * cfg.d_k + 2 * cfg.n_v_heads * cfg.d_v


def _path_of(cfg, layers, capfd, monkeypatch):
    monkeypatch.setenv("DN_VERBOSE", "1")
    st = make_stack(cfg, layers)
    monkeypatch.delenv("DN_VERBOSE")
    return st, capfd.readouterr().err


def _per_seq_out_err(gout, ref):
    """max over layers and sequences of the per-token error relative to that sequence's RMS."""
    T, L, B, D = ref.shape
    return max(out_err(gout[:, l, b], ref[:, l, b]) for l in range(L) for b in range(B))


CASES = [(n, None) for n in BATCHED] + [(n, "1") for n in WHOLE_K]


@pytest.mark.parametrize("name,bproj", CASES)
def test_batched_parity(name, bproj, capfd, monkeypatch):
    cfg = BATCHED[name]
    layers, stream = gi.generate(cfg)
    print(f"[batched] {name} (DN_BPROJ={bproj})", flush=True)
    if bproj:
        monkeypatch.setenv("DN_BPROJ", bproj)
    st, err = _path_of(cfg, layers, capfd, monkeypatch)
    if bproj:
        monkeypatch.delenv("DN_BPROJ")
    try:
        assert "batched kernels" in err, err
        whole_k = cfg.weight_bits == 8 and (bproj or (_in_rows(cfg) >= 48 * 256 and cfg.d_model in (1024, 2048)))
        assert ("in_proj whole-K" if whole_k else "in_proj split-K") in err, err
        gout = run_gpu(st, stream)
        gS, gH = st.get_state()
    finally:
        st.close()
    ref_out, ref_S, ref_H = orc.run(cfg, layers, stream)
    e = _per_seq_out_err(gout, ref_out)
    es = state_err(gS.cpu().numpy(), ref_S)
    eh = state_err(gH.cpu().numpy(), ref_H) if cfg.conv_k > 1 else 0.0
    print(f"[batched] {name} (DN_BPROJ={bproj}): out {e:.2e} state {es:.2e} ring {eh:.2e}", flush=True)
    assert e <= OUT_TOL and es <= STATE_TOL and eh <= STATE_TOL


def test_batched_agrees_with_layer_kernels(monkeypatch):
    cfg = BATCHED["b_stack"]
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
    assert _per_seq_out_err(out_a, out_b.astype(np.float64)) <= 1e-4
    assert state_err(Sa.cpu().numpy(), Sb.cpu().numpy()) <= 1e-5
    assert state_err(Ra.cpu().numpy(), Rb.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("name", ["b_ragged", "b_wide"])
def test_batched_rerun_bitwise(name):
    """Split-K partial sums, and the whole-K kernel's K quarters, are added in a fixed order (whatever
    order the staged weight chunks land in): two runs are byte-identical."""
    cfg = BATCHED[name]
    layers, stream = gi.generate(cfg)
    outs, states = [], []
    for _ in range(2):
        st = make_stack(cfg, layers)
        outs.append(run_gpu(st, stream))
        states.append(st.get_state()[0].cpu().numpy())
        st.close()
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(states[0], states[1])
