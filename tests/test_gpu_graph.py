"""dn_step captured in a HIP graph (through torch.cuda.graph) and replayed token by token: every
replay, with eager copies and synchronisations between the replays, gives bit for bit the output
and state of the same tokens run eagerly. One case per execution path: the whole-stack kernel,
the batched kernels and the per-layer kernels. Capture is this library's own concern (callers that
replay a step without host work per token); the pages do not describe it."""
import numpy as np
import pytest
import torch

import dn_inputs as gi

from gpu_util import make_stack, upload_stream

pytestmark = pytest.mark.gpu

CASES = {
    "whole_stack": gi.custom("gr_stack", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=3,
                             n_tokens=6, flags=gi.DN_X_RMSNORM, ring_std=1.0),
    "batched": gi.custom("gr_batched", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, batch=5,
                         n_layers=2, n_tokens=6, ring_std=1.0),
    "per_layer": gi.custom("gr_layer", d_model=512, n_k_heads=2, d_k=64, n_v_heads=4, d_v=64, batch=2,
                           n_layers=2, n_tokens=6, ring_std=1.0),
}
PATHS = {"whole_stack": "whole-stack kernel", "batched": "batched kernels", "per_layer": "per-layer kernels"}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name, capfd, monkeypatch):
    cfg = CASES[name]
    layers, stream = gi.generate(cfg)
    T = cfg.n_tokens
    print(f"[graph] {name}: L={cfg.n_layers} B={cfg.batch} T={T}", flush=True)
    monkeypatch.setenv("DN_VERBOSE", "1")
    st = make_stack(cfg, layers)
    monkeypatch.delenv("DN_VERBOSE")
    assert PATHS[name] in capfd.readouterr().err
    try:
        x, a, b = upload_stream(stream)
        S0, H0 = st.get_state()
        # eager reference
        eager = []
        for t in range(T):
            out = st.new_out()
            st.step(x[t], a[t], b[t], out)
            eager.append(out)
        torch.cuda.synchronize()
        eager = [o.cpu().numpy() for o in eager]
        S_eager, H_eager = (v.cpu().numpy() for v in st.get_state())

        # the same tokens through a captured step
        st.set_state(S0, H0)
        xs, as_, bs = x[0].clone(), a[0].clone(), b[0].clone()
        out_s = st.new_out()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # one eager step on the capture stream before capturing
            st.step(xs, as_, bs, out_s)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        st.set_state(S0, H0)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st.step(xs, as_, bs, out_s)
        torch.cuda.synchronize()
        # capturing does not run the step: the state is still S0
        gS, _ = st.get_state()
        assert torch.equal(gS, S0)
        for t in range(T):
            xs.copy_(x[t])
            as_.copy_(a[t])
            bs.copy_(b[t])
            g.replay()
            torch.cuda.synchronize()
            got = out_s.cpu().numpy()
            assert np.array_equal(got, eager[t]), (name, t, float(np.max(np.abs(got - eager[t]))))
        S_g, H_g = (v.cpu().numpy() for v in st.get_state())
        assert np.array_equal(S_g, S_eager) and np.array_equal(H_g, H_eager)
        del g
    finally:
        st.close()
    print(f"[graph] {name}: {T} replays identical to the eager steps", flush=True)


def test_prefill_graph_replays_match_eager():
    """dn_prefill captured after one eager call of the same length (which sizes the handle's
    scratch), replayed for two prompts from the same starting state: outputs and states bit for
    bit those of eager calls. 8-bit weights, so the capture holds the library GEMMs."""
    cfg = gi.custom("gr_pf", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=2, n_tokens=100,
                    flags=gi.DN_X_RMSNORM, ring_std=1.0)
    layers, stream = gi.generate(cfg)
    T = 100
    print(f"[graph] prefill: L={cfg.n_layers} T={T}", flush=True)
    st = make_stack(cfg, layers)
    try:
        x = torch.from_numpy(np.ascontiguousarray(stream.x[:T, 0])).cuda()
        a = torch.from_numpy(np.ascontiguousarray(stream.alpha[:T, :, 0])).cuda()
        b = torch.from_numpy(np.ascontiguousarray(stream.beta[:T, :, 0])).cuda()
        S0, H0 = st.get_state()
        prompts = [(x, a, b), (x.flip(0).contiguous(), a.flip(0).contiguous(), b.flip(0).contiguous())]
        eager = []
        for px, pa, pb in prompts:
            st.set_state(S0, H0)
            out = st.prefill(px, pa, pb)
            torch.cuda.synchronize()
            eager.append((out.cpu().numpy(), st.get_state()[0].cpu().numpy()))
        xs, as_, bs = x.clone(), a.clone(), b.clone()
        out_s = torch.empty((cfg.n_layers, T, cfg.d_model), device="cuda:0")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            st.prefill(xs, as_, bs, out_s)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st.prefill(xs, as_, bs, out_s)
        torch.cuda.synchronize()
        for i, (px, pa, pb) in enumerate(prompts):
            st.set_state(S0, H0)
            xs.copy_(px)
            as_.copy_(pa)
            bs.copy_(pb)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(out_s.cpu().numpy(), eager[i][0]), i
            assert np.array_equal(st.get_state()[0].cpu().numpy(), eager[i][1]), i
        del g
    finally:
        st.close()
    print("[graph] prefill: 2 replays identical to the eager calls", flush=True)
