"""Helpers shared by the GPU tests: run the HIP path through the C ABI and measure errors
against the oracle."""
import numpy as np
import torch

import gated_deltanet_layer_dn_amd as dn

# tolerances of the decode step: out max-abs error relative to each token's output RMS, and
# relative Frobenius error of the final state
OUT_TOL = 2e-3
STATE_TOL = 1e-3


def make_stack(cfg, layers, S0=None, ring0=None, dev="cuda:0"):
    st = dn.DeltaNetStack.from_config(cfg, layers, device=dev)
    S = np.stack([l.S0 for l in layers]) if S0 is None else S0
    R = np.stack([l.ring0 for l in layers]) if ring0 is None else ring0
    st.set_state(np.ascontiguousarray(S, np.float32), np.ascontiguousarray(R, np.float32))
    return st


def upload_stream(stream, T=None, dev="cuda:0"):
    T = stream.x.shape[0] if T is None else T
    x = torch.from_numpy(np.ascontiguousarray(stream.x[:T])).to(dev)
    a = torch.from_numpy(np.ascontiguousarray(stream.alpha[:T])).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(stream.beta[:T])).to(dev)
    return x, a, b


def run_gpu(st, stream, T=None, t0=0):
    """Run tokens t0..t0+T-1; returns out [T][L][B][D] (numpy fp32)."""
    T = stream.x.shape[0] - t0 if T is None else T
    x, a, b = upload_stream(stream, t0 + T)
    outs = torch.empty((T, st.L, st.B, st.D), dtype=torch.float32, device=st.device)
    for t in range(T):
        st.step(x[t0 + t], a[t0 + t], b[t0 + t], outs[t])
    torch.cuda.synchronize()
    return outs.cpu().numpy()


def out_err(gpu, ref):
    """max over tokens of max|gpu - ref| / rms(ref) (per token, over the last axis groups)."""
    g = gpu.reshape(gpu.shape[0], -1).astype(np.float64)
    r = ref.reshape(ref.shape[0], -1)
    rms = np.sqrt(np.mean(r * r, axis=1))
    return float(np.max(np.max(np.abs(g - r), axis=1) / rms))


def state_err(gS, rS):
    """max over (layer, sequence) of ||gS - rS||_F / ||rS||_F."""
    L, B = rS.shape[:2]
    g = np.asarray(gS, np.float64).reshape(L, B, -1)
    r = np.asarray(rS, np.float64).reshape(L, B, -1)
    num = np.linalg.norm(g - r, axis=2)
    den = np.linalg.norm(r, axis=2)
    return float(np.max(num / np.maximum(den, 1e-30)))


def check_layers_fed_from_the_card(cfg, layers, stream, gout, gS, gH):
    """Compare a stack run on the card layer by layer with the oracle's step of that layer fed the
    card's own input to it (x for layer 0, the card's out[l-1] after), the oracle carrying each
    layer's state and history over the tokens. gout [T][L][B][D], gS / gH the card's final state and
    history. Returns the worst (output, state, history) errors over layers: output per token relative
    to its rms, state and history relative Frobenius per layer. The chain's own amplification of
    rounding does not enter: each layer sees exactly the input the card gave it."""
    import oracle as orc
    one = cfg.replace(n_layers=1)
    worst = [0.0, 0.0, 0.0]
    for l, lay in enumerate(layers):
        S = lay.S0.astype(np.float64).copy()
        H = lay.ring0.astype(np.float64).copy()
        refs = np.empty((gout.shape[0],) + gout.shape[2:], np.float64)
        for t in range(gout.shape[0]):
            x = stream.x[t] if l == 0 else gout[t, l - 1]
            refs[t] = orc.layer_step(one, lay, S, H, x.astype(np.float64), stream.alpha[t, l], stream.beta[t, l])
        worst[0] = max(worst[0], out_err(gout[:, l], refs))
        worst[1] = max(worst[1], state_err(gS[l:l + 1], S[None]))
        if cfg.conv_k > 1:
            worst[2] = max(worst[2], state_err(gH[l:l + 1], H[None]))
    return worst
