"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
exact integer arithmetic, brute-force convolution with numpy, closed forms of the
recurrence, identities of SiLU and of the norms. Each step of the decode token
(page "qwen36: run the DeltaNet layer end to end on the card", section "What the
PR does") has at least one pin here that a dropped term, a wrong sign or index, or
a transposed operand would fail.
"""
import numpy as np
import pytest

import dn_inputs as gi
import oracle as orc


RNG = np.random.default_rng(12345)


# --------------------------------------------------------------------------- GEMV

def test_gemv_exact_on_integer_inputs():
    W = RNG.integers(-127, 128, size=(37, 96), dtype=np.int8)
    x = RNG.integers(-2, 3, size=96).astype(np.float64)
    ones = np.ones(37, np.float32)
    y = orc.gemv(W, ones, x)
    assert np.array_equal(y, (W.astype(np.int64) @ x.astype(np.int64)).astype(np.float64))


def test_gemv_scale_applies_after_the_sum():
    W = RNG.integers(-127, 128, size=(19, 64), dtype=np.int8)
    x = RNG.integers(-2, 3, size=64).astype(np.float64)
    s = RNG.uniform(0.005, 0.02, size=19).astype(np.float32)
    y = orc.gemv(W, s, x)
    # s (24-bit mantissa) times an integer below 2^17 is exact in double
    assert np.array_equal(y, s.astype(np.float64) * (W.astype(np.int64) @ x.astype(np.int64)))


def test_gemv_matches_float64_matmul():
    W = RNG.integers(-127, 128, size=(50, 300), dtype=np.int8)
    x = RNG.standard_normal(300)
    s = RNG.uniform(0.005, 0.02, size=50).astype(np.float32)
    y = orc.gemv(W, s, x)
    ref = s.astype(np.float64) * (W.astype(np.float64) @ x)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_int4_nibble_order_and_sign():
    # byte 0x9F: low nibble 0xF = -1 is element 0, high nibble 0x9 = -7 is element 1
    W = np.array([[0x9F, 0x70]], dtype=np.uint8)
    assert orc.weight(W, 4, 4, 0, 0) == -1
    assert orc.weight(W, 4, 4, 0, 1) == -7
    assert orc.weight(W, 4, 4, 0, 2) == 0
    assert orc.weight(W, 4, 4, 0, 3) == 7


def test_int4_gemv_equals_int8_gemv_of_the_unpacked_values():
    vals = RNG.integers(-7, 8, size=(33, 128), dtype=np.int8)
    packed = gi.pack_int4(vals)
    x = RNG.standard_normal(128)
    s = RNG.uniform(0.005, 0.02, size=33).astype(np.float32)
    assert np.array_equal(orc.gemv(packed, s, x, bits=4), orc.gemv(vals, s, x, bits=8))
    xi = RNG.integers(-2, 3, size=128).astype(np.float64)
    y = orc.gemv(packed, np.ones(33, np.float32), xi, bits=4)
    assert np.array_equal(y, (vals.astype(np.int64) @ xi.astype(np.int64)).astype(np.float64))


# --------------------------------------------------------------------------- SiLU

def test_silu_identities():
    assert orc.silu(0.0) == 0.0
    for a in [-30.0, -3.5, -1.0, -1e-3, 1e-3, 0.5, 1.0, 2.0, 7.0, 30.0]:
        s, t = orc.silu(a), orc.silu(-a)
        assert abs((s - t) - a) <= 1e-15 * max(1.0, abs(a))            # odd part is x/2 each
        assert abs((s + t) - a * np.tanh(a / 2)) <= 1e-14 * max(1.0, abs(a))  # even part
    assert abs(orc.silu(40.0) - 40.0) < 1e-15 * 40 * 1e3
    assert abs(orc.silu(-40.0)) < 1e-15


# --------------------------------------------------------------------------- conv

def _brute_conv(w, hist0, useq):
    """Pre-activation conv outputs by np.convolve over [history, tokens]."""
    C, K = w.shape
    full = np.concatenate([hist0, useq], axis=0)  # [(K-1)+T][C]
    T = useq.shape[0]
    pre = np.zeros((T, C))
    for c in range(C):
        # full convolution with reversed taps: y[n] = sum_j w[c][j] * full[n-(K-1)+j]
        y = np.convolve(full[:, c], w[c][::-1].astype(np.float64))
        pre[:, c] = y[(K - 1) + np.arange(T)]
    return pre


def _silu_np(a):
    # silu written through tanh, a different route than the oracle's exp form
    return 0.5 * a * (1.0 + np.tanh(0.5 * a))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("zero_hist", [True, False])
def test_conv_matches_bruteforce(K, zero_hist):
    C, T = 7, 11
    w = RNG.uniform(-0.5, 0.5, size=(C, K)).astype(np.float32)
    hist0 = np.zeros((K - 1, C)) if zero_hist else RNG.standard_normal((K - 1, C))
    useq = RNG.standard_normal((T, C)) * 3
    pre = _brute_conv(w, hist0, useq)
    hist = hist0.copy()
    for t in range(T):
        out, hist = orc.conv_silu(w, hist, useq[t])
        np.testing.assert_allclose(out, _silu_np(pre[t]), rtol=1e-13, atol=1e-13)
    # the history holds the last K-1 tokens, oldest first
    full = np.concatenate([hist0, useq], axis=0)
    np.testing.assert_array_equal(hist.reshape(K - 1, C), full[full.shape[0] - (K - 1):])


def test_conv_impulse_returns_reversed_taps_and_identity_taps():
    C, K = 3, 4
    w = RNG.uniform(-0.5, 0.5, size=(C, K)).astype(np.float32)
    hist = np.zeros((K - 1, C))
    # impulse of height 1e-9: silu(a) ~ a/2 for tiny a, so out*2 recovers the pre-activation
    seq = [np.full(C, 1e-9)] + [np.zeros(C)] * (K - 1)
    outs = []
    for u in seq:
        o, hist = orc.conv_silu(w, hist, u)
        outs.append(o)
    pre = np.array(outs) * 2 / 1e-9
    np.testing.assert_allclose(pre, w[:, ::-1].T.astype(np.float64), rtol=1e-8, atol=1e-12)
    # taps e_{K-1}: out = silu(u)
    w_id = np.zeros((C, K), np.float32); w_id[:, K - 1] = 1
    u = np.array([-2.0, 0.0, 3.0])
    o, _ = orc.conv_silu(w_id, RNG.standard_normal((K - 1, C)), u)
    np.testing.assert_allclose(o, [orc.silu(-2.0), 0.0, orc.silu(3.0)], rtol=0, atol=0)


# --------------------------------------------------------------------------- norms

def test_l2norm_eps_inside_the_sqrt():
    for n in [16, 128]:
        v = RNG.standard_normal(n) * 0.01
        ss = float(np.dot(v, v))
        for eps in [0.0, 1e-6, 1e-3]:
            vh = orc.l2norm(v, eps)
            assert abs(np.dot(vh, vh) - ss / (ss + eps)) <= 1e-14
            # direction is kept: vh * sqrt(ss + eps) recovers v
            np.testing.assert_allclose(vh * np.sqrt(ss + eps), v, rtol=1e-14, atol=0)
    z = orc.l2norm(np.zeros(8), 1e-6)
    assert np.all(z == 0)


def test_rms_prenorm():
    x = RNG.standard_normal(2048) * 40
    y = orc.rms_prenorm(x, 1e-6)
    m = np.mean(x * x)
    assert abs(np.sqrt(np.mean(y * y)) - np.sqrt(m / (m + 1e-6))) < 1e-14
    np.testing.assert_allclose(y / x, np.full_like(x, y[0] / x[0]), rtol=1e-13)


def test_gated_rmsnorm_scale_invariance_and_gate():
    dv = 32
    o = RNG.standard_normal(dv)
    z = RNG.standard_normal(dv) * 3
    w = RNG.uniform(0.5, 1.5, size=dv).astype(np.float32)
    y0 = orc.gated_rmsnorm(o, z, w, 0.0)
    for c in [1e-3, 7.0, -2.0]:
        yc = orc.gated_rmsnorm(c * o, z, w, 0.0)
        np.testing.assert_allclose(yc, np.sign(c) * y0, rtol=1e-13, atol=1e-15)
    # w = 1 and a large z (silu(z) ~ z): rms(y / z) = sqrt(m / (m + eps))
    ones = np.ones(dv, np.float32)
    zz = np.full(dv, 50.0)
    eps = 0.3
    y = orc.gated_rmsnorm(o, zz, ones, eps)
    m = np.mean(o * o)
    assert abs(np.sqrt(np.mean((y / orc.silu(50.0)) ** 2)) - np.sqrt(m / (m + eps))) < 1e-13
    # the gate zeroes where z = 0
    zg = z.copy(); zg[::3] = 0
    yg = orc.gated_rmsnorm(o, zg, w, 1e-6)
    assert np.all(yg[::3] == 0)


# --------------------------------------------------------------------------- recurrence

def _unit(v):
    return v / np.linalg.norm(v)


def test_delta_beta0_alpha1_keeps_state_bitwise():
    S = RNG.standard_normal((16, 24))
    S1, o = orc.delta_head(S, _unit(RNG.standard_normal(16)), RNG.standard_normal(24),
                           _unit(RNG.standard_normal(16)), 1.0, 0.0)
    assert np.array_equal(S1, S)


def test_delta_alpha0_beta1_writes_outer_product():
    S = RNG.standard_normal((16, 24))
    k = _unit(RNG.standard_normal(16)); v = RNG.standard_normal(24)
    S1, _ = orc.delta_head(S, k, v, k, 0.0, 1.0)
    np.testing.assert_allclose(S1, np.outer(k, v), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("dk,dv", [(16, 16), (128, 128), (32, 48)])
def test_delta_rule_retrieval_identity(dk, dv):
    for _ in range(5):
        S = RNG.standard_normal((dk, dv)) * 0.3
        k = RNG.standard_normal(dk); k = k / np.sqrt(k @ k + 1e-6)
        v = RNG.standard_normal(dv)
        q = k.copy()
        alpha = float(np.exp(-RNG.uniform(0, 0.1))); beta = float(1 / (1 + np.exp(-RNG.standard_normal())))
        S1, o = orc.delta_head(S, k, v, q, alpha, beta, q_scale=1.0)
        kk = float(k @ k)
        Sd = alpha * S
        lhs = S1.T @ k
        rhs = (1 - beta * kk) * (Sd.T @ k) + beta * kk * v
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
        # the readout uses the updated state: with q = k it is the same vector
        np.testing.assert_allclose(o, lhs, rtol=1e-12, atol=1e-12)
        # S'' - S' is the rank-1 update k d^T with d = beta (v - S'^T k)
        d = beta * (v - Sd.T @ k)
        np.testing.assert_allclose(S1 - Sd, np.outer(k, d), rtol=1e-11, atol=1e-12)


def test_readout_is_linear_in_q_and_scaled():
    dk, dv = 16, 16
    S = RNG.standard_normal((dk, dv)); k = _unit(RNG.standard_normal(dk)); v = RNG.standard_normal(dv)
    q1 = RNG.standard_normal(dk); q2 = RNG.standard_normal(dk)
    Sa, o1 = orc.delta_head(S, k, v, q1, 0.9, 0.4)
    _, o2 = orc.delta_head(S, k, v, q2, 0.9, 0.4)
    _, o12 = orc.delta_head(S, k, v, 2 * q1 - q2, 0.9, 0.4, q_scale=0.5)
    np.testing.assert_allclose(o12, 0.5 * (2 * o1 - o2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o1, Sa.T @ q1, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------- whole layer

def _tiny_layer(**kw):
    cfg = gi.CONFIGS["tiny"].replace(**kw)
    layers, stream = gi.generate(cfg)
    return cfg, layers[0], stream


def _np_front(cfg, lay, x, hist):
    """in_proj and conv by numpy (matmul + np.convolve), pre-activation and post."""
    u = lay.s_in.astype(np.float64) * (lay.w_in_vals.astype(np.float64) @ x)
    C = cfg.conv_channels
    full = np.concatenate([hist, u[None, :C]], axis=0)
    K = cfg.conv_k
    pre = np.array([np.convolve(full[:, c], lay.conv_w[c][::-1].astype(np.float64))[K - 1 + (full.shape[0] - K)]
                    for c in range(C)])
    return u, _silu_np(pre)


@pytest.mark.parametrize("q_scale", [1.0, 0.25])
def test_layer_alpha0_closed_form(q_scale):
    """With alpha = 0 the state is beta k v^T after one step, so out follows from the front
    of the layer alone: o = c v with c = q_scale beta (q.k), y = w c v / sqrt(c^2 mean v^2 + eps) silu(z)."""
    cfg, lay, stream = _tiny_layer(q_scale=q_scale)
    Hk, Hv, dk, dv = cfg.n_k_heads, cfg.n_v_heads, cfg.d_k, cfg.d_v
    S = RNG.standard_normal((1, Hv, dk, dv))
    hist = RNG.standard_normal((1, cfg.conv_k - 1, cfg.conv_channels))
    x = stream.x[0].astype(np.float64)
    alpha = np.zeros((1, Hv), np.float32)
    beta = stream.beta[0, 0]
    u, c = _np_front(cfg, lay, x[0], hist[0])
    out = orc.layer_step(cfg, lay, S, hist, x, alpha, beta)
    QK = Hk * dk
    y = np.zeros(Hv * dv)
    for h in range(Hv):
        g = h // (Hv // Hk)
        q = c[g * dk:(g + 1) * dk]; k = c[QK + g * dk:QK + (g + 1) * dk]
        qh = q / np.sqrt(q @ q + cfg.eps_l2); kh = k / np.sqrt(k @ k + cfg.eps_l2)
        v = c[2 * QK + h * dv:2 * QK + (h + 1) * dv]
        z = u[cfg.conv_channels + h * dv:cfg.conv_channels + (h + 1) * dv]
        cc = q_scale * float(beta[0, h]) * float(qh @ kh)
        y[h * dv:(h + 1) * dv] = lay.norm_w.astype(np.float64) * cc * v / np.sqrt(cc * cc * np.mean(v * v) + cfg.eps_rms) * _silu_np(z)
        np.testing.assert_allclose(S[0, h], float(beta[0, h]) * np.outer(kh, v), rtol=1e-12, atol=1e-14)
    ref = lay.s_out.astype(np.float64) * (lay.w_out_vals.astype(np.float64) @ y)
    np.testing.assert_allclose(out[0], ref, rtol=1e-10, atol=1e-10 * np.max(np.abs(ref)))


def test_layer_beta0_alpha1_state_constant_and_readout():
    cfg, lay, stream = _tiny_layer()
    Hv = cfg.n_v_heads
    S0 = RNG.standard_normal((1, Hv, cfg.d_k, cfg.d_v))
    S = S0.copy()
    hist = np.zeros((1, cfg.conv_k - 1, cfg.conv_channels))
    for t in range(3):
        orc.layer_step(cfg, lay, S, hist, stream.x[t].astype(np.float64), np.ones((1, Hv), np.float32),
                       np.zeros((1, Hv), np.float32))
    assert np.array_equal(S, S0)
    # history = last K-1 pre-conv inputs (oldest first), each being s_in * W_in x
    for j, t in enumerate(range(3 - (cfg.conv_k - 1), 3)):
        u = lay.s_in.astype(np.float64) * (lay.w_in_vals.astype(np.float64) @ stream.x[t, 0].astype(np.float64))
        np.testing.assert_allclose(hist[0, j], u[:cfg.conv_channels], rtol=1e-12, atol=1e-12)


def test_run_chains_layers_and_applies_prenorm():
    cfg = gi.custom("chain", d_model=64, n_k_heads=2, d_k=16, n_v_heads=4, d_v=16, n_layers=3, n_tokens=3,
                    flags=gi.DN_X_RMSNORM, ring_std=1.0)
    layers, stream = gi.generate(cfg)
    out, S, H = orc.run(cfg, layers, stream)
    S2, H2 = orc.initial_state(layers)
    for t in range(3):
        x = stream.x[t].astype(np.float64)
        for l in range(3):
            o = orc.layer_step(cfg.replace(n_layers=1), layers[l], S2[l], H2[l], x,
                               stream.alpha[t, l], stream.beta[t, l])
            np.testing.assert_array_equal(o, out[t, l])
            x = o
    # prenorm: with eps = 0, scaling the input of a layer by c > 0 leaves its output unchanged
    l0 = layers[0]
    Sa, Ha = orc.initial_state([l0])
    Sb, Hb = orc.initial_state([l0])
    c1 = cfg.replace(n_layers=1, eps_rms=0.0)
    oa = orc.layer_step(c1, l0, Sa[0], Ha[0], stream.x[0].astype(np.float64), stream.alpha[0, 0], stream.beta[0, 0])
    ob = orc.layer_step(c1, l0, Sb[0], Hb[0], 1000 * stream.x[0].astype(np.float64), stream.alpha[0, 0],
                        stream.beta[0, 0])
    np.testing.assert_allclose(oa, ob, rtol=1e-11, atol=1e-11 * np.max(np.abs(oa)))


def test_stack_without_prenorm_grows_per_layer():
    """Why the stack normalises layer inputs: without it the output grows ~1e3x per layer."""
    cfg = gi.CONFIGS["stack"].replace(d_model=256, n_k_heads=2, n_v_heads=4, flags=0, n_layers=3,
                                      layer_seeds=(7, 8, 9), stream_seed=10)
    layers, stream = gi.generate(cfg, n_tokens=1)
    out, _, _ = orc.run(cfg, layers, stream)
    r = [np.sqrt(np.mean(out[0, l] ** 2)) for l in range(3)]
    assert r[1] / r[0] > 50 and r[2] / r[1] > 50


# --------------------------------------------------------------------------- decay per key channel

def test_per_key_decay_with_equal_entries_is_the_scalar_step_bitwise():
    dk, dv = 32, 24
    S = RNG.standard_normal((dk, dv)); k = _unit(RNG.standard_normal(dk)); v = RNG.standard_normal(dv)
    q = _unit(RNG.standard_normal(dk))
    S1, o1 = orc.delta_head(S, k, v, q, 0.93, 0.6, q_scale=0.7)
    S2, o2 = orc.delta_head_vec(S, k, v, q, np.full(dk, 0.93), 0.6, q_scale=0.7)
    assert np.array_equal(S1, S2) and np.array_equal(o1, o2)


def test_per_key_decay_scales_key_rows():
    """beta = 0: the step is the decay alone, S'[i][j] = alpha[i] S[i][j]; a one-hot alpha keeps one
    key row and zeroes the rest (rows, not columns)."""
    dk, dv = 16, 24
    S = RNG.standard_normal((dk, dv)); k = _unit(RNG.standard_normal(dk)); v = RNG.standard_normal(dv)
    a = np.zeros(dk); a[5] = 1.0
    S1, o = orc.delta_head_vec(S, k, v, k, a, 0.0)
    assert np.array_equal(S1[5], S[5]) and not np.any(np.delete(S1, 5, axis=0))
    np.testing.assert_allclose(o, k[5] * S[5], rtol=1e-14, atol=1e-15)
    S1, _ = orc.delta_head_vec(S, k, v, k, np.ones(dk), 0.0)
    assert np.array_equal(S1, S)
    S1, _ = orc.delta_head_vec(S, k, v, k, np.zeros(dk), 1.0)
    np.testing.assert_allclose(S1, np.outer(k, v), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("dk,dv", [(16, 16), (128, 128), (64, 32)])
def test_per_key_delta_rule_retrieval_identity(dk, dv):
    for _ in range(5):
        S = RNG.standard_normal((dk, dv)) * 0.3
        k = RNG.standard_normal(dk); k = k / np.sqrt(k @ k + 1e-6)
        v = RNG.standard_normal(dv)
        a = np.exp(-RNG.uniform(0, 0.5, size=dk)); beta = float(1 / (1 + np.exp(-RNG.standard_normal())))
        S1, o = orc.delta_head_vec(S, k, v, k, a, beta)
        kk = float(k @ k)
        Sd = S * a[:, None]
        np.testing.assert_allclose(S1.T @ k, (1 - beta * kk) * (Sd.T @ k) + beta * kk * v, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(o, S1.T @ k, rtol=1e-12, atol=1e-12)


def test_per_key_run_with_constant_rows_equals_scalar_run():
    base = gi.custom("pk_eq", d_model=64, n_k_heads=2, d_k=16, n_v_heads=4, d_v=16, n_layers=2, n_tokens=3,
                     flags=gi.DN_X_RMSNORM, ring_std=1.0)
    layers, stream = gi.generate(base)
    out1, S1, H1 = orc.run(base, layers, stream)
    pk = base.replace(flags=gi.DN_X_RMSNORM | gi.DN_ALPHA_PER_KEY)
    a = np.ascontiguousarray(np.repeat(stream.alpha[..., None], base.d_k, axis=-1))
    out2, S2, H2 = orc.run(pk, layers, gi.Stream(stream.x, a, stream.beta))
    assert np.array_equal(out1, out2) and np.array_equal(S1, S2) and np.array_equal(H1, H2)


def test_per_key_run_decay_only_closed_form():
    """beta = 0 at every token: each key row of every (layer, sequence, head) state is multiplied by
    the product over tokens of its own alpha, so any slip in the [T][L][B][Hv][dk] indexing shows."""
    cfg = gi.custom("pk_idx", d_model=64, n_k_heads=2, d_k=16, n_v_heads=4, d_v=8, n_layers=2, batch=3,
                    n_tokens=3, flags=gi.DN_ALPHA_PER_KEY, ring_std=1.0)
    layers, stream = gi.generate(cfg)
    a = np.exp(-RNG.uniform(0.0, 1.0, size=stream.alpha.shape)).astype(np.float32)
    zero = np.zeros_like(stream.beta)
    S0, H0 = orc.initial_state(layers)
    _, S, _ = orc.run(cfg, layers, gi.Stream(stream.x, a, zero), S=S0, hist=H0)
    want = S0 * np.prod(a.astype(np.float64), axis=0)[..., None]
    np.testing.assert_allclose(S, want, rtol=1e-14, atol=0)


# --------------------------------------------------------------------------- gates on the card
# The pages name the two gates (a/b, one output per value head each) and leave their formula to
# the engine; the oracle states the decay form alpha = exp(-exp(a_log) softplus(a + a_bias)),
# beta = sigmoid(b). These pins tie it to values that follow from that statement alone.

def test_softplus_special_values_and_identity():
    assert orc.softplus(0.0) == pytest.approx(np.log(2.0), rel=1e-15)
    assert orc.softplus(np.log(np.e - 1.0)) == pytest.approx(1.0, rel=1e-15)
    assert orc.softplus(40.0) == pytest.approx(40.0 + np.exp(-40.0), rel=1e-15)
    assert orc.softplus(-40.0) == pytest.approx(np.exp(-40.0), rel=1e-12)
    for y in (-30.0, -3.5, -0.25, 0.7, 5.0, 31.0):
        # log(1 + e^y) - log(1 + e^-y) = y
        assert orc.softplus(y) - orc.softplus(-y) == pytest.approx(y, rel=1e-14, abs=1e-14)


def test_gates_special_values():
    # a + a_bias = 0: softplus = ln 2, so alpha = 2^(-e^a_log)
    assert orc.gates(0.0, 0.0, 0.0, 0.0) == pytest.approx((0.5, 0.5), rel=1e-15)
    assert orc.gates(1.5, 0.0, np.log(2.0), -1.5)[0] == pytest.approx(0.25, rel=1e-14)
    assert orc.gates(-2.0, 0.0, np.log(3.0), 2.0)[0] == pytest.approx(0.125, rel=1e-14)
    # softplus = 1: alpha = exp(-e^a_log)
    assert orc.gates(np.log(np.e - 1.0), 0.0, 0.0, 0.0)[0] == pytest.approx(np.exp(-1.0), rel=1e-14)
    # beta = sigmoid(b)
    assert orc.gates(0.0, np.log(3.0), 0.0, 0.0)[1] == pytest.approx(0.75, rel=1e-15)
    assert orc.gates(0.0, -np.log(3.0), 0.0, 0.0)[1] == pytest.approx(0.25, rel=1e-15)
    # a strongly negative gate input keeps the state (alpha -> 1), a strongly positive one clears it
    assert orc.gates(-60.0, 0.0, 1.0, 0.0)[0] == pytest.approx(1.0, abs=1e-20)
    assert orc.gates(60.0, 0.0, 0.0, 0.0)[0] == pytest.approx(np.exp(-60.0), rel=1e-12)
    # alpha depends on a + a_bias only; beta on b only
    for a, c, d in ((0.3, -4.0, 1.7), (-2.0, -6.5, -0.4)):
        assert orc.gates(a, 0.2, 1.1, c) == pytest.approx(orc.gates(a + d, 0.2, 1.1, c - d), rel=1e-14)


def _gates_layer(weight_bits=8):
    cfg = gi.custom("gates_pin", d_model=64, n_k_heads=2, d_k=16, n_v_heads=4, d_v=16, n_tokens=3,
                    flags=gi.DN_GATES_ON_DEVICE, weight_bits=weight_bits, ring_std=1.0)
    layers, stream = gi.generate(cfg)
    return cfg, layers[0], stream


def _with_gate_rows(cfg, lay, a_rows, b_rows, a_bias=None):
    """The layer with its gate rows' integer values replaced (0 keeps, None zeroes the block)."""
    import copy
    lay = copy.copy(lay)
    vals = lay.w_in_vals.copy()
    R0, Hv = cfg.conv_channels + cfg.v_dim, cfg.n_v_heads
    if a_rows is None:
        vals[R0:R0 + Hv] = 0
    if b_rows is None:
        vals[R0 + Hv:R0 + 2 * Hv] = 0
    lay.w_in_vals = vals
    lay.w_in = vals if cfg.weight_bits == 8 else gi.pack_int4(vals)
    if a_bias is not None:
        lay.a_bias = np.asarray(a_bias, np.float32)
    return lay


def _explicit_step(cfg, lay, S, hist, x, alpha, beta):
    """The same layer without the gate flag, gates given: the oracle's pinned explicit-gate path."""
    import copy
    plain = cfg.replace(flags=cfg.flags & ~gi.DN_GATES_ON_DEVICE)
    lay2 = copy.copy(lay)
    R = plain.in_rows
    lay2.w_in = np.ascontiguousarray(lay.w_in[:R]); lay2.s_in = np.ascontiguousarray(lay.s_in[:R])
    return orc.layer_step(plain, lay2, S, hist, x, np.asarray(alpha, np.float32)[None],
                          np.asarray(beta, np.float32)[None])


@pytest.mark.parametrize("bits", [8, 4])
def test_gates_zero_rows_give_closed_form_gates(bits):
    """a = b = 0 and a_bias = 0: every head decays by 2^(-e^a_log[h]) with beta = 1/2."""
    cfg, lay, stream = _gates_layer(bits)
    lay = _with_gate_rows(cfg, lay, None, None, a_bias=np.zeros(cfg.n_v_heads))
    Hv = cfg.n_v_heads
    S1 = RNG.standard_normal((1, Hv, cfg.d_k, cfg.d_v)); S2 = S1.copy()
    h1 = RNG.standard_normal((1, cfg.conv_k - 1, cfg.conv_channels)); h2 = h1.copy()
    x = stream.x[0].astype(np.float64)
    out = orc.layer_step(cfg, lay, S1, h1, x, np.zeros((1, Hv), np.float32), np.zeros((1, Hv), np.float32))
    alpha = 2.0 ** (-np.exp(lay.a_log.astype(np.float64)))
    ref = _explicit_step(cfg, lay, S2, h2, x, alpha, np.full(Hv, 0.5))
    np.testing.assert_allclose(out, ref, rtol=1e-5, atol=1e-6 * np.max(np.abs(ref)))
    np.testing.assert_allclose(S1, S2, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("which", ["a", "b"])
def test_gates_read_their_own_rows_and_head(which):
    """Only one gate block nonzero: the other gate keeps its closed form, and the nonzero one
    follows from that block's rows for each head (a swapped block or a shifted head shows)."""
    cfg, lay, stream = _gates_layer()
    Hv, R0 = cfg.n_v_heads, cfg.conv_channels + cfg.v_dim
    lay = _with_gate_rows(cfg, lay, 0 if which == "a" else None, 0 if which == "b" else None)
    x = stream.x[0].astype(np.float64)
    rows = lay.s_in[R0:].astype(np.float64) * (lay.w_in_vals[R0:].astype(np.float64) @ x[0])
    a, b = rows[:Hv], rows[Hv:]
    assert np.all(a == 0) != (which == "a") and np.all(b == 0) != (which == "b")
    y = a + lay.a_bias.astype(np.float64)
    alpha = np.exp(-np.exp(lay.a_log.astype(np.float64)) * (np.maximum(y, 0) + np.log1p(np.exp(-np.abs(y)))))
    beta = 1.0 / (1.0 + np.exp(-b))
    S1 = RNG.standard_normal((1, Hv, cfg.d_k, cfg.d_v)); S2 = S1.copy()
    h1 = RNG.standard_normal((1, cfg.conv_k - 1, cfg.conv_channels)); h2 = h1.copy()
    out = orc.layer_step(cfg, lay, S1, h1, x, np.zeros((1, Hv), np.float32), np.zeros((1, Hv), np.float32))
    ref = _explicit_step(cfg, lay, S2, h2, x, alpha, beta)
    np.testing.assert_allclose(out, ref, rtol=1e-5, atol=1e-6 * np.max(np.abs(ref)))
    np.testing.assert_allclose(S1, S2, rtol=1e-5, atol=1e-7)


def test_gates_ignore_the_gate_arrays():
    cfg, lay, stream = _gates_layer()
    cfg3 = cfg.replace(n_tokens=3)
    out1, S1, H1 = orc.run(cfg3, [lay], stream)
    noise = gi.Stream(stream.x, RNG.uniform(0, 1, stream.alpha.shape).astype(np.float32),
                      RNG.uniform(0, 1, stream.beta.shape).astype(np.float32))
    out2, S2, H2 = orc.run(cfg3, [lay], noise)
    assert np.array_equal(out1, out2) and np.array_equal(S1, S2)
