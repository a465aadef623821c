"""Seeded synthetic inputs for the gated-DeltaNet decode step.

This module is shared by the CPU oracle and the HIP path. It only draws random
numbers and lays them out in memory; it holds none of the layer's arithmetic.

Layouts (all C-contiguous, little-endian):

* ``w_in``   int8  [R_in][D]      rows ordered q (Hk*dk) | k (Hk*dk) | v (Hv*dv) | z (Hv*dv),
                                   each block head-major with the head dimension contiguous;
                                   with DN_GATES_ON_DEVICE two more blocks a (Hv) | b (Hv).
                                   For 4-bit weights: uint8 [R_in][D/2], element 2c in the low
                                   nibble and 2c+1 in the high nibble, 4-bit two's complement.
* ``s_in``   fp32  [R_in]         one scale per in_proj row.
* ``conv_w`` fp32  [C][K]         depthwise causal conv taps; tap K-1 multiplies the current token.
* ``norm_w`` fp32  [dv]           gated RMSNorm weight, shared by all value heads.
* ``w_out``  int8  [D][Hv*dv]     (or packed uint8 [D][Hv*dv/2]), ``s_out`` fp32 [D].
* ``a_log``, ``a_bias`` fp32 [Hv] (DN_GATES_ON_DEVICE only): per value head parameters of the
                                   decay gate.
* ``S0``     fp32  [B][Hv][dk][dv] initial recurrent state.
* ``ring0``  fp32  [B][K-1][C]    conv history, oldest token first.
* stream: ``x`` fp32 [T][B][D] (input of layer 0), ``alpha``/``beta`` fp32 [T][L][B][Hv].

Distributions follow the workload description of the layer: integer weights
uniform over the symmetric int8 (or int4) range, per-row scales U[0.005, 0.02],
x ~ N(0, 1), alpha = exp(-U[0, 0.1]), beta = sigmoid(N(0, 1)), state N(0, 0.02).
Conv taps U[-0.5, 0.5] and norm weights U[0.5, 1.5] are this module's choice
(the pages give no values for them). With DN_GATES_ON_DEVICE the gate rows a, b take
the same integer range with row scales U[0.5, 1.5] / (rms of the integers * sqrt(D)),
so that a and b are of order one for a unit-rms input; a_log = log U[1, 16] and
a_bias ~ U[-7, -2]. These are drawn after everything else of the layer, so every other
array equals that of the same seed without the flag.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

DN_X_RMSNORM = 1  # flag bit: RMS-normalise each layer's input (stack pre-norm)
DN_ALPHA_PER_KEY = 2  # flag bit: one decay per key channel, alpha [T][L][B][Hv][dk]
DN_GATES_ON_DEVICE = 4  # flag bit: alpha and beta computed from two more in_proj rows per value head


@dataclass(frozen=True)
class Config:
    name: str
    d_model: int
    n_k_heads: int
    d_k: int
    n_v_heads: int
    d_v: int
    conv_k: int = 4
    batch: int = 1
    n_layers: int = 1
    n_tokens: int = 8
    weight_bits: int = 8
    flags: int = 0
    eps_l2: float = 1e-6
    eps_rms: float = 1e-6
    q_scale: float = 1.0
    layer_seeds: tuple = (0,)
    stream_seed: int | None = None  # None: draw the stream from the last layer's generator
    state_std: float = 0.02
    ring_std: float = 0.0  # 0 => zero ring
    zero_state: bool = False

    # derived sizes -----------------------------------------------------
    @property
    def qk_dim(self) -> int:
        return self.n_k_heads * self.d_k

    @property
    def v_dim(self) -> int:
        return self.n_v_heads * self.d_v

    @property
    def conv_channels(self) -> int:
        return 2 * self.qk_dim + self.v_dim

    @property
    def gate_rows(self) -> int:
        return 2 * self.n_v_heads if self.flags & DN_GATES_ON_DEVICE else 0

    @property
    def in_rows(self) -> int:
        return self.conv_channels + self.v_dim + self.gate_rows

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    # metric bytes: quantised matrices + fp32 scales + conv taps + norm weight + 2 x fp32 state
    def weight_bytes_per_layer(self) -> int:
        D, R, V, C, K = self.d_model, self.in_rows, self.v_dim, self.conv_channels, self.conv_k
        if self.weight_bits == 8:
            mat = R * D + D * V
        else:
            mat = R * D // 2 + D * V // 2
        gates = 8 * self.n_v_heads if self.flags & DN_GATES_ON_DEVICE else 0
        return mat + 4 * (R + D) + 4 * C * K + 4 * self.d_v + gates

    def state_bytes_per_layer(self) -> int:
        return 4 * self.batch * self.n_v_heads * self.d_k * self.d_v

    def metric_bytes_per_step(self) -> int:
        """Bytes one step (one token for every sequence, through every layer) must move."""
        return self.n_layers * (self.weight_bytes_per_layer() + 2 * self.state_bytes_per_layer())


def _tiny() -> Config:
    return Config("tiny", d_model=64, n_k_heads=2, d_k=16, n_v_heads=4, d_v=16, n_tokens=8,
                  layer_seeds=(0,), zero_state=True)


CONFIGS = {
    # tiny single layer, seed 0, S0 = 0, 8 tokens
    "tiny": _tiny(),
    # one layer at the hybrid-35B DeltaNet shape, 256 tokens
    "layer": Config("layer", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128,
                    n_tokens=256, layer_seeds=(1,)),
    # 30 independent layers chained, 200 tokens, single sequence
    "stack": Config("stack", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128,
                    n_tokens=200, n_layers=30, layer_seeds=tuple(2000 + l for l in range(30)),
                    stream_seed=2999, ring_std=1.0, flags=DN_X_RMSNORM),
    # 64 independent sequences stepped together
    "batched": Config("batched", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128,
                      n_tokens=128, batch=64, layer_seeds=(3,)),
    # the stack with packed signed int4 weights
    "stack_int4": Config("stack_int4", d_model=2048, n_k_heads=16, d_k=128, n_v_heads=32, d_v=128,
                         n_tokens=200, n_layers=30, weight_bits=4,
                         layer_seeds=tuple(4000 + l for l in range(30)), stream_seed=4999,
                         ring_std=1.0, flags=DN_X_RMSNORM),
}


def pack_int4(vals: np.ndarray) -> np.ndarray:
    """Pack int8 values in [-8, 7] two per byte along the last axis (even index -> low nibble)."""
    v = np.asarray(vals, dtype=np.int8)
    assert v.shape[-1] % 2 == 0
    u = (v.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


@dataclass
class Layer:
    w_in: np.ndarray       # int8 [R][D] or uint8 packed [R][D/2]
    s_in: np.ndarray
    conv_w: np.ndarray
    norm_w: np.ndarray
    w_out: np.ndarray
    s_out: np.ndarray
    S0: np.ndarray
    ring0: np.ndarray
    w_in_vals: np.ndarray = field(repr=False, default=None)   # int8 values (for 4-bit configs)
    w_out_vals: np.ndarray = field(repr=False, default=None)
    a_log: np.ndarray = None   # [Hv] (DN_GATES_ON_DEVICE)
    a_bias: np.ndarray = None  # [Hv] (DN_GATES_ON_DEVICE)


@dataclass
class Stream:
    x: np.ndarray      # [T][B][D]
    alpha: np.ndarray  # [T][L][B][Hv] ([T][L][B][Hv][dk] with DN_ALPHA_PER_KEY)
    beta: np.ndarray   # [T][L][B][Hv]


def _ints(rng, shape, bits):
    hi = 127 if bits == 8 else 7
    return rng.integers(-hi, hi + 1, size=shape, dtype=np.int8)


def gen_layer(cfg: Config, seed: int, rng=None) -> tuple[Layer, np.random.Generator]:
    rng = np.random.default_rng(seed) if rng is None else rng
    D, V, C, K = cfg.d_model, cfg.v_dim, cfg.conv_channels, cfg.conv_k
    R = C + V  # rows q | k | v | z; gate rows are drawn last
    B, Hv, dk, dv = cfg.batch, cfg.n_v_heads, cfg.d_k, cfg.d_v
    w_in_v = _ints(rng, (R, D), cfg.weight_bits)
    s_in = rng.uniform(0.005, 0.02, size=R).astype(np.float32)
    conv_w = rng.uniform(-0.5, 0.5, size=(C, K)).astype(np.float32)
    norm_w = rng.uniform(0.5, 1.5, size=dv).astype(np.float32)
    w_out_v = _ints(rng, (D, V), cfg.weight_bits)
    s_out = rng.uniform(0.005, 0.02, size=D).astype(np.float32)
    if cfg.zero_state:
        S0 = np.zeros((B, Hv, dk, dv), np.float32)
    else:
        S0 = (rng.standard_normal((B, Hv, dk, dv)) * cfg.state_std).astype(np.float32)
    if cfg.ring_std > 0:
        ring0 = (rng.standard_normal((B, K - 1, C)) * cfg.ring_std).astype(np.float32)
    else:
        ring0 = np.zeros((B, K - 1, C), np.float32)
    a_log = a_bias = None
    if cfg.flags & DN_GATES_ON_DEVICE:
        hi = 127 if cfg.weight_bits == 8 else 7
        rms_int = np.sqrt(hi * (hi + 1) / 3.0)
        G = cfg.gate_rows
        w_in_v = np.concatenate([w_in_v, _ints(rng, (G, D), cfg.weight_bits)])
        s_in = np.concatenate([s_in, (rng.uniform(0.5, 1.5, size=G) / (rms_int * np.sqrt(D))).astype(np.float32)])
        a_log = np.log(rng.uniform(1.0, 16.0, size=Hv)).astype(np.float32)
        a_bias = rng.uniform(-7.0, -2.0, size=Hv).astype(np.float32)
    if cfg.weight_bits == 8:
        lay = Layer(w_in_v, s_in, conv_w, norm_w, w_out_v, s_out, S0, ring0, w_in_v, w_out_v, a_log, a_bias)
    else:
        lay = Layer(pack_int4(w_in_v), s_in, conv_w, norm_w, pack_int4(w_out_v), s_out, S0, ring0,
                    w_in_v, w_out_v, a_log, a_bias)
    return lay, rng


def gen_stream(cfg: Config, rng: np.random.Generator, n_tokens: int | None = None) -> Stream:
    T = cfg.n_tokens if n_tokens is None else n_tokens
    B, D, L, Hv = cfg.batch, cfg.d_model, cfg.n_layers, cfg.n_v_heads
    x = rng.standard_normal((T, B, D)).astype(np.float32)
    ashape = (T, L, B, Hv, cfg.d_k) if cfg.flags & DN_ALPHA_PER_KEY else (T, L, B, Hv)
    alpha = np.exp(-rng.uniform(0.0, 0.1, size=ashape)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, L, B, Hv))))).astype(np.float32)
    return Stream(x, alpha, beta)


def generate(cfg: Config, n_tokens: int | None = None, n_layers: int | None = None):
    """Return (layers, stream). ``n_layers`` truncates a stack (the first layers keep their seeds)."""
    L = cfg.n_layers if n_layers is None else n_layers
    layers = []
    rng = None
    for l in range(L):
        lay, rng = gen_layer(cfg, cfg.layer_seeds[l])
        layers.append(lay)
    if cfg.stream_seed is not None:
        rng = np.random.default_rng(cfg.stream_seed)
    stream = gen_stream(cfg.replace(n_layers=L), rng, n_tokens)
    return layers, stream


def custom(name: str, **kw) -> Config:
    """A small config for parity tests (seeds default to a hash of the name)."""
    base = dict(conv_k=4, batch=1, n_layers=1, n_tokens=8)
    base.update(kw)
    L = base["n_layers"]
    if "layer_seeds" not in base:
        h = sum(ord(c) * (i + 1) for i, c in enumerate(name)) % 100000
        base["layer_seeds"] = tuple(10_000 + 100 * h + l for l in range(L))
    return Config(name, **base)
