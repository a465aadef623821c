"""ctypes binding of the fp64 CPU oracle (``dn_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline of ``bench.py`` use it; the HIP library never does. It imports nothing
from the HIP package and the HIP package imports nothing from here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dn_oracle.c")
_LIB = os.path.join(_HERE, "libdn_oracle.so")
_lock = threading.Lock()
_lib = None

X_RMSNORM = 1
GATES_ON_DEVICE = 4


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int), ("n_k_heads", ctypes.c_int), ("d_k", ctypes.c_int),
                ("n_v_heads", ctypes.c_int), ("d_v", ctypes.c_int), ("conv_k", ctypes.c_int),
                ("batch", ctypes.c_int), ("n_layers", ctypes.c_int), ("weight_bits", ctypes.c_int),
                ("flags", ctypes.c_uint), ("eps_l2", ctypes.c_double), ("eps_rms", ctypes.c_double),
                ("q_scale", ctypes.c_double)]


class _LayerW(ctypes.Structure):
    _fields_ = [("w_in", ctypes.c_void_p), ("s_in", ctypes.c_void_p), ("conv_w", ctypes.c_void_p),
                ("norm_w", ctypes.c_void_p), ("w_out", ctypes.c_void_p), ("s_out", ctypes.c_void_p),
                ("a_log", ctypes.c_void_p), ("a_bias", ctypes.c_void_p)]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("DN_ORACLE_LIB")  # a planted-mistake build (mutation tests)
            if not path:
                path = _LIB
                if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                    build(force=True)
            L = ctypes.CDLL(path)
            P = ctypes.c_void_p
            I = ctypes.c_int
            Dd = ctypes.c_double
            L.dno_silu.argtypes = [Dd]; L.dno_silu.restype = Dd
            L.dno_weight.argtypes = [P, I, ctypes.c_long, ctypes.c_long, ctypes.c_long]; L.dno_weight.restype = I
            L.dno_gemv.argtypes = [I, I, P, I, P, P, P]; L.dno_gemv.restype = None
            L.dno_rms_prenorm.argtypes = [I, P, Dd, P]; L.dno_rms_prenorm.restype = None
            L.dno_conv_silu.argtypes = [I, I, P, P, P, P]; L.dno_conv_silu.restype = None
            L.dno_l2norm.argtypes = [I, P, Dd, P]; L.dno_l2norm.restype = None
            L.dno_delta_head.argtypes = [I, I, P, P, P, P, Dd, Dd, Dd, P]; L.dno_delta_head.restype = None
            L.dno_delta_head_vec.argtypes = [I, I, P, P, P, P, P, Dd, Dd, P]; L.dno_delta_head_vec.restype = None
            L.dno_gated_rmsnorm.argtypes = [I, P, P, P, Dd, P]; L.dno_gated_rmsnorm.restype = None
            L.dno_softplus.argtypes = [Dd]; L.dno_softplus.restype = Dd
            L.dno_gates.argtypes = [Dd, Dd, Dd, Dd, P, P]; L.dno_gates.restype = None
            L.dno_layer_step.argtypes = [P, P, P, P, P, P, P, P]; L.dno_layer_step.restype = I
            L.dno_run.argtypes = [P, P, P, P, I, P, P, P, P]; L.dno_run.restype = I
            L.dno_threads.argtypes = []; L.dno_threads.restype = I
            _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# --- single steps -----------------------------------------------------------

def silu(a: float) -> float:
    return lib().dno_silu(float(a))


def gemv(W: np.ndarray, s, x, bits: int = 8) -> np.ndarray:
    """y[r] = s[r] * sum_c W[r][c] x[c]; W int8 [R][C] or packed uint8 [R][C/2] (bits=4)."""
    W = np.ascontiguousarray(W)
    rows = W.shape[0]
    cols = W.shape[1] * (2 if bits == 4 else 1)
    s = _f32(s); x = _f64(x)
    assert s.shape == (rows,) and x.shape == (cols,)
    y = np.zeros(rows, np.float64)
    lib().dno_gemv(rows, cols, _p(W), bits, _p(s), _p(x), _p(y))
    return y


def weight(W: np.ndarray, bits: int, cols: int, r: int, c: int) -> int:
    W = np.ascontiguousarray(W)
    return lib().dno_weight(_p(W), bits, cols, r, c)


def rms_prenorm(x, eps: float) -> np.ndarray:
    x = _f64(x); y = np.zeros_like(x)
    lib().dno_rms_prenorm(x.size, _p(x), eps, _p(y))
    return y


def conv_silu(w, hist, u):
    """One token of the depthwise conv + SiLU; returns (out, new_hist). hist [K-1][C] oldest first."""
    w = _f32(w); C, K = w.shape
    hist = _f64(hist).copy().reshape(K - 1, C) if K > 1 else np.zeros((0, C))
    u = _f64(u); out = np.zeros(C, np.float64)
    lib().dno_conv_silu(C, K, _p(w), _p(hist), _p(u), _p(out))
    return out, hist


def l2norm(v, eps: float) -> np.ndarray:
    v = _f64(v); o = np.zeros_like(v)
    lib().dno_l2norm(v.size, _p(v), eps, _p(o))
    return o


def delta_head(S, k, v, q, alpha, beta, q_scale=1.0):
    """Returns (S_new, o). S [dk][dv]."""
    S = _f64(S).copy(); dk, dv = S.shape
    k = _f64(k); v = _f64(v); q = _f64(q); o = np.zeros(dv, np.float64)
    lib().dno_delta_head(dk, dv, _p(S), _p(k), _p(v), _p(q), float(alpha), float(beta), float(q_scale), _p(o))
    return S, o


def delta_head_vec(S, k, v, q, alpha, beta, q_scale=1.0):
    """The recurrence with a decay per key channel: alpha [dk] scales key row i. Returns (S_new, o)."""
    S = _f64(S).copy(); dk, dv = S.shape
    k = _f64(k); v = _f64(v); q = _f64(q); a = _f64(alpha); o = np.zeros(dv, np.float64)
    assert a.shape == (dk,)
    lib().dno_delta_head_vec(dk, dv, _p(S), _p(k), _p(v), _p(q), _p(a), float(beta), float(q_scale), _p(o))
    return S, o


def softplus(y: float) -> float:
    return lib().dno_softplus(float(y))


def gates(a: float, b: float, a_log: float, a_bias: float):
    """(alpha, beta) of a value head from its gate rows a, b and parameters a_log, a_bias."""
    al = ctypes.c_double(); be = ctypes.c_double()
    lib().dno_gates(float(a), float(b), float(a_log), float(a_bias), ctypes.byref(al), ctypes.byref(be))
    return al.value, be.value


def gated_rmsnorm(o, z, w, eps: float) -> np.ndarray:
    o = _f64(o); z = _f64(z); w = _f32(w); y = np.zeros_like(o)
    lib().dno_gated_rmsnorm(o.size, _p(o), _p(z), _p(w), eps, _p(y))
    return y


# --- whole layers / runs ----------------------------------------------------

def _dims(cfg, n_layers=None) -> _Dims:
    return _Dims(cfg.d_model, cfg.n_k_heads, cfg.d_k, cfg.n_v_heads, cfg.d_v, cfg.conv_k, cfg.batch,
                 cfg.n_layers if n_layers is None else n_layers, cfg.weight_bits, cfg.flags,
                 cfg.eps_l2, cfg.eps_rms, cfg.q_scale)


def _weights(layers):
    arr = (_LayerW * len(layers))()
    keep = []
    for i, lay in enumerate(layers):
        ws = [np.ascontiguousarray(lay.w_in), _f32(lay.s_in), _f32(lay.conv_w), _f32(lay.norm_w),
              np.ascontiguousarray(lay.w_out), _f32(lay.s_out)]
        gs = [None if getattr(lay, n, None) is None else _f32(getattr(lay, n)) for n in ("a_log", "a_bias")]
        keep += ws + [g for g in gs if g is not None]
        arr[i] = _LayerW(*[a.ctypes.data for a in ws], *[None if g is None else g.ctypes.data for g in gs])
    return arr, keep


def layer_step(cfg, layer, S, hist, x, alpha, beta):
    """One token through one layer. S [B][Hv][dk][dv], hist [B][K-1][C] (double, updated in place),
    x [B][D]; returns out [B][D]."""
    d = _dims(cfg, 1)
    W, keep = _weights([layer])
    x = _f64(x); a = _f32(alpha); b = _f32(beta)
    out = np.zeros((cfg.batch, cfg.d_model), np.float64)
    assert S.dtype == np.float64 and S.flags["C_CONTIGUOUS"] and hist.dtype == np.float64
    rc = lib().dno_layer_step(ctypes.byref(d), W, _p(S), _p(hist), _p(x), _p(a), _p(b), _p(out))
    if rc:
        raise ValueError("oracle rejected the dimensions")
    return out


def initial_state(layers):
    S = np.stack([l.S0 for l in layers]).astype(np.float64)
    H = np.stack([l.ring0 for l in layers]).astype(np.float64)
    return np.ascontiguousarray(S), np.ascontiguousarray(H)


def run(cfg, layers, stream, n_tokens=None, S=None, hist=None):
    """Run the oracle over a token stream. Returns (out [T][L][B][D], S [L][B][Hv][dk][dv], hist)."""
    L = len(layers)
    T = stream.x.shape[0] if n_tokens is None else n_tokens
    if S is None:
        S, hist = initial_state(layers)
    else:
        S = np.ascontiguousarray(S, np.float64).copy(); hist = np.ascontiguousarray(hist, np.float64).copy()
    d = _dims(cfg, L)
    W, keep = _weights(layers)
    x = _f32(stream.x[:T]); a = _f32(stream.alpha[:T, :L]); b = _f32(stream.beta[:T, :L])
    out = np.zeros((T, L, cfg.batch, cfg.d_model), np.float64)
    rc = lib().dno_run(ctypes.byref(d), W, _p(S), _p(hist), T, _p(x), _p(a), _p(b), _p(out))
    if rc:
        raise ValueError("oracle rejected the dimensions")
    return out, S, hist


def threads() -> int:
    return lib().dno_threads()
