"""Thin Python binding of libdn (the gated-DeltaNet decode step on MI355X).

Argument marshalling only: every step of the decode token runs in the HIP kernels of
``libdn.so`` (``dn_create``, ``dn_set_state``, ``dn_get_state``, ``dn_step``, ``dn_destroy``),
and of a prompt in those of ``libdn_prefill.so`` (``dn_prefill``). PyTorch provides device
memory and streams. The functions carry the C ABI's names; ``DeltaNetStack`` wraps them.
Loading fails loudly when a library is not built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# DN_LIB selects another build of the library (an instrumented one, for instance)
LIB_PATH = os.environ.get("DN_LIB") or os.path.join(_PKG, "libdn.so")
PREFILL_LIB_PATH = os.environ.get("DN_PREFILL_LIB") or os.path.join(_PKG, "libdn_prefill.so")
PROBE_LIB_PATH = os.path.join(_PKG, "libdn_probe.so")  # measurement only (bench.py)

DN_OK, DN_E_INVAL, DN_E_NOMEM, DN_E_DEVICE, DN_E_DISABLED, DN_E_FAULT = 0, -1, -2, -3, -4, -5
DN_X_RMSNORM = 1
DN_ALPHA_PER_KEY = 2  # alpha [L][B][Hv][dk]: one decay per key channel
DN_GATES_ON_DEVICE = 4  # gates from two more in_proj rows per value head; alpha/beta not read
DN_PREFILL_MAX_TOKENS = 65535  # prompt tokens per dn_prefill call
DN_PREFILL_NOALLOC_SCRATCH_BYTES = 64 << 20  # the static scratch of dn_prefill_noalloc, per device
EXPORTED = ("dn_create", "dn_set_state", "dn_get_state", "dn_step", "dn_destroy")  # libdn.so
PREFILL_EXPORTED = ("dn_prefill", "dn_prefill_noalloc")  # libdn_prefill.so

_ERR = {DN_OK: "ok", DN_E_INVAL: "invalid argument", DN_E_NOMEM: "out of device memory",
        DN_E_DEVICE: "device error", DN_E_DISABLED: "layer disabled after a failed step",
        DN_E_FAULT: "injected fault"}


class DNError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"{what}: {_ERR.get(rc, 'unknown error')} ({rc})")
        self.rc = rc


class dn_config(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int), ("n_k_heads", ctypes.c_int), ("d_k", ctypes.c_int),
                ("n_v_heads", ctypes.c_int), ("d_v", ctypes.c_int), ("conv_k", ctypes.c_int),
                ("batch", ctypes.c_int), ("n_layers", ctypes.c_int), ("weight_bits", ctypes.c_int),
                ("flags", ctypes.c_uint), ("eps_l2", ctypes.c_float), ("eps_rms", ctypes.c_float),
                ("q_scale", ctypes.c_float)]


class dn_weights(ctypes.Structure):
    _fields_ = [("w_in", ctypes.c_void_p), ("s_in", ctypes.c_void_p), ("conv_w", ctypes.c_void_p),
                ("norm_w", ctypes.c_void_p), ("w_out", ctypes.c_void_p), ("s_out", ctypes.c_void_p),
                ("a_log", ctypes.c_void_p), ("a_bias", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libdn.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libdn.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.dn_create.argtypes = [ctypes.POINTER(dn_config), ctypes.POINTER(dn_weights), ctypes.POINTER(P)]
        L.dn_create.restype = ctypes.c_int
        L.dn_set_state.argtypes = [P, P, P]; L.dn_set_state.restype = ctypes.c_int
        L.dn_get_state.argtypes = [P, P, P]; L.dn_get_state.restype = ctypes.c_int
        L.dn_step.argtypes = [P, P, P, P, P, P]; L.dn_step.restype = ctypes.c_int
        L.dn_destroy.argtypes = [P]; L.dn_destroy.restype = None
        _lib = L
    return _lib


_plib = None


def prefill_lib():
    """Load libdn_prefill.so (after libdn.so, whose handles it takes); raises if it is missing."""
    global _plib
    if _plib is None:
        lib()
        if not os.path.exists(PREFILL_LIB_PATH):
            raise ImportError(f"libdn_prefill.so is not built ({PREFILL_LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(PREFILL_LIB_PATH)
        P = ctypes.c_void_p
        L.dn_prefill.argtypes = [P, P, ctypes.c_int, P, P, P, P]; L.dn_prefill.restype = ctypes.c_int
        L.dn_prefill_noalloc.argtypes = [P, P, ctypes.c_int, P, P, P, P]; L.dn_prefill_noalloc.restype = ctypes.c_int
        _plib = L
    return _plib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        assert t.is_contiguous(), "tensors passed to libdn must be contiguous"
        return t.data_ptr()
    return int(t)


def _check(rc: int, what: str):
    if rc != DN_OK:
        raise DNError(rc, what)


# --- the calls -------------------------------------------------------------------------

def dn_create(cfg: dn_config, weights: list[dn_weights]) -> int:
    arr = (dn_weights * len(weights))(*weights)
    h = ctypes.c_void_p()
    _check(lib().dn_create(ctypes.byref(cfg), arr, ctypes.byref(h)), "dn_create")
    return h.value


def dn_set_state(h: int, S, ring=None) -> None:
    _check(lib().dn_set_state(h, _ptr(S), _ptr(ring)), "dn_set_state")


def dn_get_state(h: int, S, ring=None) -> None:
    _check(lib().dn_get_state(h, _ptr(S), _ptr(ring)), "dn_get_state")


def dn_status(h: int) -> int:
    """dn_get_state with no buffers: wait for the device and return the C return code that
    reports whether every step so far completed."""
    return lib().dn_get_state(h, None, None)


def _stream(stream, ref):
    """The stream handle to pass: the given one, else the current stream of ref's device."""
    if stream is None:
        dev = ref.device if isinstance(ref, torch.Tensor) and ref.is_cuda else None
        return torch.cuda.current_stream(dev).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def dn_step(h: int, x, alpha, beta, out, stream=None) -> int:
    """Enqueue one token; returns the C return code (no exception, so callers can test errors)."""
    return lib().dn_step(h, _ptr(x), _ptr(alpha), _ptr(beta), _ptr(out), _stream(stream, out))


def dn_prefill(h: int, x, n_tokens: int, alpha, beta, out, stream=None) -> int:
    """Enqueue a prompt of n_tokens tokens (x [T][D], alpha/beta [T][L][Hv], out [L][T][D]);
    returns the C return code."""
    return prefill_lib().dn_prefill(h, _ptr(x), int(n_tokens), _ptr(alpha), _ptr(beta), _ptr(out),
                                    _stream(stream, out))


def dn_prefill_noalloc(h: int, x, n_tokens: int, alpha, beta, out, stream=None) -> int:
    """dn_prefill on the library's static scratch, allocating nothing; returns the C return code."""
    return prefill_lib().dn_prefill_noalloc(h, _ptr(x), int(n_tokens), _ptr(alpha), _ptr(beta), _ptr(out),
                                            _stream(stream, out))


def dn_destroy(h: int) -> None:
    if h:
        lib().dn_destroy(h)


# --- convenience wrapper -------------------------------------------------------------------

def _dev(a, dtype, device):
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=dtype).contiguous()
    return torch.from_numpy(a).to(device=device, dtype=dtype).contiguous()


class DeltaNetStack:
    """A handle over n_layers layers. ``layers`` are objects with attributes w_in, s_in, conv_w,
    norm_w, w_out, s_out (numpy arrays or tensors, in the layouts of include/dn.h), and a_log,
    a_bias with DN_GATES_ON_DEVICE."""

    def __init__(self, *, d_model, n_k_heads, d_k, n_v_heads, d_v, layers, conv_k=4, batch=1,
                 weight_bits=8, flags=0, eps_l2=1e-6, eps_rms=1e-6, q_scale=1.0, device="cuda:0"):
        self.device = torch.device(device)
        self.cfg = dn_config(d_model, n_k_heads, d_k, n_v_heads, d_v, conv_k, batch, len(layers),
                             weight_bits, flags, eps_l2, eps_rms, q_scale)
        wdt = torch.int8 if weight_bits == 8 else torch.uint8
        self._keep = []
        ws = []
        for lay in layers:
            t = [_dev(lay.w_in, wdt, self.device), _dev(lay.s_in, torch.float32, self.device),
                 _dev(lay.conv_w, torch.float32, self.device), _dev(lay.norm_w, torch.float32, self.device),
                 _dev(lay.w_out, wdt, self.device), _dev(lay.s_out, torch.float32, self.device)]
            g = [None if getattr(lay, n, None) is None else _dev(getattr(lay, n), torch.float32, self.device)
                 for n in ("a_log", "a_bias")]
            self._keep.append(t + [x for x in g if x is not None])
            ws.append(dn_weights(*[x.data_ptr() for x in t], *[None if x is None else x.data_ptr() for x in g]))
        with torch.cuda.device(self.device):
            self.h = dn_create(self.cfg, ws)
        self.L, self.B, self.D = len(layers), batch, d_model
        self.Hv, self.dk, self.dv, self.K = n_v_heads, d_k, d_v, conv_k
        self.C = 2 * n_k_heads * d_k + n_v_heads * d_v

    @classmethod
    def from_config(cls, cfg, layers, device="cuda:0"):
        return cls(d_model=cfg.d_model, n_k_heads=cfg.n_k_heads, d_k=cfg.d_k, n_v_heads=cfg.n_v_heads,
                   d_v=cfg.d_v, layers=layers, conv_k=cfg.conv_k, batch=cfg.batch,
                   weight_bits=cfg.weight_bits, flags=cfg.flags, eps_l2=cfg.eps_l2, eps_rms=cfg.eps_rms,
                   q_scale=cfg.q_scale, device=device)

    def state_shapes(self):
        return (self.L, self.B, self.Hv, self.dk, self.dv), (self.L, self.B, self.K - 1, self.C)

    def set_state(self, S, ring=None):
        S = _dev(S, torch.float32, self.device)
        ring = None if ring is None else _dev(ring, torch.float32, self.device)
        dn_set_state(self.h, S, ring)

    def get_state(self):
        ss, rs = self.state_shapes()
        S = torch.empty(ss, dtype=torch.float32, device=self.device)
        ring = torch.empty(rs, dtype=torch.float32, device=self.device)
        dn_get_state(self.h, S, ring)
        return S, ring

    def status(self) -> int:
        """Wait for the device; DN_OK if every step so far completed, else the error code."""
        return dn_status(self.h)

    def new_out(self):
        return torch.empty((self.L, self.B, self.D), dtype=torch.float32, device=self.device)

    def step(self, x, alpha=None, beta=None, out=None, stream=None, check=True):
        if out is None:
            out = self.new_out()
        rc = dn_step(self.h, x, alpha, beta, out, stream)
        if check:
            _check(rc, "dn_step")
        return out if check else rc

    def prefill(self, x, alpha=None, beta=None, out=None, stream=None, check=True):
        """Run a prompt through every layer: x [T][D] (or [B][T][D], one prompt per sequence),
        alpha/beta [T][L][Hv] (or [T][L][B][Hv]; None with DN_GATES_ON_DEVICE); returns out
        [L][T][D] (or [L][B][T][D])."""
        T = x.shape[-2]
        if out is None:
            shape = (self.L, T, self.D) if self.B == 1 else (self.L, self.B, T, self.D)
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        rc = dn_prefill(self.h, x, T, alpha, beta, out, stream)
        if check:
            _check(rc, "dn_prefill")
        return out if check else rc

    def close(self):
        if getattr(self, "h", None):
            dn_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
