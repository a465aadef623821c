"""The C-ABI libraries load and export exactly the entry points their headers declare (no compute
calls: runs without a GPU). libdn exports the five calls of the page's per-layer object (page
"qwen36: run the DeltaNet layer end to end on the card", section "Verified": the loader's ABI
tripwire counts five optional symbols); the prompt path is a library of its own."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gated_deltanet_layer_dn_amd")
LIB = os.path.join(PKG, "libdn.so")
PLIB = os.path.join(PKG, "libdn_prefill.so")
HDR = os.path.join(ROOT, "include", "dn.h")
PHDR = os.path.join(ROOT, "include", "dn_prefill.h")
FIVE = {"dn_create", "dn_set_state", "dn_get_state", "dn_step", "dn_destroy"}


def _declared(path):
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:int|void)\s+\*?\s*(dn_\w+)\s*\(", src, flags=re.M))


def _exports(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    return {l.split()[-1] for l in out.splitlines() if l.split() and l.split()[-1].startswith("dn")}


@pytest.fixture(scope="module")
def built():
    if not (os.path.exists(LIB) and os.path.exists(PLIB)):
        from gated_deltanet_layer_dn_amd import build
        build.build()
    return LIB, PLIB


def test_header_declares_the_five_calls():
    assert _declared(HDR) == FIVE


def test_prefill_header_declares_the_prompt_calls():
    assert _declared(PHDR) == {"dn_prefill", "dn_prefill_noalloc"}


def test_library_exports_exactly_the_five_calls(built):
    assert _exports(built[0]) == FIVE


def test_prefill_library_exports_exactly_its_declared_calls(built):
    assert _exports(built[1]) == _declared(PHDR)


def test_probe_library_exports_exactly_its_declared_calls(built):
    probe = os.path.join(PKG, "libdn_probe.so")
    declared = _declared(os.path.join(ROOT, "include", "dn_probe.h"))
    assert declared == {"dn_probe_read_stream", "dn_probe_rmw_stream", "dn_probe_exchange"}
    assert _exports(probe) == declared


def test_libraries_load_and_resolve(built):
    L = ctypes.CDLL(built[0])
    for n in FIVE:
        assert getattr(L, n) is not None
    P = ctypes.CDLL(built[1])
    for n in _declared(PHDR):
        assert getattr(P, n) is not None


def test_libdn_does_not_link_the_gemm_library(built):
    """The decode step runs only in libdn's own kernels; the library GEMMs are the prompt path's."""
    out = subprocess.run(["readelf", "-d", built[0]], capture_output=True, text=True, check=True).stdout
    needed = re.findall(r"\(NEEDED\).*\[(.*)\]", out)
    assert not any("blas" in n for n in needed), needed


def test_binding_names_match():
    import gated_deltanet_layer_dn_amd as dn
    assert set(dn.EXPORTED) == _declared(HDR)
    assert set(dn.PREFILL_EXPORTED) == _declared(PHDR)
    for n in dn.EXPORTED + dn.PREFILL_EXPORTED:
        assert callable(getattr(dn, n))


def test_binding_constants_match_the_headers():
    """Every #define of the headers has the same value in the binding."""
    import gated_deltanet_layer_dn_amd as dn
    defs = {}
    for path in (HDR, PHDR):
        src = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        defs.update(re.findall(r"^#define\s+(DN_\w+)\s+(-?\d+)u?\s*$", src, flags=re.M))
    assert {"DN_OK", "DN_E_INVAL", "DN_X_RMSNORM", "DN_GATES_ON_DEVICE", "DN_PREFILL_MAX_TOKENS"} <= set(defs)
    for name, val in defs.items():
        assert getattr(dn, name) == int(val), name
