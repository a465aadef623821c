"""Build libdn.so, libdn_prefill.so and libdn_probe.so (HIP, gfx950) in-tree with hipcc.

libdn.so holds the five calls of include/dn.h; libdn_prefill.so holds the prompt path of
include/dn_prefill.h; libdn_probe.so holds the measurement probe of include/dn_probe.h. Each
source is compiled once into an object (in parallel); the kernels two libraries need are linked
into each of them.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdn.so")
LIB_PREFILL = os.path.join(PKG, "libdn_prefill.so")
LIB_PROBE = os.path.join(PKG, "libdn_probe.so")
OBJ = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# sources of each library
DN_SOURCES = ["dn_kernels.hip", "dn_persist.hip", "dn_batched.hip", "dn_api.cpp"]
PREFILL_SOURCES = ["dn_kernels.hip", "dn_batched.hip", "dn_prefill.hip", "dn_lt.cpp", "dn_prefill_api.cpp"]
PROBE_SOURCES = ["dn_probe.hip"]  # measurement only: the read-stream ceiling
SOURCES = sorted(set(DN_SOURCES) | set(PREFILL_SOURCES) | set(PROBE_SOURCES))

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
# the prefill projections with 8-bit weights call the library's int8 GEMMs
PREFILL_LIBS = ["-lhipblaslt"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + errs)
    if verbose and errs.strip():
        print(errs, flush=True)


def _compile(src: str, obj: str, defines, verbose: bool):
    cmd = [HIPCC, "-c"] + FLAGS + ["-D" + d for d in defines] + [
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", obj, os.path.join(CSRC, src)]
    _run(cmd, verbose)


def _link(objs, out: str, libs, verbose: bool):
    tmp = out + ".tmp%d" % os.getpid()
    # -z defs: a symbol left undefined (a kernel the host pass did not emit, say) fails the link
    # here rather than the library's load
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs + libs, verbose)
    os.replace(tmp, out)


def build(verbose: bool = False, out: str = LIB, defines=(), prefill_out: str | None = LIB_PREFILL) -> str:
    """Compile libdn.so (to `out`), and libdn_prefill.so (to `prefill_out`) and libdn_probe.so
    unless prefill_out is None;
    `defines` adds preprocessor macros (DN_PHASE_TIMERS for an instrumented build)."""
    tag = "%d_%s" % (os.getpid(), "_".join(defines) or "std")
    odir = os.path.join(OBJ, tag)
    os.makedirs(odir, exist_ok=True)
    need = SOURCES if prefill_out else DN_SOURCES
    objs = {s: os.path.join(odir, s.rsplit(".", 1)[0] + ".o") for s in need}
    with cf.ThreadPoolExecutor(max_workers=min(len(need), os.cpu_count() or 4)) as ex:
        for f in [ex.submit(_compile, s, objs[s], defines, verbose) for s in need]:
            f.result()
    _link([objs[s] for s in DN_SOURCES], out, [], verbose)
    if prefill_out:
        _link([objs[s] for s in PREFILL_SOURCES], prefill_out, PREFILL_LIBS, verbose)
        _link([objs[s] for s in PROBE_SOURCES], LIB_PROBE, [], verbose)
    for o in objs.values():
        os.remove(o)
    os.rmdir(odir)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
