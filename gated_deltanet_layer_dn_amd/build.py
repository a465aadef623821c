"""Build libdn.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["dn_kernels.hip", "dn_persist.hip", "dn_batched.hip", "dn_prefill.hip", "dn_lt.cpp", "dn_api.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
# the prefill projections with 8-bit weights call the library's int8 GEMMs
LIBS = ["-lhipblaslt"]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile libdn.so; `defines` adds preprocessor macros (DN_PHASE_TIMERS for an
    instrumented build written to `out`)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                                          "-o", tmp] + sources() + LIBS
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + errs)
    if verbose and errs.strip():
        print(errs, flush=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
