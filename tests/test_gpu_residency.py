"""The engine's residency protocol (include/dn_residency.h) over the real libraries on the card.

The page "qwen36: run the DeltaNet layer end to end on the card", section "What the PR does", Engine
paragraph, keeps the host arrays canonical with the fresh/ahead flags; a failing device step pulls
what the card holds and the engine continues on the host (section "Verified", first bullet: the host
copy stays untouched while the card advances, and a failing step pulls and continues on the host).

tests/residency/gpu_engine.c is such an engine, in checked mode, over libdn: twelve tokens through a
3-layer stack on the whole-stack kernel, with
  * token 3: dn_step fails at once (DN_FAULT_STEP): nothing of the token ran; the engine pulls and runs
    the token on the host (the oracle's layer step stands for the engine's host path);
  * token 5: a host step on purpose, after a pull;
  * token 9: the launch abandons its token on the device (DN_FAULT_STALL: every hand-off between
    workgroups gets one poll round); the library keeps the state from before the token, the checked
    step reports the failure for that very token, and the engine runs it on the host;
  * the other tokens on the card, each device step after a host step re-arming the handle by its upload.
Every token's output (all layers) and the final state and history are compared with the oracle run
over all twelve tokens; the transfers are counted against the protocol."""
import os
import subprocess

import numpy as np
import pytest

import dn_inputs as gi
import oracle as orc

from gpu_util import OUT_TOL, STATE_TOL, out_err, state_err

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gated_deltanet_layer_dn_amd")
ORA = os.path.join(ROOT, "oracle")
SRC = os.path.join(ROOT, "tests", "residency", "gpu_engine.c")


def _build(tmp):
    orc.build(force=False)
    exe = os.path.join(tmp, "gpu_engine")
    rp = f"-Wl,-rpath,{PKG}:{ORA}:/opt/rocm/lib"
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", "-o", exe, SRC, "-L", PKG, "-l:libdn.so", "-l:libdn_prefill.so", "-L", ORA,
           "-l:libdn_oracle.so", "-L", "/opt/rocm/lib", "-lamdhip64", "-lm", rp]
    subprocess.check_call(cmd)
    return exe


def _write_inputs(tmp, cfg, layers, stream):
    with open(os.path.join(tmp, "dims.txt"), "w") as f:
        f.write(f"{cfg.d_model} {cfg.n_k_heads} {cfg.d_k} {cfg.n_v_heads} {cfg.d_v} {cfg.conv_k} {cfg.n_layers} "
                f"{cfg.n_tokens} {cfg.weight_bits} {cfg.flags} {cfg.eps_l2!r} {cfg.eps_rms!r} {cfg.q_scale!r}\n")
    for l, lay in enumerate(layers):
        for name in ("w_in", "s_in", "conv_w", "norm_w", "w_out", "s_out"):
            np.ascontiguousarray(getattr(lay, name)).tofile(os.path.join(tmp, f"{name}_{l}.bin"))
    np.ascontiguousarray(np.stack([l.S0 for l in layers]), np.float32).tofile(os.path.join(tmp, "S0.bin"))
    np.ascontiguousarray(np.stack([l.ring0 for l in layers]), np.float32).tofile(os.path.join(tmp, "ring0.bin"))
    for name in ("x", "alpha", "beta"):
        np.ascontiguousarray(getattr(stream, name), np.float32).tofile(os.path.join(tmp, f"{name}.bin"))


def test_engine_over_the_libraries(tmp_path):
    cfg = gi.custom("residency_gpu", d_model=1024, n_k_heads=4, d_k=128, n_v_heads=8, d_v=128, n_layers=3,
                    n_tokens=12, flags=gi.DN_X_RMSNORM, ring_std=1.0)
    layers, stream = gi.generate(cfg)
    tmp = str(tmp_path)
    exe = _build(tmp)
    _write_inputs(tmp, cfg, layers, stream)
    env = dict(os.environ, DN_FAULT_STEP="4", DN_FAULT_STALL="9", DN_VERBOSE="1")
    print("[residency] engine: 12 tokens, 3 layers, faults at dn_step 4 (at once) and 9 (on the device)", flush=True)
    r = subprocess.run([exe, tmp], env=env, capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "engine done" in r.stdout
    rep = dict(l.split(" ", 1) for l in open(os.path.join(tmp, "report.txt")).read().splitlines())
    print("[residency] report:", rep, flush=True)
    assert rep["where"] == "dddhdhdddhdd"
    rcs = [int(v) for v in rep["rcs"].split()]
    assert rcs[3] == -5 and rcs[9] == -3 and all(v == 0 for i, v in enumerate(rcs) if i not in (3, 9))
    # uploads before tokens 0, 4, 6, 10; downloads at the two failures, the host step and the end
    assert int(rep["pushes"]) == 4 and int(rep["pulls"]) == 4
    assert rep["host_untouched"] == "1" and rep["final_pull"] == "0"

    T, L, D = cfg.n_tokens, cfg.n_layers, cfg.d_model
    ref_out, ref_S, ref_H = orc.run(cfg, layers, stream)
    outs = np.fromfile(os.path.join(tmp, "out.bin"), np.float64).reshape(T, L, 1, D)
    S = np.fromfile(os.path.join(tmp, "S_final.bin"), np.float32).reshape(ref_S.shape)
    H = np.fromfile(os.path.join(tmp, "ring_final.bin"), np.float32).reshape(ref_H.shape)
    e = max(out_err(outs[:, l], ref_out[:, l]) for l in range(L))
    es, eh = state_err(S, ref_S), state_err(H, ref_H)
    per_tok = [max(out_err(outs[t:t + 1, l], ref_out[t:t + 1, l]) for l in range(L)) for t in range(T)]
    print("[residency] per-token output error: " + " ".join(f"{v:.1e}" for v in per_tok), flush=True)
    print(f"[residency] out {e:.2e} state {es:.2e} ring {eh:.2e}", flush=True)
    assert e <= OUT_TOL and es <= STATE_TOL and eh <= STATE_TOL
