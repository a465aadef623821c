"""Critical-path breakdown of the whole-stack kernel, per layer, from an instrumented build.

    python -m gated_deltanet_layer_dn_amd.phases build           # on any machine with hipcc
    python -m gated_deltanet_layer_dn_amd.phases run [config]    # on the card (default: stack)

`build` compiles libdn_timers.so beside libdn.so with DN_PHASE_TIMERS: every workgroup records the
100 MHz wall clock at eight phase boundaries of each layer into LDS (the instrumentation holds no
registers across the phases, so the kernel's register allocation is the production one) and copies
them out when the launch ends. `run` drives twelve decode tokens through that library, reads the
marks of the last one and prints, per layer (median over the inner layers), how long each step of
the chain between workgroups took:

  x_hand    the previous layer's last out_proj row written -> this workgroup has all of x
  split     RMSNorm statistics and the three-term int8 split of x into LDS
  A         in_proj rows of this workgroup (median workgroup)
  A_spread  the slowest workgroup's phase A end minus the median one
  u_hand    the last phase-A end -> a phase-B workgroup has its q, k, v, z, gate rows
  B         the recurrence on the workgroup's state slice, up to its gated readout
  B_spread  the slowest phase-B workgroup minus the median one
  G_hand    the last readout written -> this workgroup has all gated readouts and norm partials
  G_to_C    per-head norm, scale and staging of the readout for phase C
  C         out_proj rows of this workgroup
  C_spread  the slowest workgroup's phase C end minus the median one
  layer     the layer's whole span (last C end of layer l-1 to last C end of layer l)
"""
from __future__ import annotations

import os
import sys

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_TIMERS = os.path.join(PKG, "libdn_timers.so")
TICK_US = 0.01  # the wall clock runs at 100 MHz
# mark indices recorded by the instrumented kernel (DN_MARK in dn_persist.hip)
M_X, M_SPLIT, M_A, M_U, M_B, M_G, M_C0, M_C1 = 1, 2, 3, 4, 15, 6, 7, 8


def build_timers(verbose: bool = False) -> str:
    from gated_deltanet_layer_dn_amd import build
    return build.build(verbose=verbose, out=LIB_TIMERS, defines=["DN_PHASE_TIMERS"], prefill_out=None)


def breakdown(t: np.ndarray, nb: int) -> dict:
    """t: [workgroups][layers][32] marks in microseconds; nb: the workgroups that hold state slices
    (the phase-B ones). Returns the per-layer medians over layers 1..L-2."""
    L = t.shape[1]
    rows = []
    for l in range(1, L - 1):
        prev_c = t[:, l - 1, M_C1].max()
        rows.append({
            "x_hand": np.median(t[:, l, M_X]) - prev_c,
            "split": np.median(t[:, l, M_SPLIT] - t[:, l, M_X]),
            "A": np.median(t[:, l, M_A] - t[:, l, M_SPLIT]),
            "A_spread": t[:, l, M_A].max() - np.median(t[:, l, M_A]),
            "u_hand": np.median(t[:nb, l, M_U]) - t[:, l, M_A].max(),
            "B": np.median(t[:nb, l, M_B] - t[:nb, l, M_U]),
            "B_spread": t[:nb, l, M_B].max() - np.median(t[:nb, l, M_B]),
            "G_hand": np.median(t[:, l, M_G]) - t[:nb, l, M_B].max(),
            "G_to_C": np.median(t[:, l, M_C0] - t[:, l, M_G]),
            "C": np.median(t[:, l, M_C1] - t[:, l, M_C0]),
            "C_spread": t[:, l, M_C1].max() - np.median(t[:, l, M_C1]),
            "layer": t[:, l, M_C1].max() - prev_c,
        })
    return {k: float(np.median([r[k] for r in rows])) for k in rows[0]}


def run(config: str = "stack", n_tokens: int = 12) -> dict:
    out_path = os.path.join(os.environ.get("TMPDIR", "/tmp"), "dn_phase_timers_%d.bin" % os.getpid())
    if not os.path.exists(LIB_TIMERS):
        raise RuntimeError(f"{LIB_TIMERS} is not built: run `python -m gated_deltanet_layer_dn_amd.phases build`")
    os.environ["DN_PHASE_TIMERS"] = out_path  # read by dn_destroy of the instrumented build
    sys.path.insert(0, ROOT)
    import torch

    import dn_inputs as gi
    import gated_deltanet_layer_dn_amd as dn

    if dn._lib is not None and dn.LIB_PATH != LIB_TIMERS:
        raise RuntimeError("another build of libdn is already loaded in this process")
    dn.LIB_PATH = LIB_TIMERS

    if config == "stack_perkey":  # the stack with one decay per key channel (as bench.py builds it)
        cfg = gi.CONFIGS["stack"].replace(name="stack_perkey", flags=gi.DN_X_RMSNORM | gi.DN_ALPHA_PER_KEY)
    elif config == "stack_gates":  # the stack with the gates computed on the card
        cfg = gi.CONFIGS["stack"].replace(name="stack_gates", flags=gi.DN_X_RMSNORM | gi.DN_GATES_ON_DEVICE)
    else:
        cfg = gi.CONFIGS[config]
    layers, stream = gi.generate(cfg, n_tokens=n_tokens)
    st = dn.DeltaNetStack.from_config(cfg, layers)
    try:
        st.set_state(np.stack([l.S0 for l in layers]), np.stack([l.ring0 for l in layers]))
        x = torch.from_numpy(stream.x).cuda()
        a = torch.from_numpy(stream.alpha).cuda()
        b = torch.from_numpy(stream.beta).cuda()
        out = st.new_out()
        for t in range(n_tokens):
            st.step(x[t], a[t], b[t], out)
        torch.cuda.synchronize()
        if st.status() != 0:
            raise RuntimeError("the instrumented run failed on the card")
        nwg = torch.cuda.get_device_properties(0).multi_processor_count  # one workgroup per CU
    finally:
        st.close()  # dn_destroy writes the last launch's marks to out_path
    L = cfg.n_layers
    t = np.fromfile(out_path, dtype=np.uint64).astype(np.int64).reshape(nwg, L, 32) * TICK_US
    os.remove(out_path)
    nb = cfg.n_v_heads * cfg.d_v // 16  # phase-B workgroups: one 128 x 16 slice of a head's state each
    med = breakdown(t, nb)
    med["kernel_span"] = float(t[:, -1, M_C1].max() - t[:, 0, M_X].min())
    return med


def main(argv) -> int:
    mode = argv[1] if len(argv) > 1 else "run"
    if mode == "build":
        print(build_timers(verbose="-v" in argv))
        return 0
    config = argv[2] if len(argv) > 2 else "stack"
    med = run(config)
    print(f"per-layer critical path of the whole-stack kernel ({config}), medians over the inner layers, us:")
    for k, v in med.items():
        print(f"  {k:12s} {v:7.2f}")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
