#!/usr/bin/env python3
"""Decode-throughput benchmark of the gated-DeltaNet stack on one MI355X.

A step is one decode token through the whole stack (every layer: in_proj GEMV, conv + SiLU,
L2 norms, decay, delta rule, readout, gated RMSNorm, out_proj GEMV). The default workload is 30
independent layers at the hybrid-35B DeltaNet shape (d_model 2048, 16 key heads x 128, 32 value
heads x 128, int8 weights with per-row fp32 scales, fp32 32x128x128 state per layer), single
sequence, 200 tokens, synthetic seeded inputs already resident in HBM.

Prints ONE JSON line. Bytes per step = quantised weights + fp32 scales + conv taps + norm weight
+ 2 x fp32 state, over all layers.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = ("gated_deltanet_layer_dn_amd/csrc/dn_persist.hip", "gated_deltanet_layer_dn_amd/csrc/dn_internal.h")


def bench_config(gi, name):
    """The decode workloads: the named configurations, and the stack's variants."""
    stack = gi.CONFIGS["stack"]
    if name == "stack_perkey":  # one decay per key channel
        return stack.replace(name=name, flags=gi.DN_X_RMSNORM | gi.DN_ALPHA_PER_KEY)
    if name == "stack_gates":  # the gates computed on the card
        return stack.replace(name=name, flags=gi.DN_X_RMSNORM | gi.DN_GATES_ON_DEVICE)
    if name == "stack_heads48":  # 48 value heads over the 16 key heads (the whole-stack kernel's two-wave form)
        return stack.replace(name=name, n_v_heads=48)
    if name == "stack_dim256":  # heads of 256: 8 key heads and 16 value heads of 256 columns
        return stack.replace(name=name, n_k_heads=8, d_k=256, n_v_heads=16, d_v=256)
    return gi.CONFIGS[name]


def create_reporting_path(dn, cfg, layers):
    """Create the handle with DN_VERBOSE set and read which execution path the library chose
    from the line it prints on stderr (file descriptor 2)."""
    import tempfile
    os.environ["DN_VERBOSE"] = "1"
    sys.stderr.flush()
    saved = os.dup(2)
    with tempfile.TemporaryFile() as tf:
        os.dup2(tf.fileno(), 2)
        try:
            st = dn.DeltaNetStack.from_config(cfg, layers)
        finally:
            os.dup2(saved, 2)
            os.close(saved)
            del os.environ["DN_VERBOSE"]
        tf.seek(0)
        text = tf.read().decode(errors="replace")
    path = next((p for p in ("whole-stack kernel", "batched kernels") if p in text), "per-layer kernels")
    return st, path


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM-side bytes per launch of the whole-stack kernel, from the committed counter summary.

    The summary holds FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by what the same counter
    read for a plain copy of known size, and the hash of the kernel source it was taken on; once
    the source differs the figure no longer describes this kernel and None is returned."""
    path = os.path.join(ROOT, "profiles", f"k_persist_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="stack",
                    choices=["stack", "stack_int4", "stack_perkey", "stack_gates", "stack_heads48", "stack_dim256",
                             "layer", "batched", "prefill"])
    ap.add_argument("--prompt", type=int, default=2048, help="prompt length of --config prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 10 times (reference for the HBM byte counters)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the read-stream and read-modify-write ceilings of the device (libdn_probe) and print them")
    ap.add_argument("--exchange", action="store_true",
                    help="only measure the latency of hand-offs between workgroups (libdn_probe) and print it")
    ap.add_argument("--cpu-leg", type=int, default=0, metavar="THREADS",
                    help=argparse.SUPPRESS)  # internal: the oracle sample, run in a child process
    args = ap.parse_args()

    if args.cpu_leg:
        return cpu_leg(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the decode step of one stack "
                                   "is measured on a single MI355X (--gpus 1)"}))
        sys.exit(2)

    # the CPU baseline first, in child processes that never touch the GPU (OpenMP settings are
    # read when the oracle's library loads)
    cpu = None if args.no_cpu_baseline or args.ceiling or args.copy_calibration or args.exchange else cpu_baseline(args)

    import numpy as np
    import torch

    if args.ceiling:
        print(json.dumps(read_ceiling()), flush=True)
        print(json.dumps(rmw_ceiling()), flush=True)
        return

    if args.exchange:
        print(json.dumps(exchange_latency()), flush=True)
        return

    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": src.numel() * 4,
                          "copy_calibration_bytes_written_per_launch": dst.numel() * 4}))
        return

    import dn_inputs as gi
    import gated_deltanet_layer_dn_amd as dn

    if args.config == "prefill":
        return bench_prefill(args, gi, dn, cpu)
    cfg = bench_config(gi, args.config)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    t0 = time.time()
    layers, stream = gi.generate(cfg)
    log(f"[bench] generated {cfg.name}: L={cfg.n_layers} B={cfg.batch} T={cfg.n_tokens} in {time.time() - t0:.1f}s")

    st, path = create_reporting_path(dn, cfg, layers)
    log(f"[bench] execution path: {path}")
    S0 = np.ascontiguousarray(np.stack([l.S0 for l in layers]))
    R0 = np.ascontiguousarray(np.stack([l.ring0 for l in layers]))
    S0d = torch.from_numpy(S0).to(dev)
    R0d = torch.from_numpy(R0).to(dev)
    st.set_state(S0d, R0d)
    x = torch.from_numpy(np.ascontiguousarray(stream.x)).to(dev)
    al = torch.from_numpy(np.ascontiguousarray(stream.alpha)).to(dev)
    be = torch.from_numpy(np.ascontiguousarray(stream.beta)).to(dev)
    T = cfg.n_tokens
    outs = torch.empty((max(args.steps, 1), cfg.n_layers, cfg.batch, cfg.d_model), dtype=torch.float32, device=dev)
    scratch_out = st.new_out()

    # an untimed run of the same steps from the initial state, kept for the bitwise comparison
    # with the timed run (the decode step is deterministic run to run)
    ref_outs = torch.empty_like(outs)
    for i in range(args.steps):
        t = i % T
        st.step(x[t], al[t], be[t], ref_outs[i])
    torch.cuda.synchronize()
    # warmup, then restart from the initial state so the timed run is the workload itself
    for i in range(args.warmup):
        t = i % T
        st.step(x[t], al[t], be[t], scratch_out)
    torch.cuda.synchronize()
    st.set_state(S0d, R0d)
    torch.cuda.synchronize()

    # every launch goes to this stream; an event after each one brackets each launch
    stream_t = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream_t)
    for i in range(args.steps):
        t = i % T
        st.step(x[t], al[t], be[t], outs[i], stream=stream_t)
        evs[i + 1].record(stream_t)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1])
    launch_us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)])
    sec = ms / 1e3
    steps_per_s = args.steps / sec
    tokens_per_s = steps_per_s * cfg.batch
    bytes_step = cfg.metric_bytes_per_step()
    gbs = bytes_step * args.steps / sec / 1e9
    assert torch.isfinite(outs).all().item(), "non-finite output"
    assert st.status() == dn.DN_OK, "a step failed on the device"
    same = bool(torch.equal(outs, ref_outs))
    log(f"[bench] timed run bitwise equal to the untimed run: {same}")
    log(f"[bench] {args.steps} steps in {ms:.3f} ms: {ms * 1e3 / args.steps:.2f} us/step, "
        f"{tokens_per_s:.1f} tok/s, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f})")

    # Dominant kernel: for single-sequence stacks one whole-stack launch per step moves all the
    # metric bytes, so its algorithmic bytes per launch are the step's; elsewhere (per-layer
    # kernels) the step's rate is reported.
    whole_stack = path == "whole-stack kernel"
    kern_us = float(launch_us.mean())
    achieved = bytes_step / (kern_us * 1e-6) / 1e9 if whole_stack else gbs
    traffic = measured_traffic(cfg.name) if whole_stack else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_persist (whole-stack decode, one launch per token)" if whole_stack
                          else f"{path} (whole step)",
                "launch_us_mean": round(kern_us, 2), "launch_us_min": round(float(launch_us.min()), 2),
                "launch_us_max": round(float(launch_us.max()), 2), "bytes_per_launch": bytes_step}
    log(f"[bench] launch time mean {kern_us:.2f} us (min {launch_us.min():.2f}, max {launch_us.max():.2f})")
    # measured ceiling of this step's bytes: the weights at the read-stream ceiling, the state (read,
    # updated and written back) at the read-modify-write ceiling, both measured here
    ceil = read_ceiling()
    rmw = rmw_ceiling()
    w_bytes = cfg.n_layers * cfg.weight_bytes_per_layer()
    s_bytes = cfg.n_layers * 2 * cfg.state_bytes_per_layer()
    ceil_s = w_bytes / (ceil["read_ceiling_gbs"] * 1e9) + s_bytes / (rmw["rmw_ceiling_gbs"] * 1e9)
    ceil_gbs = bytes_step / ceil_s / 1e9
    roofline["measured_ceiling"] = round(ceil_gbs, 1)
    roofline["frac_of_measured_ceiling"] = round(achieved / ceil_gbs, 4)
    roofline["read_ceiling_gbs"] = ceil["read_ceiling_gbs"]
    roofline["rmw_ceiling_gbs"] = rmw["rmw_ceiling_gbs"]
    log(f"[bench] read-stream ceiling {ceil['read_ceiling_gbs']:.0f} GB/s, read-modify-write ceiling "
        f"{rmw['rmw_ceiling_gbs']:.0f} GB/s; this step's bytes at those: {ceil_gbs:.0f} GB/s, "
        f"{ceil_s * 1e6:.1f} us: {100 * roofline['frac_of_measured_ceiling']:.1f}% of it")

    rec = {
        "metric": "DeltaNet decode tokens/s (30-layer stack) + achieved HBM GB/s % of peak",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if cfg.weight_bits == 8 else "int4",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.n_layers} layers x d_model {cfg.d_model}, "
                               f"{cfg.n_k_heads}x{cfg.d_k} key / {cfg.n_v_heads}x{cfg.d_v} value heads, "
                               f"batch {cfg.batch}, {T} tokens, {cfg.weight_bits}-bit weights",
                   "layers": cfg.n_layers, "batch": cfg.batch, "tokens": T,
                   "bytes_per_step": bytes_step},
        "hbm_gbs": round(gbs, 1),
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "timed_equals_untimed": same,
        "device": f"{props.name} {getattr(props, 'gcnArchName', '')}".strip(),
    }
    st.close()
    print(json.dumps(rec), flush=True)


def read_ceiling(gib: int = 2, reps: int = 4):
    """The read-stream ceiling of the device: a plain streaming read of `gib` GiB (beyond the
    last-level cache) with every compute unit, over a few grid sizes and loads in flight, timed with
    HIP events; the best rate of all runs after a warm-up run of each shape."""
    import ctypes

    import torch

    import gated_deltanet_layer_dn_amd as dn
    lib = ctypes.CDLL(dn.PROBE_LIB_PATH)
    lib.dn_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p]
    lib.dn_probe_read_stream.restype = ctypes.c_int
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(cus * 32, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    best, shape = 0.0, None
    for blocks in (cus * 4, cus * 8, cus * 16, cus * 32):
        for inflight in (4, 8, 16):
            for r in range(reps + 1):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                rc = lib.dn_probe_read_stream(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, inflight,
                                              st.cuda_stream)
                e1.record(st)
                torch.cuda.synchronize()
                assert rc == 0, rc
                rate = nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
                if r and rate > best:  # the first run of each shape warms up
                    best, shape = rate, (blocks, inflight)
    del buf
    return {"read_ceiling_gbs": round(best, 1), "bytes": nbytes, "blocks": shape[0], "loads_in_flight": shape[1],
            "frac_of_peak": round(best / HBM_PEAK_GBS, 4)}


def rmw_ceiling(gib: int = 2, reps: int = 4):
    """The read-modify-write ceiling of the device: an in-place stream over `gib` GiB (beyond the
    last-level cache), every piece read and written back with nontemporal accesses, over a few grid
    sizes and pieces in flight; bytes counted both ways (read + written), best rate after a warm-up
    run of each shape."""
    import ctypes

    import torch

    import gated_deltanet_layer_dn_amd as dn
    lib = ctypes.CDLL(dn.PROBE_LIB_PATH)
    lib.dn_probe_rmw_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.dn_probe_rmw_stream.restype = ctypes.c_int
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream()
    best, shape = 0.0, None
    for blocks in (cus * 4, cus * 8, cus * 16, cus * 32):
        for inflight in (4, 8, 16):
            for r in range(reps + 1):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                rc = lib.dn_probe_rmw_stream(buf.data_ptr(), nbytes, blocks, inflight, st.cuda_stream)
                e1.record(st)
                torch.cuda.synchronize()
                assert rc == 0, rc
                rate = 2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
                if r and rate > best:
                    best, shape = rate, (blocks, inflight)
    del buf
    return {"rmw_ceiling_gbs": round(best, 1), "bytes": 2 * nbytes, "blocks": shape[0], "pieces_in_flight": shape[1],
            "frac_of_peak": round(best / HBM_PEAK_GBS, 4)}


def exchange_latency(rounds: int = 2000):
    """What a hand-off between workgroups costs on this device (libdn_probe's dn_probe_exchange, 256
    workgroups of 768 threads, device-coherent polls as in the whole-stack kernel): a one-word ping
    between workgroup 0 and workgroup 8 (the same XCD under the dispatcher's round-robin placement)
    or 1 (another XCD), and a 256-way all-gather of 2048 and 4096 words; each with the device
    otherwise quiet and with eight waves per compute unit streaming reads at 3 loads in flight per
    lane, as the weight prefetch of the whole-stack kernel does. Microseconds: one way for the ping,
    per round (median and slowest workgroup) for the all-gather."""
    import ctypes

    import numpy as np
    import torch

    import gated_deltanet_layer_dn_amd as dn
    lib = ctypes.CDLL(dn.PROBE_LIB_PATH)
    lib.dn_probe_exchange.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.dn_probe_exchange.restype = ctypes.c_int
    nwg = torch.cuda.get_device_properties(0).multi_processor_count
    words = torch.zeros(2 * 8 * 4096, dtype=torch.int32, device="cuda:0")
    sbytes = 1 << 30
    stream_buf = torch.ones(sbytes // 4, dtype=torch.float32, device="cuda:0")
    ticks = torch.zeros(nwg, dtype=torch.int64, device="cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(nwg * 8, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()

    def run(mode, arg, sif):
        words.zero_()
        ticks.zero_()
        err.zero_()
        torch.cuda.synchronize()
        rc = lib.dn_probe_exchange(mode, arg, rounds, sif, words.data_ptr(), words.numel() * 4, stream_buf.data_ptr(),
                                   sbytes, ticks.data_ptr(), err.data_ptr(), sink.data_ptr(), nwg, st.cuda_stream)
        torch.cuda.synchronize()
        assert rc == 0, rc
        if int(err.item()) != 0:
            return None  # a bounded wait ran out (the grid was not resident at once)
        t = ticks.cpu().numpy().astype(np.float64) * 0.01  # 100 MHz ticks -> us
        if mode == 0:
            return round(float(t[0]) / (2 * rounds), 3)
        return {"median": round(float(np.median(t)) / rounds, 3), "slowest": round(float(t.max()) / rounds, 3)}

    out = {"workgroups": nwg, "rounds": rounds}
    for sif, tag in ((0, "quiet"), (3, "streaming")):
        out[tag] = {"ping_same_xcd_us": run(0, 8, sif), "ping_other_xcd_us": run(0, 1, sif),
                    "allgather_2048_us": run(1, 2048, sif), "allgather_4096_us": run(1, 4096, sif)}
    del stream_buf
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(args):
    """Child process: the oracle over a bounded sample of the workload, with the OpenMP settings
    of its environment; prints one JSON line."""
    import dn_inputs as gi
    import oracle as orc
    if args.config == "prefill":
        cfg = gi.CONFIGS["stack"].replace(name="prefill", n_tokens=args.prompt)
    else:
        cfg = bench_config(gi, args.config)
    layers, stream = gi.generate(cfg)
    orc.lib()
    # calibrate on one token, then run a bounded sample of the same workload
    c0 = time.time()
    orc.run(cfg, layers, stream, n_tokens=1)
    per_tok = max(time.time() - c0, 1e-3)
    n = int(max(1, min(cfg.n_tokens, args.cpu_seconds / per_tok)))
    c0 = time.time()
    orc.run(cfg, layers, stream, n_tokens=n)
    csec = time.time() - c0
    print(json.dumps({"tokens": n, "seconds": csec, "threads": orc.threads(), "batch": cfg.batch,
                      "of_tokens": cfg.n_tokens}), flush=True)


def cpu_baseline(args):
    """The oracle timed on the host's cores: all of them (OMP_PLACES=cores, OMP_PROC_BIND=close),
    then one thread, each on a bounded sample of the same workload, in child processes."""
    import subprocess
    allc = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    res = {}
    for n, secs in ((allc, args.cpu_seconds), (1, max(2.0, args.cpu_seconds / 3))):
        env = dict(os.environ, OMP_NUM_THREADS=str(n), OMP_PLACES="cores", OMP_PROC_BIND="close")
        cmd = [sys.executable, os.path.abspath(__file__), "--cpu-leg", str(n), "--config", args.config,
               "--prompt", str(args.prompt), "--cpu-seconds", str(secs)]
        r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            log(f"[bench] oracle leg with {n} thread(s) failed: {r.stderr[-500:]}")
            return None
        res[n] = json.loads(r.stdout.strip().splitlines()[-1])
        log(f"[bench] oracle: {res[n]['tokens']} tokens in {res[n]['seconds']:.1f}s on {res[n]['threads']} thread(s)")
    a, o = res[allc], res[1]
    return {"value": round(a["tokens"] * a["batch"] / a["seconds"], 3), "unit": "tokens/s", "cores": a["threads"],
            "kind": "oracle",
            "sample": f"first {a['tokens']} of {a['of_tokens']} tokens of the same workload (fp64 oracle, "
                      f"{a['seconds']:.1f} s, OMP_PLACES=cores OMP_PROC_BIND=close)",
            "one_thread_value": round(o["tokens"] * o["batch"] / o["seconds"], 3),
            "one_thread_sample": f"first {o['tokens']} tokens ({o['seconds']:.1f} s)",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def bench_prefill(args, gi, dn, cpu):
    """Prompt throughput: one step is a prompt of --prompt tokens through the 30-layer stack
    (dn_prefill), starting from the seeded initial states each time (the reset is outside the
    timed region). Synthetic inputs of the stack workload's distributions."""
    import numpy as np
    import torch

    base = gi.CONFIGS["stack"]
    T = args.prompt
    cfg = base.replace(name="prefill", n_tokens=T)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    t0 = time.time()
    layers, stream = gi.generate(cfg)
    log(f"[bench] generated prefill workload: L={cfg.n_layers} prompt {T} tokens in {time.time() - t0:.1f}s")
    st, path = create_reporting_path(dn, cfg, layers)
    S0d = torch.from_numpy(np.ascontiguousarray(np.stack([l.S0 for l in layers]))).to(dev)
    R0d = torch.from_numpy(np.ascontiguousarray(np.stack([l.ring0 for l in layers]))).to(dev)
    x = torch.from_numpy(np.ascontiguousarray(stream.x[:, 0])).to(dev)
    al = torch.from_numpy(np.ascontiguousarray(stream.alpha[:, :, 0])).to(dev)
    be = torch.from_numpy(np.ascontiguousarray(stream.beta[:, :, 0])).to(dev)
    out = torch.empty((cfg.n_layers, T, cfg.d_model), dtype=torch.float32, device=dev)
    stream_t = torch.cuda.current_stream()
    for _ in range(args.warmup):
        st.set_state(S0d, R0d)
        st.prefill(x, al, be, out, stream=stream_t)
    torch.cuda.synchronize()
    times = []
    for _ in range(args.steps):
        st.set_state(S0d, R0d)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream_t)
        st.prefill(x, al, be, out, stream=stream_t)
        e1.record(stream_t)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    assert torch.isfinite(out).all().item(), "non-finite output"
    ms = float(np.sum(times))
    per = float(np.mean(times))
    tok_s = T / (per / 1e3)
    # algorithmic work of the two projections: 2 flops per weight per token
    w_per_layer = cfg.d_model * (2 * cfg.qk_dim + 2 * cfg.v_dim) + cfg.v_dim * cfg.d_model
    proj_flops = 2.0 * w_per_layer * T * cfg.n_layers
    log(f"[bench] prefill of {T} tokens x {cfg.n_layers} layers: {per:.3f} ms ({tok_s:.0f} prompt tokens/s); "
        f"projections {proj_flops / (per * 1e-3) / 1e12:.1f} TFLOP/s algorithmic")
    rec = {
        "metric": "DeltaNet prefill prompt tokens/s (30-layer stack)",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(per, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"prefill: a {T}-token prompt through 30 layers x d_model {cfg.d_model}, "
                               f"{cfg.n_k_heads}x{cfg.d_k} key / {cfg.n_v_heads}x{cfg.d_v} value heads, 8-bit weights",
                   "layers": cfg.n_layers, "prompt_tokens": T},
        "projection_tflops_algorithmic": round(proj_flops / (per * 1e-3) / 1e12, 2),
        # the prompt's dominant work is the two projections on the int8 matrix cores: their
        # algorithmic ops (2 per weight per token) over the whole step's time, against the int8
        # dense peak; the three-term split executes three times those ops
        "roofline": {"bound": "mfma", "achieved": round(proj_flops / (per * 1e-3) / 1e12, 1), "peak": 5000.0,
                     "unit": "TOP/s (int8)", "frac": round(proj_flops / (per * 1e-3) / 1e12 / 5000.0, 4),
                     "traffic": None, "kernel": "dn_prefill step (every kernel of the prompt)",
                     "executed_int8_tops": round(3 * proj_flops / (per * 1e-3) / 1e12, 1)},
        "cpu_baseline": cpu,
        "device": f"{props.name} {getattr(props, 'gcnArchName', '')}".strip(),
    }
    st.close()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
