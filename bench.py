#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

A step is one attn_fwd call: the whole fused path (load, Q K^T, mask, online
softmax, P V, normalise, store) over one batch of synthetic inputs already
resident in HBM.  Prints ONE JSON line.  By default the line is quoted on the
largest workload, B=8 H=32 S=512 D=128 causal; besides the main (warm)
record it carries a "cold" record (the same workload cycling through
--cold-sets copies of its inputs, more bytes between two uses of a set than the
256 MB Infinity Cache holds), a "workloads" list with every one of the five
workloads timed the same way, and the shader clock sampled while the timed
steps ran.

    python bench.py [--steps K] [--warmup W] [--workload C] [--rotate R] [--eager]
    python bench.py --suite            # all five workloads, warm and cold

Timing protocol (after "An Optimal Mapper Meets a Real GPU", section
"Experiment one": CUDA-event timing over many interleaved reps on an
exclusively held GPU, and the cold-start lesson of arXiv 2609.33916 section
2.3: one process, untimed warmup first):
  * W untimed warm-up calls;
  * the timed region: the K calls captured once into a HIP graph and replayed
    (untimed once, then between two events on the launch stream, with a
    synchronize on both sides) -> ms_per_step, the throughput `value` and the
    roofline's launch duration; --eager times K host launches instead;
  * a second pass brackets every call with its own pair of HIP events on the
    launch stream -> per-call median/p10/p90 (host launch latency included).
With --rotate R the calls cycle through R independent input sets (R*inputs
larger than the 256 MB Infinity Cache gives HBM-cold inputs); the default
R = 1 re-reads the same buffers, so inputs are largely cache-resident.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd µs/call + effective TFLOP/s (% FP16 MFMA peak), 1 MI355X"
# --path bwd times the backward (dQ, dK, dV), so its line carries its own name
METRIC_BWD = "attention bwd µs/call + effective TFLOP/s of the five products (% FP16 MFMA peak), 1 MI355X"

# MI355X published peaks (dense): FP16 MFMA 2.5 PFLOP/s, here 256 CU x 2.4 GHz x
# 4096 FLOP/clk/CU = 2516.6 TFLOP/s; HBM3E 8 TB/s.
PEAK_FP16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
PEAK_HBM_GBS = 8000.0
SPIN_CYCLES = 2_000_000  # about 1 ms of GPU-side spin ahead of each suite round


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--workload", type=int, default=4,
                   help="1..5 (default 4: B=8 H=32 S=512 D=128 causal, the largest)")
    p.add_argument("--rotate", type=int, default=1,
                   help="cycle through this many independent input sets")
    p.add_argument("--path", choices=["fused", "unfused", "splitkv", "decode", "bwd"],
                   default="fused")
    p.add_argument("--decode", type=int, default=1,
                   help="decode path: 1..3, the decode workload (Sq rows against Sk keys)")
    p.add_argument("--splits", type=int, default=3,
                   help="split-KV path: chunks of the longest key range (D = 512 only)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", action="store_true",
                   help="time the K steps as K host launches instead of one HIP graph replay")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum wall time of the oracle timing loop")
    p.add_argument("--cold-sets", type=int, default=6,
                   help="fused path: input buffers cycled by the cold record (each set is "
                        "a copy of the inputs in its own memory; 0 skips the record)")
    p.add_argument("--no-workloads", action="store_true",
                   help="fused path: skip the per-workload records of all five workloads")
    p.add_argument("--suite", action="store_true",
                   help="time all five workloads in one process, interleaved round by round "
                        "(warm and cold), plus the oracle at 1 thread and at all cores; prints "
                        "one JSON line with a row per workload instead of the bench line")
    p.add_argument("--rounds", type=int, default=300, help="suite: timed rounds")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of this many MiB (the reference "
                        "kernel for scaling HBM byte counters) and exit")
    return p.parse_args()


def cpu_baseline_bwd(w, min_seconds):
    """The float64 oracle's backward on this host's cores, over the first
    heads of the workload (as many as fit about min_seconds), scaled to the
    algorithmic FLOPs of those heads."""
    import oracle
    from scaled_dot_product_attn_amd import inputs
    oracle.build(force=False)
    q, k, v = w.qkv()
    do = inputs.normal_f16(w.seed_base + 50, w.shape, 1.0)
    threads = oracle.max_threads()
    h = 1
    while True:
        sl = (slice(0, 1), slice(0, h))
        t0 = time.perf_counter()
        oracle.attn_bwd(q[sl], k[sl], v[sl], do[sl], w.causal, w.scale, nthreads=threads)
        sec = time.perf_counter() - t0
        if sec >= min_seconds or h >= w.H:
            break
        h = min(w.H, h * 2)
    flops = 2.5 * w.flops() * h / (w.B * w.H)
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds_per_call": sec,
            "sample": f"{h} of the {w.B * w.H} heads of {w.name} (float64 C oracle backward, "
                      f"OpenMP over heads), one call"}


def cpu_baseline(w, min_seconds):
    """The float64 oracle as it stands, on this host's cores, over the whole
    workload (repeated until min_seconds have passed, at least twice)."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    q, k, v = w.qkv()
    threads = oracle.max_threads()
    oracle.attn_fwd(q[:, :1, :64], k[:, :1, :64], v[:, :1, :64], w.causal, w.scale)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.attn_fwd(q, k, v, w.causal, w.scale, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if reps >= 2 and el >= min_seconds:
            break
    sec = el / reps
    del np
    return {"value": w.flops() / sec / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds_per_call": sec,
            "sample": f"whole workload {w.name} (float64 C oracle, OpenMP over rows), "
                      f"{reps} calls"}


def measured_traffic(workload_name, path):
    """HBM bytes per launch from the committed PMC summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by the same counter on a plain copy of known size),
    or None when no summary covers this workload or the kernel sources have
    changed since the counters were taken."""
    import glob
    import hashlib
    if path != "fused":
        return None
    for fn in glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")):
        with open(fn) as f:
            t = json.load(f)
        if t.get("workload") != workload_name:
            continue
        try:
            h = hashlib.sha256(b"".join(open(os.path.join(ROOT, s), "rb").read()
                                        for s in t["kernel_sources"])).hexdigest()
        except OSError:  # a source the counters were taken on is gone
            continue
        if h == t["kernel_source_sha256"]:
            return t["traffic_bytes_per_launch"]
    return None


def shader_clock_mhz():
    """The current shader clock from sysfs (the line marked '*'), or None."""
    import glob
    for fn in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(fn):
                if "*" in line:
                    return int(line.split(":")[1].strip().rstrip("*").strip().lower()
                               .replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            continue
    return None


def suite(args):
    """All five workloads in one process, per the measurement protocol: 20
    untimed calls per workload, then `rounds` rounds with the workloads
    interleaved inside each round, every call bracketed by its own events on
    the launch stream.  Two modes: warm (the same buffers every call) and cold
    (12 rotating input sets, about 1.8 GB between two uses of one set, far
    more than the 256 MB Infinity Cache).  Then the float64 oracle once per
    workload at 1 thread and once at all threads, same inputs."""
    import numpy as np
    import torch
    import scaled_dot_product_attn_amd as attn
    from scaled_dot_product_attn_amd import inputs
    dev = torch.device("cuda:0")
    attn.load_library()
    stream = torch.cuda.current_stream(dev)  # the stream attn.fwd launches on
    ws = sorted(inputs.WORKLOADS.items())
    nsets = 12
    sets = {}
    for c, w in ws:
        sets[c] = []
        for r in range(nsets):
            qkv = w.qkv() if r == 0 else tuple(
                inputs.normal_f16(w.seed_base + 100 * r + t, w.shape, w.sigma) for t in range(3))
            sets[c].append(tuple(torch.from_numpy(x).to(dev) for x in qkv))
    outs = {c: (torch.empty(w.shape, dtype=torch.float16, device=dev),
                torch.empty(w.shape[:3], dtype=torch.float32, device=dev)) for c, w in ws}

    def call(c, w, i):
        q, k, v = sets[c][i]
        o, lse = outs[c]
        attn.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    def timed(cold):
        for c, w in ws:
            for i in range(20):
                call(c, w, i % nsets if cold else 0)
        torch.cuda.synchronize(dev)
        times = {c: [] for c, _ in ws}
        for rnd in range(args.rounds):
            # a GPU-side spin first, so that the host enqueues the whole round
            # before the GPU reaches it: the events then bracket the kernels,
            # not the host's launch latency
            torch.cuda._sleep(SPIN_CYCLES)
            evs = []
            for c, w in ws:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                call(c, w, rnd % nsets if cold else 0)
                b.record(stream)
                evs.append((c, a, b))
            if rnd == args.rounds // 2:
                sclk.append(shader_clock_mhz())  # sampled while the round runs
            torch.cuda.synchronize(dev)
            for c, a, b in evs:
                times[c].append(a.elapsed_time(b) * 1e3)
        rows = []
        digests = {}
        if not cold:
            # output bytes of input set 0, for reproducibility across runs
            for c, w in ws:
                call(c, w, 0)
                torch.cuda.synchronize(dev)
                o, lse = outs[c]
                digests[c] = {"O": inputs.sha256(o.cpu().numpy()),
                              "LSE": inputs.sha256(lse.cpu().numpy())}
        for c, w in ws:
            t = np.sort(np.array(times[c]))
            med = float(np.median(t))
            tf = w.flops() / med / 1e6
            rows.append({"workload": w.name, "us_median": med,
                         "us_p10": float(t[int(0.1 * (len(t) - 1))]),
                         "us_p90": float(t[int(0.9 * (len(t) - 1))]),
                         "tflops": tf, "pct_fp16_peak": 100 * tf / PEAK_FP16_TFLOPS,
                         "alg_GBps": w.alg_bytes() / med / 1e3,
                         **({"out_sha256": digests[c]} if c in digests else {})})
        return rows

    sclk = []
    out = {"suite": "attention forward, five workloads interleaved per round",
           "rounds": args.rounds, "timing": "events around each call, on the launch stream, "
           "behind a GPU-side spin so that the round is enqueued before it runs"}
    out["warm"] = timed(False)
    out["cold"] = timed(True)
    out["sclk_mhz_mid_round"] = sclk
    print(json.dumps(out), flush=True)
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        allt = oracle.max_threads()
        model = None
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        orc = {"cpu": model, "nproc": os.cpu_count(), "threads_all": allt, "rows": []}
        for c, w in ws:
            q, k, v = w.qkv()
            rec = {"workload": w.name}
            for nt in (1, allt):
                t0 = time.perf_counter()
                oracle.attn_fwd(q, k, v, w.causal, w.scale, nthreads=nt)
                rec[f"seconds_{nt}_threads"] = time.perf_counter() - t0
            orc["rows"].append(rec)
            print(json.dumps({"oracle_row": rec}), flush=True)
        out["oracle"] = orc
        print(json.dumps(out), flush=True)

def replay_us(step, steps, dev, stream):
    """Microseconds per step of `steps` calls of step(i) captured once into a
    HIP graph and replayed: once untimed, then between two events on the
    launch stream (a synchronize on both sides)."""
    import torch
    for i in range(min(steps, 5)):
        step(i)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    graph.replay()
    b.record(stream)
    torch.cuda.synchronize(dev)
    del graph
    return a.elapsed_time(b) * 1e3 / steps


def binding_roof(flops, nbytes, us):
    """The roofline of a launch of `flops` and `nbytes` algorithmic bytes that
    takes `us`: the roof whose time at peak is the longer one (FLOPs at the
    FP16 MFMA peak, or the bytes at the HBM peak), and the fraction of it
    reached."""
    if flops / (PEAK_FP16_TFLOPS * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9):
        a = flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": a, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                "frac": a / PEAK_FP16_TFLOPS}
    a = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": a / PEAK_HBM_GBS}


def fused_record(w, us):
    """Per-launch figures of one fused-forward workload at `us` per call."""
    tf = w.flops() / (us * 1e-6) / 1e12
    return {"workload": w.name, "us": us, "tflops": tf,
            "pct_fp16_peak": 100 * tf / PEAK_FP16_TFLOPS,
            "alg_GBps": w.alg_bytes() / (us * 1e-6) / 1e9,
            "roofline": binding_roof(w.flops(), w.alg_bytes(), us)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on exactly one GPU; the attention forward "
              "shards over (batch, head) slices with no exchange, so a multi-GPU "
              "figure is not measured here.", file=sys.stderr)
        sys.exit(2)

    if args.suite:
        suite(args)
        return
    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 10}))
        return
    import scaled_dot_product_attn_amd as attn
    from scaled_dot_product_attn_amd import inputs

    decode = args.path == "decode"
    w = inputs.DECODE_WORKLOADS[args.decode] if decode else inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    attn.load_library()
    sets = []
    for r in range(args.rotate):
        if r == 0:
            q, k, v = w.qkv()
        elif decode:
            q, k, v = inputs.DecodeWorkload(w.name, w.B, w.H, w.Sq, w.Sk, w.D, w.causal,
                                            w.seed_base + 100 * r).qkv()
        else:
            q, k, v = (inputs.normal_f16(w.seed_base + 100 * r + t, w.shape, w.sigma)
                       for t in range(3))
        sets.append(tuple(torch.from_numpy(x).to(dev) for x in (q, k, v)))
    qshape = (w.B, w.H, w.Sq, w.D) if decode else w.shape
    o = torch.empty(qshape, dtype=torch.float16, device=dev)
    lse = torch.empty(qshape[:3], dtype=torch.float32, device=dev)
    ws = None
    if args.path == "unfused":
        ws = torch.empty(attn.unfused_workspace_bytes(w.B, w.H, w.S), dtype=torch.uint8,
                         device=dev)
    elif args.path == "splitkv":
        nbytes = attn.splitkv_workspace_bytes(w.B, w.H, w.S, w.D, w.causal, args.splits)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif decode:
        dsplits = attn.decode_splits(w.B, w.H, w.Sq, w.Sk)
        nbytes = attn.decode_workspace_bytes(w.B, w.H, w.Sq, w.Sk, w.D, w.causal, dsplits)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif args.path == "bwd":
        # the forward's O and LSE of every input set, and dO drawn like Q
        fw = []
        for r, (q, k, v) in enumerate(sets):
            of, lf = attn.fwd(q, k, v, causal=w.causal, scale=w.scale)
            do = torch.from_numpy(inputs.normal_f16(w.seed_base + 50 + 100 * r, w.shape,
                                                    1.0)).to(dev)
            fw.append((of, lf, do))
        grads = tuple(torch.empty(w.shape, dtype=torch.float16, device=dev) for _ in range(3))
        ws = torch.empty(attn.bwd_workspace_bytes(w.B, w.H, w.S, w.D), dtype=torch.uint8,
                         device=dev)

    def step(i):
        q, k, v = sets[i % len(sets)]
        if args.path == "fused":
            attn.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        elif args.path == "unfused":
            attn.fwd_unfused(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse,
                             workspace=ws)
        elif args.path == "splitkv":
            attn.fwd_splitkv(q, k, v, causal=w.causal, scale=w.scale, splits=args.splits,
                             out=o, lse=lse, workspace=ws)
        elif args.path == "bwd":
            of, lf, do = fw[i % len(sets)]
            attn.bwd(q, k, v, of, lf, do, causal=w.causal, scale=w.scale, dq=grads[0],
                     dk=grads[1], dv=grads[2], workspace=ws)
        else:
            attn.fwd_decode(q, k, v, causal=w.causal, scale=w.scale, splits=dsplits,
                            out=o, lse=lse, workspace=ws)

    stream = torch.cuda.current_stream(dev)  # the stream attn.fwd launches on
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)
    sclk = []

    # timed region: K back-to-back steps.  By default the K steps are captured
    # once into a HIP graph (every buffer is allocated above; the C ABI
    # launches on torch's current stream, which is the capture stream inside
    # the capture) and the graph is replayed, untimed once, then timed: the
    # same K launches without K host round trips in between.
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(i)
        graph.replay()
        torch.cuda.synchronize(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t_wall = time.perf_counter()
    start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    end.record(stream)
    # the shader clock, sampled every 2 ms until the timed steps end (host
    # reads of sysfs; the first sample can still show the idle level)
    sclk.append(shader_clock_mhz())
    while not end.query():
        time.sleep(0.002)
        sclk.append(shader_clock_mhz())
    torch.cuda.synchronize(dev)
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    if graph is not None:
        del graph

    # per-call events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize(dev)
    per_us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    mean_us = statistics.fmean(per_us)
    med_us = statistics.median(per_us)
    p10 = per_us[int(0.1 * (len(per_us) - 1))]
    p90 = per_us[int(0.9 * (len(per_us) - 1))]

    flops, nbytes = w.flops(), w.alg_bytes()
    if args.path == "bwd":
        # five products (recomputed S, dP, dV, dK, dQ) against the forward's two;
        # bytes: read Q, K, V, O, dO, LSE, write dQ, dK, dV
        flops = 2.5 * flops
        n = w.B * w.H * w.S
        nbytes = 16 * n * w.D + 4 * n
    value = flops / (ms_per_step * 1e-3) / 1e12
    # the roofline takes the launch duration from the timed region (K launches
    # back to back between two events on the launch stream); bracketing each
    # call with its own events adds the launch latency to every call
    step_us = ms_per_step * 1e3
    # the binding roof: causal attention does 2 S^2 D FLOPs on 8 S D bytes per
    # (batch, head), S/4 FLOP per byte, under the FP16/HBM ridge (~315) for
    # S < 1260, so every causal workload here is HBM-bound on the roofline;
    # pct_fp16_peak below keeps the MFMA fraction
    roof = binding_roof(flops, nbytes, step_us)
    roof["traffic"] = measured_traffic(w.name, args.path)
    roof["launch_us"] = step_us
    roof["launches_per_step"] = {"fused": 1, "unfused": 3,
                                 "splitkv": 1 if args.path != "splitkv" or
                                 attn.splitkv_workspace_bytes(w.B, w.H, w.S, w.D, w.causal,
                                                              args.splits) == 0 else 2,
                                 "decode": 1 if not decode or
                                 attn.decode_workspace_bytes(w.B, w.H, w.Sq, w.Sk, w.D, w.causal,
                                                             dsplits) == 0 else 2,
                                 "bwd": 9 if w.D == 512 else 2}[args.path]
    roof["per_launch"] = {"flops": flops, "alg_bytes": nbytes}

    out = {
        "metric": METRIC_BWD if args.path == "bwd" else METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 (fp32 accumulate)",
        "data": "synthetic (seeded SplitMix64/Box-Muller normals, fp16 RNE)",
        "config": {"workload": w.name, "B": w.B, "H": w.H,
                   **({"Sq": w.Sq, "Sk": w.Sk, "splits": dsplits} if decode else {"S": w.S}),
                   "D": w.D,
                   "causal": w.causal, "scale": w.scale, "sigma": getattr(w, "sigma", 1.0),
                   "path": args.path, "input_sets": args.rotate,
                   **({"splits": args.splits} if args.path == "splitkv" else {}),
                   "cache": "warm (same buffers)" if args.rotate == 1 else
                            f"rotating {args.rotate} input sets",
                   "launch": "eager, one host launch per step" if args.eager else
                             "one HIP graph of the K steps, replayed"},
        "us_per_call": {"mean": mean_us, "median": med_us, "p10": p10, "p90": p90,
                        "back_to_back": ms_per_step * 1e3},
        "pct_fp16_peak": 100 * value / PEAK_FP16_TFLOPS,
        "alg_GBps": nbytes / (ms_per_step * 1e-3) / 1e9,
        "wall_s_timed": t_wall,
        "roofline": roof,
        "cpu_baseline": None,
    }
    out["sclk_mhz"] = sclk
    out["sclk_source"] = ("sysfs pp_dpm_sclk level, sampled every 2 ms while the timed steps "
                          "run; the level ramps over tens of ms, so a ~10 ms run reads low "
                          "(not the clock the kernels ran at)")
    if args.path == "fused" and args.cold_sets > 0:
        # cold: the calls cycle through cold_sets copies of the inputs, each in
        # its own memory, so that every call's inputs were last touched
        # (cold_sets - 1) * input bytes earlier -- past the 256 MB Infinity
        # Cache when that exceeds it
        cold = [sets[0]] + [tuple(t.clone() for t in sets[0]) for _ in range(args.cold_sets - 1)]

        def cold_step(i):
            q, k, v = cold[i % len(cold)]
            attn.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        nsteps = max(args.steps, 5 * args.cold_sets)
        us = replay_us(cold_step, nsteps, dev, stream)
        rec = fused_record(w, us)
        between = (args.cold_sets - 1) * 3 * w.B * w.H * w.S * w.D * 2
        rec.update({"input_sets": args.cold_sets, "steps": nsteps,
                    "input_bytes_between_reuse": between,
                    "launch": "one HIP graph of the steps, replayed"})
        del cold
        out["cold"] = rec
    if args.path == "fused" and not args.no_workloads:
        # every workload, warm (same buffers), as a graph replay like the main record
        recs = []
        for c, wc in sorted(inputs.WORKLOADS.items()):
            if c == args.workload:
                recs.append(fused_record(wc, ms_per_step * 1e3))
                continue
            qc, kc, vc = (torch.from_numpy(x).to(dev) for x in wc.qkv())
            oc = torch.empty(wc.shape, dtype=torch.float16, device=dev)
            lc = torch.empty(wc.shape[:3], dtype=torch.float32, device=dev)

            def wstep(i, wc=wc, qc=qc, kc=kc, vc=vc, oc=oc, lc=lc):
                attn.fwd(qc, kc, vc, causal=wc.causal, scale=wc.scale, out=oc, lse=lc)
            recs.append(fused_record(wc, replay_us(wstep, 300, dev, stream)))
            del qc, kc, vc, oc, lc
        out["workloads"] = recs
    if not args.no_cpu_baseline and args.path == "bwd":
        out["cpu_baseline"] = cpu_baseline_bwd(w, args.cpu_seconds)
    elif not args.no_cpu_baseline and not decode:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
