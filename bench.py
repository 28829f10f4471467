"""Benchmark: batched in-place Walsh-Hadamard transform on one MI355X.

A step is one fwt_execute over the whole synthetic state of the workload
(every pass of the plan, normalised): by default 256 complex fp32 vectors
of 2^20 amplitudes (planar re/im, 2 GiB), inputs resident in HBM before
the timed region.  Prints one JSON line with the throughput (complex
amplitudes per second), the roofline of the dominant kernel (measured
with HIP events on the launch stream), and the CPU oracle timed on the
host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, 8 TB/s
KERNEL_SRC = os.path.join(ROOT, "quantum_state_encoding_amd", "csrc", "fwt_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload, dominant_pass):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, or None if absent or taken on an older
    kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get("workloads", {}).get(workload)
    if not rec or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    p = rec.get("passes", {}).get(str(dominant_pass))
    return None if p is None else p.get("bytes_per_launch")


def time_events(torch, stream, fn, reps):
    """Average ms per call of fn() over reps calls, HIP events on stream."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def cpu_baseline(w, repeats=2):
    """The oracle's timed mode (textbook transform in the workload's dtype,
    a pool of POSIX threads over the real vectors) on the whole batch."""
    import oracle
    threads = min(16, len(os.sched_getaffinity(0)))
    re, im = workloads.gen(w)
    state = np.concatenate([re, im])          # 2 * batch real vectors
    times = []
    used = threads
    for _ in range(repeats):
        x = state.copy()
        t0 = time.perf_counter()
        used = oracle.fwt_threaded_inplace(x, w.n, w.normalize, threads)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    amps = w.batch * w.N
    return {"value": amps / t, "unit": "amplitudes/s", "cores": int(used), "kind": "oracle",
            "sample": "whole workload: %d complex vectors of 2^%d (%d real transforms, %s), "
                      "median of %d runs of %.3f s" % (w.batch, w.n, 2 * w.batch, w.dtype,
                                                     repeats, t)}


def bench_workload(torch, w, steps, warmup, with_passes=True):
    import quantum_state_encoding_amd as qse
    dev = torch.device("cuda:0")
    tdt = torch.float32 if w.dtype == "f32" else torch.float64
    log("generating %s (%.2f GiB)" % (w.name, w.state_bytes / 2**30))
    hre = torch.empty((w.batch, w.N), dtype=tdt).pin_memory()
    him = torch.empty((w.batch, w.N), dtype=tdt).pin_memory()
    workloads.gen(w, hre.numpy(), him.numpy())
    re = hre.to(dev)
    im = him.to(dev)
    plan = qse.Plan(w.n, w.dtype, split=w.split or None)
    stream = torch.cuda.current_stream()
    passes = plan.num_passes

    step = plan.bind(re, im, normalize=w.normalize)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log("timing %d steps" % steps)
    t0 = time.perf_counter()
    ms_events = time_events(torch, stream, step, steps)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = ms_events
    # Per-kernel durations: the same passes, one event pair per launch.
    per_pass = []
    if with_passes:
        for i in range(passes):
            per_pass.append(time_events(
                torch, stream, lambda: plan.execute_pass(i, re, im, normalize=w.normalize),
                max(10, steps // 2)))
    # Stream-copy ceiling: one read and one write of the whole state.
    copy_ms = None
    if with_passes:
        dre, dim = torch.empty_like(re), torch.empty_like(im)

        def copy_state():
            qse.stream_copy(dre, re)
            qse.stream_copy(dim, im)
        copy_ms = time_events(torch, stream, copy_state, max(10, steps // 2))
        del dre, dim
    del re, im
    torch.cuda.empty_cache()
    S = w.state_bytes
    return {"ms": ms, "wall_ms": wall_ms, "passes": passes, "pass_bits": plan.pass_bits,
            "per_pass_ms": per_pass, "copy_ms": copy_ms, "S": S}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="n20_b256_f32", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(batches shard across GPUs with no communication); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(2)

    w = workloads.WORKLOADS[args.workload]
    r = bench_workload(torch, w, args.steps, args.warmup)
    S = r["S"]
    amps_per_s = w.batch * w.N / (r["ms"] * 1e-3)
    gbps_accounted = 2 * S * r["passes"] / (r["ms"] * 1e-3) / 1e9
    gbps_alg = 2 * S / (r["ms"] * 1e-3) / 1e9
    dom = int(np.argmax(r["per_pass_ms"])) if r["per_pass_ms"] else 0
    dom_ms = r["per_pass_ms"][dom] if r["per_pass_ms"] else r["ms"]
    achieved = 2 * S / (dom_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name, dom)

    also = {}
    if w.name == "n20_b256_f32":
        w14 = workloads.WORKLOADS["n14_b64_f32"]
        r14 = bench_workload(torch, w14, max(args.steps, 200), args.warmup, with_passes=False)
        also[w14.name] = {"ms_per_step": r14["ms"], "passes": r14["passes"],
                          "pass_bits": r14["pass_bits"],
                          "amplitudes_per_s": w14.batch * w14.N / (r14["ms"] * 1e-3),
                          "gbps_accounted": 2 * w14.state_bytes * r14["passes"] /
                          (r14["ms"] * 1e-3) / 1e9,
                          "note": "8 MiB state: resident in L2/MALL across steps"}

    cpu = None if args.no_cpu else cpu_baseline(w)
    out = {
        "metric": "FWT amplitudes/sec + achieved HBM GB/s (% of peak)",
        "value": amps_per_s,
        "unit": "amplitudes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded Gaussian states, L2-normalised per vector",
        "config": {"workload": w.name, "n": w.n, "batch": w.batch, "normalize": w.normalize,
                   "layout": "planar re/im", "passes": r["passes"], "pass_bits": r["pass_bits"]},
        "gbps_accounted": gbps_accounted,
        "pct_peak_accounted": 100 * gbps_accounted / HBM_PEAK_GBS,
        "gbps_algorithmic": gbps_alg,
        "pct_peak_algorithmic": 100 * gbps_alg / HBM_PEAK_GBS,
        "per_pass_ms": r["per_pass_ms"],
        "copy_ms": r["copy_ms"],
        "copy_gbps": 2 * S / (r["copy_ms"] * 1e-3) / 1e9 if r["copy_ms"] else None,
        "wall_ms_per_step": r["wall_ms"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "pass %d (%d bits, %s)" % (dom, r["pass_bits"][dom] if r["pass_bits"] else 0,
                                                           "row" if dom == 0 else "column"),
                     "bytes_per_launch": 2 * S},
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
