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
    """Hash of the kernel source's code: comments and whitespace are
    dropped first, so that an edit of either keeps the counter record."""
    import re as _re
    with open(KERNEL_SRC) as f:
        src = f.read()
    src = _re.sub(r"/\*.*?\*/", "", src, flags=_re.S)
    src = _re.sub(r"//[^\n]*", "", src)
    src = _re.sub(r"\s+", "", src)
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def traffic_record(workload, dominant_pass):
    """The committed rocprofv3 counter record of the dominant kernel
    (profiles/traffic.json), or None if absent or taken on an older kernel
    source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get("workloads", {}).get(workload)
    if not rec or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    p = rec.get("passes", {}).get(str(dominant_pass))
    if p is None:
        return None
    out = dict(p)
    out["fetch_scale"], out["write_scale"] = rec.get("fetch_scale"), rec.get("write_scale")
    return out


def measured_traffic(workload, dominant_pass):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, or None if absent or taken on an older
    kernel source."""
    p = traffic_record(workload, dominant_pass)
    return None if p is None else p.get("bytes_per_launch")


def lds_conflicts(workload, kernel):
    """Bank-conflict cycles per LDS-active cycle of `kernel` from the
    committed profiles/<workload>_lds.txt, or None."""
    try:
        with open(os.path.join(ROOT, "profiles", "%s_lds.txt" % workload)) as f:
            for line in f:
                cols = [c.strip() for c in line.split("|")]
                if len(cols) >= 7 and cols[0] == kernel:
                    return {"kernel": kernel, "conflict_cycles": float(cols[5]),
                            "lds_active_cycles": float(cols[4]),
                            "conflict_per_active": float(cols[6])}
    except (OSError, ValueError):
        return None
    return None


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


def cache_copy_ceiling(torch, mib=64, reps=200):
    """GB/s of the streaming copy between two mib-MiB buffers that stay in
    the Infinity Cache across calls (read + write bytes per call): the
    ceiling of a chunked pass, whose chunk also stays there between its
    passes."""
    import quantum_state_encoding_amd as qse
    dev = torch.device("cuda:0")
    src = torch.randn((mib << 20) // 4, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    fn = lambda: qse.stream_copy(dst, src)
    for _ in range(10):
        fn()
    torch.cuda.synchronize()
    ms = min(time_events(torch, stream, fn, reps) for _ in range(3))
    del src, dst
    return {"gbps": 2 * (mib << 20) / (ms * 1e-3) / 1e9, "bytes_per_call": 2 * (mib << 20),
            "us_per_call": ms * 1e3}


def cpu_baseline(w, repeats=5):
    """The oracle's timed mode (textbook transform in the workload's dtype,
    a pool of POSIX threads over the real vectors) on the whole batch, run
    `repeats` times (about 10 thread-seconds of CPU work at n=20, batch
    256); the median is reported."""
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
            "ms": t * 1e3,
            "sample": "whole workload: %d complex vectors of 2^%d (%d real transforms, %s), "
                      "median of %d runs of %.3f s on %d threads" % (
                          w.batch, w.n, 2 * w.batch, w.dtype, repeats, t, int(used))}


def bench_workload(torch, w, steps, warmup, with_passes=True, split="configured"):
    import quantum_state_encoding_amd as qse
    dev = torch.device("cuda:0")
    tdt = torch.float32 if w.dtype == "f32" else torch.float64
    log("generating %s (%.2f GiB)" % (w.name, w.state_bytes / 2**30))
    hre = torch.empty((w.batch, w.N), dtype=tdt).pin_memory()
    him = torch.empty((w.batch, w.N), dtype=tdt).pin_memory()
    workloads.gen(w, hre.numpy(), him.numpy())
    re = hre.to(dev)
    im = him.to(dev)
    sp = (w.split or None) if split == "configured" else split
    plan = qse.Plan(w.n, w.dtype, split=sp)
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
    # Spread: five more short repeats, after the timed region.
    reps = [time_events(torch, stream, step, max(5, steps // 10)) for _ in range(5)] \
        if with_passes else []
    # Per-kernel durations: the schedule fwt_execute runs (all passes of one
    # chunk of vectors, chunk after chunk), each kernel timed by HIP events
    # that its own dispatch records at its start and end; averaged per pass
    # over `steps` steps.
    per_pass = []
    chunk = plan.chunk_vectors(w.batch, True) or w.batch
    if with_passes:
        evs = []
        for _ in range(steps):
            for c0 in range(0, w.batch, chunk):
                sl = slice(c0, min(w.batch, c0 + chunk))
                for i in range(passes):
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    plan.execute_pass_timed(i, re[sl], im[sl], a, b, normalize=w.normalize)
                    evs.append((i, a, b))
        torch.cuda.synchronize()
        tot = [0.0] * passes
        cnt = [0] * passes
        for i, a, b in evs:
            tot[i] += a.elapsed_time(b)
            cnt[i] += 1
        per_pass = [tot[i] / cnt[i] for i in range(passes)]
    # Self-check without the oracle: H is its own inverse up to 2^n
    # (H H = 2^n I), so two calls from the original input must give the
    # input back (normalised) or 2^n times it (unnormalised, exact for the
    # integer workload).  Sampled vectors are compared on the host.
    check = None
    if with_passes:
        re.copy_(hre, non_blocking=False)
        im.copy_(him, non_blocking=False)
        step()
        step()
        torch.cuda.synchronize()
        scale = 1.0 if w.normalize else float(2 ** w.n)
        rows = sorted(set(int(r) for r in np.linspace(0, w.batch - 1, min(8, w.batch))))
        worst = 0.0
        exact = True
        for r in rows:
            x_re = hre[r].numpy().astype(np.float64)
            x_im = him[r].numpy().astype(np.float64)
            g_re = re[r].cpu().numpy().astype(np.float64)
            g_im = im[r].cpu().numpy().astype(np.float64)
            err = max(np.abs(g_re - scale * x_re).max(), np.abs(g_im - scale * x_im).max())
            norm = np.sqrt(np.sum(x_re ** 2) + np.sum(x_im ** 2)) * scale
            worst = max(worst, err / norm if norm > 0 else err)
            exact = exact and err == 0.0
        check = {"calls": 2, "vectors": len(rows), "max_err_over_norm": worst,
                 "exact": bool(exact)}
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
            "per_pass_ms": per_pass, "copy_ms": copy_ms, "S": S, "chunk": chunk,
            "check": check, "reps_ms": reps,
            "kernel_names": [plan.kernel_name(i, w.batch) for i in range(passes)]}


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError("no *%s under %s" % (suffix, dirpath))


def summarize_profile(workload, kt_dir, fetch_dir, write_dir, command, lds_dir=None):
    """Turn rocprofv3 CSV output of this benchmark into the text summaries
    under profiles/ and profiles/traffic.json (HBM bytes per launch)."""
    import quantum_state_encoding_amd as qse
    w = workloads.WORKLOADS[workload]
    plan = qse.Plan(w.n, w.dtype, split=w.split or None)
    trace = _read_csv(_find(kt_dir, "kernel_trace.csv"))
    groups = {}
    for r in trace:
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))

    def counters(d):
        out = {}
        for r in _read_csv(_find(d, "counter_collection.csv")):
            key = (r["Kernel_Name"], int(r["Grid_Size"]))
            out.setdefault(key, []).append(float(r["Counter_Value"]))
        return out
    fetch, write = counters(fetch_dir), counters(write_dir)

    def short(name):
        return name.replace("qse::(anonymous namespace)::", "").split("(float*")[0].split(
            "(double*")[0]

    # Calibration: the streaming copy of one component moves S/2 bytes each way.
    half_kib = w.state_bytes / 2 / 1024
    cf = [v for (k, g), v in fetch.items() if "stream_copy_kernel" in k]
    cw = [v for (k, g), v in write.items() if "stream_copy_kernel" in k]
    f_scale = half_kib / float(np.mean(cf[0])) if cf else None
    w_scale = half_kib / float(np.mean(cw[0])) if cw else None
    chunk = plan.chunk_vectors(w.batch, True) or w.batch
    chunk_bytes = w.state_bytes * chunk // w.batch
    lines = ["# rocprofv3 kernel trace: %s" % workload,
             "# command: " + command,
             "# kernel | grid (threads x, y) | dispatches | avg us | min us | max us"]
    for (name, gx, gy), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append("%s | %d x %d | %d | %.2f | %.2f | %.2f" % (
            short(name), gx, gy, len(d), np.mean(d) / 1e3, np.min(d) / 1e3, np.max(d) / 1e3))
    passes = {}

    def run_command(counters, out_dir, out_name):
        # the recorded trace command, with the counter run's options and
        # output directory
        c = command.replace("--kernel-trace --stats", counters).replace(" -o kt ", " -o %s " % out_name)
        return c.replace(os.path.basename(os.path.normpath(kt_dir)),
                         os.path.basename(os.path.normpath(out_dir)))
    tl = ["# rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (separate runs): %s" % workload,
          "# commands: " + run_command("--pmc FETCH_SIZE", fetch_dir, "f"),
          "#           " + run_command("--pmc WRITE_SIZE", write_dir, "w"),
          "# calibration on fwt_stream_copy of %.0f KiB each way: FETCH_SIZE x %.4f, "
          "WRITE_SIZE x %.4f" % (half_kib, f_scale or float("nan"), w_scale or float("nan")),
          "# pass | kernel | launches | FETCH KiB | WRITE KiB | scaled HBM bytes/launch | "
          "algorithmic bytes/launch | ratio | avg us (trace)"]
    for i in range(plan.num_passes):
        kname = plan.kernel_name(i, w.batch)
        cand = [(k, v) for k, v in groups.items() if kname in k[0]]
        if not cand:
            continue
        (name, gx, gy), d = max(cand, key=lambda kv: kv[0][1] * kv[0][2])
        fv = fetch.get((name, gx * gy)) or fetch.get((name, gx))
        wv = write.get((name, gx * gy)) or write.get((name, gx))
        rec = {"kernel": short(name), "grid": [gx, gy], "dispatches": len(d),
               "avg_us": float(np.mean(d) / 1e3), "algorithmic_bytes_per_launch": 2 * chunk_bytes}
        if fv and wv and f_scale and w_scale:
            b = (float(np.mean(fv)) * f_scale + float(np.mean(wv)) * w_scale) * 1024
            rec.update({"fetch_kib": float(np.mean(fv)), "write_kib": float(np.mean(wv)),
                        "bytes_per_launch": b})
            tl.append("%d | %s | %d | %.1f | %.1f | %.4g | %.4g | %.4f | %.2f" % (
                i, short(name), len(fv), np.mean(fv), np.mean(wv), b, 2 * chunk_bytes,
                b / (2 * chunk_bytes), rec["avg_us"]))
        passes[str(i)] = rec
    lds_lines = []
    if lds_dir:
        per = {}
        for r in _read_csv(_find(lds_dir, "counter_collection.csv")):
            key = (r["Kernel_Name"], int(r["Grid_Size"]), r["Dispatch_Id"])
            per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
        agg = {}
        for (name, grid, _), cs in per.items():
            a = agg.setdefault((short(name), grid), {})
            for k, v in cs.items():
                a[k] = a.get(k, 0.0) + v
            a["dispatches"] = a.get("dispatches", 0) + 1
        lds_lines = ["# rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS "
                     "SQ_LDS_MEM_VIOLATIONS SQ_LDS_UNALIGNED_STALL: %s" % workload,
                     "# command: " + run_command("--pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
                                                 "SQ_INSTS_LDS SQ_LDS_MEM_VIOLATIONS "
                                                 "SQ_LDS_UNALIGNED_STALL", lds_dir, "l"),
                     "# kernel | grid | dispatches | LDS instructions | LDS active cycles | "
                     "bank-conflict cycles | conflict / active | memory violations | "
                     "unaligned stalls"]
        for (name, grid), a in sorted(agg.items(), key=lambda kv: -kv[1].get("SQ_LDS_IDX_ACTIVE", 0)):
            act = a.get("SQ_LDS_IDX_ACTIVE", 0.0)
            bc = a.get("SQ_LDS_BANK_CONFLICT", 0.0)
            lds_lines.append("%s | %d | %d | %.0f | %.0f | %.0f | %.4f | %.0f | %.0f" % (
                name, grid, a["dispatches"], a.get("SQ_INSTS_LDS", 0.0), act, bc,
                bc / act if act else 0.0, a.get("SQ_LDS_MEM_VIOLATIONS", 0.0),
                a.get("SQ_LDS_UNALIGNED_STALL", 0.0)))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    if lds_lines:
        with open(os.path.join(ROOT, "profiles", "%s_lds.txt" % workload), "w") as f:
            f.write("\n".join(lds_lines) + "\n")
    with open(os.path.join(ROOT, "profiles", "%s_kernel_trace.txt" % workload), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(ROOT, "profiles", "%s_traffic.txt" % workload), "w") as f:
        f.write("\n".join(tl) + "\n")
    try:
        with open(TRAFFIC_FILE) as f:
            allt = json.load(f)
    except (OSError, ValueError):
        allt = {"workloads": {}}
    allt["workloads"][workload] = {"kernel_source_sha256_16": kernel_source_hash(),
                                   "fetch_scale": f_scale, "write_scale": w_scale,
                                   "chunk_vectors": chunk, "passes": passes}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allt, f, indent=1, sort_keys=True)
        f.write("\n")
    print("\n".join(lines + [""] + tl + [""] + lds_lines))


def summarize_ablations(workload, kt_dir, command):
    """Per-kernel durations of everything in the trace that is neither a pass
    of the workload's plan nor the streaming copy (the ablations, and the
    small workloads timed alongside the default one) into
    profiles/<workload>_ablations_kernel_trace.txt."""
    import quantum_state_encoding_amd as qse
    w = workloads.WORKLOADS[workload]
    plan = qse.Plan(w.n, w.dtype, split=w.split or None)
    main = [plan.kernel_name(i, w.batch) for i in range(plan.num_passes)] + ["stream_copy_kernel"]
    groups = {}
    for r in _read_csv(_find(kt_dir, "kernel_trace.csv")):
        name = r["Kernel_Name"]
        if any(m in name for m in main) or "at::native" in name:
            continue
        key = (name.replace("qse::(anonymous namespace)::", "").split("(")[0],
               int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = ["# rocprofv3 kernel trace: %s, every kernel other than the workload's own passes "
             "and the streaming copy: the ablations (3 timed calls after one warm-up call "
             "each) and, for the default workload, the small workloads bench.py also times"
             % workload,
             "# command: " + command,
             "# kernel | grid (threads x, y) | dispatches | avg us | min us | max us | total ms"]
    for (name, gx, gy), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append("%s | %d x %d | %d | %.2f | %.2f | %.2f | %.3f" % (
            name, gx, gy, len(d), np.mean(d) / 1e3, np.min(d) / 1e3, np.max(d) / 1e3,
            np.sum(d) / 1e6))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "%s_ablations_kernel_trace.txt" % workload), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def bench_ablations(torch, w, steps=3):
    """Time the pages' designs on the workload's state: one launch per
    butterfly stage, the popcount-GEMM Kronecker scaffold with its batch
    transposes, the matrix-core block-Hadamard row kernel followed by the
    column passes, matrix-core blocks on both factors with transposes in
    between, and (fp64) the INT8 / CRT emulation (fwt_ablation_execute).
    ms per step, same accounting."""
    import quantum_state_encoding_amd as qse
    dev = torch.device("cuda:0")
    tdt = torch.float32 if w.dtype == "f32" else torch.float64
    re = torch.randn(w.batch, w.N, device=dev, dtype=tdt) / 1024
    im = torch.randn_like(re)
    stream = torch.cuda.current_stream()
    out = {}
    kinds = [("stagewise", qse.ABLATION_STAGEWISE, w.n)]
    if w.n <= 20:
        kinds.append(("popc_gemm_transpose", qse.ABLATION_POPC_GEMM, 2))
    if w.n >= 8:
        kinds.append(("mfma_block_hadamard", qse.ABLATION_MFMA, 2))
    if 16 <= w.n <= (30 if w.dtype == "f32" else 28):
        kinds.append(("mfma_blocks_with_transposes", qse.ABLATION_MFMA_TRANSPOSE, 4))
    if w.dtype == "f64" and 5 <= w.n <= 28:
        kinds.append(("ozaki_int8_crt", qse.ABLATION_OZAKI, 3))
    for name, kind, launches in kinds:
        wsb = qse.ablation_workspace(kind, w.batch, w.n, w.dtype, True)
        ws = torch.empty(wsb // 4, device=dev) if wsb else None
        fn = lambda: qse.ablation_execute(kind, re, im, n=w.n, normalize=w.normalize,
                                          workspace=ws)
        fn()
        torch.cuda.synchronize()
        ms = time_events(torch, stream, fn, steps)
        out[name] = {"ms_per_step": ms, "amplitudes_per_s": w.batch * w.N / (ms * 1e-3),
                     "gbps_algorithmic": 2 * w.state_bytes / (ms * 1e-3) / 1e9}
        del ws
    del re, im
    torch.cuda.empty_cache()
    log("ablations: " + ", ".join("%s %.3f ms" % (k, v["ms_per_step"]) for k, v in out.items()))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="n20_b256_f32", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-ablations", action="store_true",
                    help="skip timing the pages' designs (stage-wise, popcount GEMM, "
                    "matrix-core blocks)")
    ap.add_argument("--summarize-profile", nargs="+",
                    metavar="DIR", help="KT_DIR FETCH_DIR WRITE_DIR [LDS_DIR]: write profiles/ "
                    "summaries from rocprofv3 CSV output of this benchmark")
    ap.add_argument("--summarize-ablations", metavar="KT_DIR",
                    help="write profiles/<workload>_ablations_kernel_trace.txt from a rocprofv3 "
                    "kernel trace of this benchmark")
    ap.add_argument("--profile-command", default="",
                    help="the rocprofv3 command line recorded in the summaries")
    args = ap.parse_args()
    if args.summarize_profile:
        d = args.summarize_profile
        if len(d) not in (3, 4):
            ap.error("--summarize-profile takes 3 or 4 directories")
        summarize_profile(args.workload, d[0], d[1], d[2], args.profile_command,
                          d[3] if len(d) == 4 else None)
        return
    if args.summarize_ablations:
        summarize_ablations(args.workload, args.summarize_ablations, args.profile_command)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
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
    launch_bytes = 2 * S * r["chunk"] // w.batch     # read + write of one chunk's state
    achieved = launch_bytes / (dom_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name, dom)
    trec = traffic_record(w.name, dom)
    lds = None
    if trec is not None:   # the LDS counters come from the same profiling session
        lds = lds_conflicts(w.name, trec.get("kernel", ""))

    # The other workloads, briefly: the metric also names n=14 (batch 64),
    # reported with its configured 7|7 split and with the default plan.
    also = {}
    if w.name == "n20_b256_f32":
        for name, sp, label in (("n14_b64_f32", "configured", "n14_b64_f32 (7|7 as configured)"),
                                ("n14_b64_f32", None, "n14_b64_f32 (default plan)"),
                                ("n12_b64_f32", None, "n12_b64_f32"),
                                ("n10_b8_f32_int", None, "n10_b8_f32_int")):
            ws = workloads.WORKLOADS[name]
            rs = bench_workload(torch, ws, max(args.steps, 200), args.warmup, with_passes=False,
                                split=sp)
            also[label] = {"ms_per_step": rs["ms"], "passes": rs["passes"],
                           "pass_bits": rs["pass_bits"], "kernel_names": rs["kernel_names"],
                           "amplitudes_per_s": ws.batch * ws.N / (rs["ms"] * 1e-3),
                           "gbps_accounted": 2 * ws.state_bytes * rs["passes"] /
                           (rs["ms"] * 1e-3) / 1e9,
                           "note": "%.0f KiB state, resident in cache across steps; "
                                   "latency-bound" % (ws.state_bytes / 1024)}
        # The fp64 workload (4 GiB, HBM-bound), with the same accounting.
        ws = workloads.WORKLOADS["n24_b16_f64"]
        rs = bench_workload(torch, ws, max(20, args.steps // 5), args.warmup, with_passes=False)
        gb = 2 * ws.state_bytes * rs["passes"] / (rs["ms"] * 1e-3) / 1e9
        also["n24_b16_f64"] = {"ms_per_step": rs["ms"], "passes": rs["passes"],
                               "pass_bits": rs["pass_bits"],
                               "amplitudes_per_s": ws.batch * ws.N / (rs["ms"] * 1e-3),
                               "gbps_accounted": gb,
                               "pct_peak_accounted": 100 * gb / HBM_PEAK_GBS,
                               "note": "4 GiB state, HBM-bound; %d steps" % max(20, args.steps // 5)}

    # Copy ceilings: the whole state through HBM (copy_gbps) and a working
    # set that stays in the Infinity Cache, as a chunk does between passes.
    cache_copy = cache_copy_ceiling(torch)

    # The pages' own designs for the same transform, on the same state.
    ablations = {}
    if not args.no_ablations:
        ablations = bench_ablations(torch, w)

    cpu = None if args.no_cpu else cpu_baseline(w)
    out = {
        "metric": "FWT amplitudes/sec + achieved HBM GB/s (% of peak), n=14 & n=20 fp32, "
                  "batch 64/256",
        "value": amps_per_s,
        "unit": "amplitudes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "t_ms_median": float(np.median(r["reps_ms"])) if r["reps_ms"] else None,
        "t_ms_min": float(np.min(r["reps_ms"])) if r["reps_ms"] else None,
        "seed": w.seed,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded Gaussian states, L2-normalised per vector",
        "config": {"workload": w.name, "n": w.n, "batch": w.batch, "normalize": w.normalize,
                   "layout": "planar re/im", "passes": r["passes"], "pass_bits": r["pass_bits"],
                   "chunk_vectors": r["chunk"]},
        "gbps_accounted": gbps_accounted,
        "pct_peak_accounted": 100 * gbps_accounted / HBM_PEAK_GBS,
        "gbps_algorithmic": gbps_alg,
        "pct_peak_algorithmic": 100 * gbps_alg / HBM_PEAK_GBS,
        "per_pass_ms": r["per_pass_ms"],
        "copy_ms": r["copy_ms"],
        "copy_gbps": 2 * S / (r["copy_ms"] * 1e-3) / 1e9 if r["copy_ms"] else None,
        "cache_copy": cache_copy,
        # the step against one same-run copy of the state (read S, write S)
        "copy_fraction": {"accounted": gbps_accounted / (2 * S / (r["copy_ms"] * 1e-3) / 1e9),
                          "algorithmic": gbps_alg / (2 * S / (r["copy_ms"] * 1e-3) / 1e9)}
        if r["copy_ms"] else None,
        "wall_ms_per_step": r["wall_ms"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "fetch_bytes": None if trec is None else
                     trec["fetch_kib"] * trec["fetch_scale"] * 1024,
                     "write_bytes": None if trec is None else
                     trec["write_kib"] * trec["write_scale"] * 1024,
                     "lds_bank_conflicts": lds,
                     "kernel_name": r["kernel_names"][dom] if r["kernel_names"] else None,
                     "kernel": "pass %d (%d bits, %s)" % (dom, r["pass_bits"][dom] if r["pass_bits"] else 0,
                                                           "row" if dom == 0 else "column"),
                     "bytes_per_launch": launch_bytes,
                     "frac_of_cache_copy": achieved / cache_copy["gbps"],
                     "launches_per_step": r["passes"] * (-(-w.batch // r["chunk"]))},
        "cpu_baseline": cpu,
        "involution_check": r["check"],
        "gpu_name": torch.cuda.get_device_name(0),
        "gpu_arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
        "hip_version": getattr(torch.version, "hip", None),
        "also": also,
        "ablations": ablations,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
