"""Host-side checks of bench.py's accounting (no GPU): the roofline is one
read plus one write of a chunk's state over the summed durations of that
chunk's pass kernels, the per-workload records carry the measurement
fields, and the rocprofv3 summaries calibrate the counters on the
state-sized streaming copy."""
import csv
import json
import os

import pytest

import bench
import workloads


def _measured(w, per_pass_ms, chunk, pass_bits):
    return {"ms": sum(per_pass_ms) * w.batch / chunk, "steps": 10, "wall_ms": 1.0,
            "passes": len(per_pass_ms), "pass_bits": list(pass_bits),
            "per_pass_ms": per_pass_ms, "copy_ms": 0.79, "S": w.state_bytes, "chunk": chunk,
            "check": None, "reps_ms": [1.27, 1.28, 1.29, 1.30, 1.31],
            "kernel_names": ["row", "col"][:len(per_pass_ms)], "output": None, "inputs": None}


def test_roofline_counts_one_read_and_write_per_transform(monkeypatch):
    monkeypatch.setattr(bench, "traffic_record", lambda name: None)
    w = workloads.WORKLOADS["n20_b256_f32"]
    r = _measured(w, [0.0807, 0.0775], 32, (12, 8))
    rl = bench.roofline(w, r, {"gbps": 6650.0})
    chunk_bytes = w.state_bytes * 32 // w.batch
    assert rl["algorithmic_bytes"] == 2 * chunk_bytes == 512 << 20
    assert rl["achieved"] == pytest.approx(2 * chunk_bytes / (0.1582e-3) / 1e9)
    assert rl["frac"] == pytest.approx(rl["achieved"] / 8000.0)
    assert 0.42 < rl["frac"] < 0.43
    assert rl["peak"] == 8000.0 and rl["unit"] == "GB/s" and rl["bound"] == "hbm"
    assert rl["traffic"] is None            # no counter record for this source
    assert rl["launches_per_step"] == 2 * 8
    # per pass: the rate at which it moves its chunk
    assert rl["passes"][0]["pass_fabric_gbps"] == pytest.approx(2 * chunk_bytes / 0.0807e-3 / 1e9)


def test_roofline_sums_the_counter_bytes_of_every_pass(monkeypatch):
    w = workloads.WORKLOADS["n24_b16_f64"]
    rec = {"fetch_scale": 2.0, "write_scale": 1.0,
           "passes": {"0": {"bytes_per_launch": 5.0e8, "fetch_kib": 1000.0, "write_kib": 2000.0,
                            "kernel": "k0"},
                      "1": {"bytes_per_launch": 6.0e8, "fetch_kib": 3000.0, "write_kib": 4000.0,
                            "kernel": "k1"}}}
    monkeypatch.setattr(bench, "traffic_record", lambda name: rec)
    monkeypatch.setattr(bench, "lds_conflicts", lambda name, kernel: None)
    rl = bench.roofline(w, _measured(w, [0.090, 0.081], 1, (14, 10)), {"gbps": 6650.0})
    assert rl["traffic"] == pytest.approx(1.1e9)
    assert rl["fetch_bytes"] == pytest.approx((1000.0 + 3000.0) * 2.0 * 1024)
    assert rl["write_bytes"] == pytest.approx((2000.0 + 4000.0) * 1.0 * 1024)


def test_roofline_of_the_one_pass_kernel(monkeypatch):
    """One launch over the whole state: algorithmic bytes 2 x S, achieved =
    2 x S over the kernel's duration; the counter record of the configured
    plan is used only when it, too, was taken on the one-pass kernel."""
    w = workloads.WORKLOADS["n20_b256_f32"]
    r = _measured(w, [1.100], w.batch, (20,))
    r.update({"onepass": True, "kernel_names": ["onepass_kernel"]})
    rec = {"fetch_scale": 2.0, "write_scale": 1.0,
           "plans": {"as configured": {"onepass": True, "passes": {
               "0": {"bytes_per_launch": 4.76e9, "fetch_kib": 1.05e6, "write_kib": 2.5e6,
                     "kernel": "onepass_kernel(OnepassArgs)"}}},
                     "two-pass": {"onepass": False, "passes": {}}}}
    monkeypatch.setattr(bench, "traffic_record", lambda name: rec)
    monkeypatch.setattr(bench, "lds_conflicts", lambda name, kernel: None)
    rl = bench.roofline(w, r, {"gbps": 6650.0})
    assert rl["algorithmic_bytes"] == 2 * w.state_bytes == 4 << 30
    assert rl["achieved"] == pytest.approx(2 * w.state_bytes / 1.100e-3 / 1e9)
    assert 0.48 < rl["frac"] < 0.49
    assert rl["launches_per_step"] == 1 and "onepass_kernel" in rl["kernel"]
    assert rl["traffic"] == pytest.approx(4.76e9)
    # a record taken on fwt_execute's passes does not price the one-pass kernel
    rec["plans"]["as configured"]["onepass"] = False
    assert bench.roofline(w, r, {"gbps": 6650.0})["traffic"] is None
    rec2 = bench.config_record(4, w, r, None, "as configured")
    assert rec2["passes"] == 1 and rec2["path"].startswith("one HBM pass")
    assert rec2["gbps_accounted"] == pytest.approx(rec2["gbps_algorithmic"])


def test_config_record_carries_the_measurement_fields():
    w = workloads.WORKLOADS["n24_b16_f64"]
    r = _measured(w, [0.090, 0.081], 1, (14, 10))
    cpu = {"cores": 16, "ms": 575.0, "value": 4.7e8, "single_thread_ms_per_real_vector": 127.0,
           "oracle_check": {"max_err_over_norm": 4e-19, "exact": False, "within_tolerance": True,
                            "vectors": 16}}
    rec = bench.config_record(5, w, r, cpu, "as configured")
    for key in ("cfg", "n", "batch", "dtype", "path", "passes", "t_ms_median", "t_ms_min",
                "amps_per_s", "gbps_accounted", "pct_peak_accounted", "pct_peak_algorithmic",
                "copy_gbps", "max_err_over_norm", "exact", "cpu_cores", "cpu_ms",
                "cpu_amps_per_s", "seed", "cpu_single_thread_ms_per_real_vector"):
        assert key in rec, key
    blocks = sorted([r["ms"]] + r["reps_ms"])                # the six timed blocks
    t_med = (blocks[2] + blocks[3]) / 2
    assert rec["t_ms_median"] == pytest.approx(t_med)
    assert rec["pct_peak_algorithmic"] == pytest.approx(
        100 * 2 * w.state_bytes / (t_med * 1e-3) / 1e9 / 8000.0)
    assert rec["gbps_accounted"] == pytest.approx(2 * rec["gbps_algorithmic"])
    assert rec["path"] == "split 10|14"


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        wr.writeheader()
        wr.writerows(rows)


def test_profile_summary_calibrates_on_the_state_copy(tmp_path, monkeypatch, lib):
    """bench.py runs a 64 MiB cache-resident copy before the state-sized
    one; each copy launch of G threads moves G x 128 bytes each way, and
    the counters are scaled by the largest one."""
    import quantum_state_encoding_amd as qse
    w = workloads.WORKLOADS["n20_b256_f32"]
    plan = qse.Plan(w.n, w.dtype)
    k0, k1 = plan.kernel_name(0, w.batch), plan.kernel_name(1, w.batch)
    names = {"row": "void qse::(anonymous namespace)::%s(float*, float*, qse::TileArgs)" % k0,
             "col": "void qse::(anonymous namespace)::%s(float*, float*, qse::TileArgs)" % k1,
             "copy": "stream_copy_kernel(int4*, int4 const*, long)"}
    grids = {"row": (2097152, 2), "col": (524288, 2), "copy_small": (524288, 1),
             "copy_state": (8388608, 1)}
    kt = []
    for key, gkey, dur in (("row", "row", 80000), ("col", "col", 78000),
                           ("copy", "copy_small", 20000), ("copy", "copy_state", 390000)):
        for i in range(4):
            kt.append({"Kernel_Name": names[key], "Grid_Size_X": grids[gkey][0],
                       "Grid_Size_Y": grids[gkey][1], "Start_Timestamp": 1000 * i,
                       "End_Timestamp": 1000 * i + dur})
    _write_csv(str(tmp_path / "kt" / "x_kernel_trace.csv"), kt)
    half_kib = w.state_bytes / 2 / 1024
    chunk_kib = w.state_bytes * 32 // w.batch / 1024

    def counters(name, small, state, row, col):
        rows = []
        for key, gkey, val in (("copy", "copy_small", small), ("copy", "copy_state", state),
                               ("row", "row", row), ("col", "col", col)):
            for i in range(2):
                rows.append({"Kernel_Name": names[key],
                             "Grid_Size": grids[gkey][0] * grids[gkey][1],
                             "Counter_Name": name, "Counter_Value": val,
                             "Dispatch_Id": "%s%d" % (gkey, i)})
        return rows
    # FETCH_SIZE reads half the bytes a copy moves, WRITE_SIZE all of them
    _write_csv(str(tmp_path / "f" / "x_counter_collection.csv"),
               counters("FETCH_SIZE", 64 * 1024 / 2, half_kib / 2, chunk_kib / 2, chunk_kib / 2))
    _write_csv(str(tmp_path / "w" / "x_counter_collection.csv"),
               counters("WRITE_SIZE", 64 * 1024, half_kib, chunk_kib, chunk_kib))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "profiles" / "traffic.json"))
    bench.summarize_profile(w.name, str(tmp_path / "kt"), str(tmp_path / "f"),
                            str(tmp_path / "w"), "rocprofv3 ...")
    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))["workloads"][w.name]
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    for p in ("0", "1"):
        assert rec["passes"][p]["bytes_per_launch"] == pytest.approx(2 * chunk_kib * 1024)
    text = open(tmp_path / "profiles" / ("%s_traffic.txt" % w.name)).read()
    assert "0.42" in text.splitlines()[-1] or "0.43" in text.splitlines()[-1]


def test_profile_summary_of_a_cache_resident_workload_keeps_both_plans(tmp_path, monkeypatch,
                                                                       lib):
    """n=14 batch 64 is timed with its configured 7|7 split and with the
    default one-pass plan: the summary keeps a counter record for each, and
    each configured record reads its own plan's bytes back per call."""
    import quantum_state_encoding_amd as qse
    w = workloads.WORKLOADS["n14_b64_f32"]
    cfg = qse.Plan(w.n, w.dtype, split=w.split)
    dflt = qse.Plan(w.n, w.dtype)
    kernels = {("cfg", i): cfg.kernel_name(i, w.batch) for i in range(cfg.num_passes)}
    kernels[("dflt", 0)] = dflt.kernel_name(0, w.batch)
    full = {k: "void qse::(anonymous namespace)::%s(float*, float*, qse::TileArgs)" % v
            for k, v in kernels.items()}
    full["copy"] = "stream_copy_kernel(int4*, int4 const*, long)"
    grid = {("cfg", 0): 65536, ("cfg", 1): 32768, ("dflt", 0): 65536, "copy": 524288}
    kt = [{"Kernel_Name": full[k], "Grid_Size_X": grid[k], "Grid_Size_Y": 2,
           "Start_Timestamp": 0, "End_Timestamp": 5000} for k in full for _ in range(3)]
    _write_csv(str(tmp_path / "kt" / "x_kernel_trace.csv"), kt)
    half = w.state_bytes / 1024 / 2          # KiB of half the state

    def counters(name, per_kernel, copy):
        rows = []
        for k in full:
            v = copy if k == "copy" else per_kernel[k]
            g = grid[k] * (1 if k == "copy" else 2)
            rows += [{"Kernel_Name": full[k], "Grid_Size": g, "Counter_Name": name,
                      "Counter_Value": v, "Dispatch_Id": str(i)} for i in range(2)]
        return rows
    # Synthetic counters: FETCH_SIZE reads half the bytes it stands for (the
    # copy: 64 MiB / 2), and the passes move different amounts so that the
    # plans can be told apart.
    fetch = {("cfg", 0): half / 4 / 2, ("cfg", 1): half / 2, ("dflt", 0): half / 2}
    write = {("cfg", 0): half, ("cfg", 1): half, ("dflt", 0): half}
    _write_csv(str(tmp_path / "f" / "x_counter_collection.csv"),
               counters("FETCH_SIZE", fetch, 64 * 1024 / 2))
    _write_csv(str(tmp_path / "w" / "x_counter_collection.csv"),
               counters("WRITE_SIZE", write, 64 * 1024))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "profiles" / "traffic.json"))
    bench.summarize_profile(w.name, str(tmp_path / "kt"), str(tmp_path / "f"),
                            str(tmp_path / "w"), "rocprofv3 ...")
    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))["workloads"][w.name]
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["calibration_copy_bytes"] == 64 << 20
    assert set(rec["plans"]) == {"as configured", "default plan"}
    assert len(rec["plans"]["as configured"]["passes"]) == 2
    assert len(rec["plans"]["default plan"]["passes"]) == 1
    monkeypatch.setattr(bench, "traffic_record", lambda name: rec)
    monkeypatch.setattr(bench, "lds_conflicts", lambda name, kernel: None)
    S = w.state_bytes
    c = bench.counter_fields(w, "as configured", {"passes": 2})
    assert c["fetch_bytes"] == pytest.approx(S / 4 / 2 + S / 2)
    assert c["write_bytes"] == pytest.approx(2 * S / 2)
    assert c["measured_over_accounted"] == pytest.approx((S / 8 + S / 2 + S) / (4 * S))
    d = bench.counter_fields(w, "default plan", {"passes": 1})
    assert d["fetch_bytes"] == pytest.approx(S / 2) and d["write_bytes"] == pytest.approx(S / 2)
    assert d["measured_over_accounted"] == pytest.approx(0.5)
    assert bench.counter_fields(w, "default plan", {"passes": 2}) == {}


def test_counter_records_are_keyed_to_the_sources_of_the_kernels_they_traced(tmp_path,
                                                                              monkeypatch):
    # Three stand-in sources: helpers, pass kernels, the one-pass kernel.
    srcs = []
    for name, text in (("h.h", "int helper;"), ("k.hip", "int pass;"), ("o.hip", "int one;")):
        p = tmp_path / name
        p.write_text(text)
        srcs.append(str(p))
    monkeypatch.setattr(bench, "KERNEL_SRC", srcs)
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    recs = {"passes_only": {"plans": {"as configured": {"onepass": False}}},
            "with_onepass": {"plans": {"as configured": {"onepass": True},
                                       "two-pass": {"onepass": False}}}}
    recs["passes_only"]["kernel_source_sha256_16"] = bench.kernel_source_hash(False)
    recs["with_onepass"]["kernel_source_sha256_16"] = bench.kernel_source_hash(True)
    traffic.write_text(json.dumps({"workloads": recs}))
    assert bench.traffic_record("passes_only") and bench.traffic_record("with_onepass")
    # Comments and whitespace do not change the key.
    (tmp_path / "o.hip").write_text("int  one; // a note\n")
    assert bench.traffic_record("with_onepass")
    # A code change in the one-pass kernel stales only the record that traced it.
    (tmp_path / "o.hip").write_text("int one2;")
    assert bench.traffic_record("passes_only")
    assert bench.traffic_record("with_onepass") is None
    # A code change in the pass kernels stales both.
    (tmp_path / "k.hip").write_text("int pass2;")
    assert bench.traffic_record("passes_only") is None
