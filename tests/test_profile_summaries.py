"""The profile summaries under profiles/ are written by bench.py from raw
rocprofv3 output: these CPU tests run the three generators on small
synthetic traces and counter files whose right answers are known by hand
(timed dispatches picked by their order, counter scaling from the bench's
calibration copy, MFMA busy from its definition)."""
import csv
import gzip
import json
import os

import pytest

import bench

NC = "void sattn::fwd_kernel<sattn::Bf16, 128, 64, 8, false, 0>(sattn::FwdParams)"
CA = "void sattn::fwd_kernel<sattn::Bf16, 128, 64, 8, true, 0>(sattn::FwdParams)"
SPLIT = "void sattn::split_row_kernel<sattn::Bf16, 128, false>(sattn::FwdParams)"
COPY = "__amd_rocclr_copyBuffer"


def _bench_log(path, steps=3, before=2, extra=None):
    line = {"metric": "m", "value": 1.0, "steps": steps, "ms_per_step": 0.75,
            "config": {"flop_per_launch": {"noncausal": 5.0e11, "causal": 2.5e11},
                       "algorithmic_bytes_per_launch": 1000.0},
            "roofline": {"achieved": 1100.0, "frac": 0.44},
            "extras": {"launches_before_timing": {"noncausal": before, "causal": before},
                       "kernel_source_sha256": "feed",
                       "noncausal_launch_ms": {"mean": 0.46, "median": 0.46},
                       "causal_launch_ms": {"mean": 0.25, "median": 0.25}}}
    line["extras"].update(extra or {})
    with open(path, "w") as fh:
        fh.write("[bench] progress\n" + json.dumps(line) + "\n")
    return str(path)


def _counters(d, counter, rows, zipped=False):
    """rows: (dispatch id, kernel, value) in dispatch order."""
    os.makedirs(d, exist_ok=True)
    name = os.path.join(d, "pmc_counter_collection.csv")
    opener = (lambda p: gzip.open(p + ".gz", "wt", newline="")) if zipped else (lambda p: open(p, "w", newline=""))
    with opener(name) as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for did, k, v in rows:
            w.writerow([did, k, counter, v])
    return str(d)


def _headline_rows(start, nc_vals, ca_vals):
    rows, did = [], start
    for a, b in zip(nc_vals, ca_vals):   # the bench alternates noncausal and causal launches
        rows.append((did, NC, a))
        rows.append((did + 1, CA, b))
        did += 2
    return rows


def test_pmc_summary_scales_and_picks_timed_dispatches(tmp_path):
    # 5 launches of each headline kernel: 2 before timing, then 3 timed
    nc_f, ca_f = [9, 9, 40, 50, 60], [9, 9, 70, 80, 90]       # FETCH_SIZE KiB
    nc_w, ca_w = [1, 1, 10, 10, 10], [1, 1, 20, 20, 20]       # WRITE_SIZE KiB
    fetch = _counters(tmp_path / "f", "FETCH_SIZE",
                      [(1, COPY, 131072.0)] + _headline_rows(2, nc_f, ca_f) + [(20, SPLIT, 512.0), (21, COPY, 9e9)],
                      zipped=True)
    write = _counters(tmp_path / "w", "WRITE_SIZE",
                      [(1, COPY, 262144.0)] + _headline_rows(2, nc_w, ca_w) + [(20, SPLIT, 4.0)])
    logs = [_bench_log(tmp_path / "bf.log", extra={"splitkv_decode": {"algorithmic_bytes_split": 1048576.0}}),
            _bench_log(tmp_path / "bw.log", extra={"splitkv_decode": {"algorithmic_bytes_split": 1048576.0}})]
    js = bench.pmc_summary(fetch, write, logs, ["cmd f", "cmd w"], out=str(tmp_path / "out.json"))
    # the first device copy (256 MiB) calibrates: FETCH_SIZE reads half of it, x2; WRITE_SIZE all of it, x1
    assert js["counter_scale"]["FETCH_SIZE"] == pytest.approx(2.0)
    assert js["counter_scale"]["WRITE_SIZE"] == pytest.approx(1.0)
    nc = js["per_launch"]["noncausal"]
    assert nc["fetch_bytes"] == pytest.approx(50 * 2.0 * 1024)     # median of the timed 40, 50, 60
    assert nc["write_bytes"] == pytest.approx(10 * 1024)
    assert nc["ratio"] == pytest.approx((50 * 2 + 10) * 1024 / 1000.0)
    assert js["per_launch"]["causal"]["fetch_bytes"] == pytest.approx(80 * 2.0 * 1024)
    assert js["hbm_bytes_per_launch"] == pytest.approx(nc["fetch_bytes"] + nc["write_bytes"])
    sp = js["per_kernel"][bench._kname(SPLIT)]
    assert sp["algorithmic_bytes"] == 1048576.0
    assert sp["fetch_bytes"] == pytest.approx(512 * 2.0 * 1024) and sp["write_bytes"] == pytest.approx(4 * 1024)
    md = open(tmp_path / "out.md").read()
    assert "cmd f" in md and "| noncausal | 0.1 | 0.0 | 0.0 | 112.64 |" in md
    assert json.load(open(tmp_path / "out.json"))["kernel_source_sha256"] == "feed"


def test_pmc_summary_rejects_runs_on_different_sources(tmp_path):
    rows = [(1, COPY, 1.0)] + _headline_rows(2, [1] * 5, [1] * 5)
    f = _counters(tmp_path / "f", "FETCH_SIZE", rows)
    w = _counters(tmp_path / "w", "WRITE_SIZE", rows)
    a = _bench_log(tmp_path / "a.log")
    b = _bench_log(tmp_path / "b.log", extra={"kernel_source_sha256": "other"})
    with pytest.raises(SystemExit):
        bench.pmc_summary(f, w, [a, b], [], out=str(tmp_path / "x.json"))


def test_trace_summary_timed_dispatches(tmp_path):
    d = tmp_path / "trace"
    os.makedirs(d)
    # ns timestamps: noncausal launches of 400, 400, 450, 460, 470 us; causal 200, 200, 240, 250, 260 us
    with open(d / "trace_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 0
        for i, (a, b) in enumerate(zip([400, 400, 450, 460, 470], [200, 200, 240, 250, 260])):
            w.writerow([2 * i + 1, NC, t, t + a * 1000])
            t += a * 1000
            w.writerow([2 * i + 2, CA, t, t + b * 1000])
            t += b * 1000
    md = bench.trace_summary(str(d), _bench_log(tmp_path / "b.log"), "the command")
    assert "the command" in md
    # timed: 450, 460, 470 (mean 460) and 240, 250, 260 (mean 250)
    assert "| noncausal | `fwd_kernel<Bf16, 128, 64, 8, false, 0>` | 3 | 460.00 | 460.00 |" in md
    assert "| causal | `fwd_kernel<Bf16, 128, 64, 8, true, 0>` | 3 | 250.00 | 250.00 |" in md
    assert "| 1087.0 | 0.4348 |" in md            # 5e11 FLOP / 460 us
    assert "sum to 710.00 us on average" in md


def test_sq_summary_mfma_busy(tmp_path):
    d = tmp_path / "sq"
    os.makedirs(d)
    with open(d / "pmc_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for did in range(1, 11):
            k = NC if did % 2 else CA
            for c in bench.SQ_COUNTERS:
                # GRBM_GUI_ACTIVE sums 8 XCDs: 8000 -> 1000 cycles; 1024 SIMDs -> 1.024e6 SIMD cycles
                v = 8000.0 if c == "GRBM_GUI_ACTIVE" else (512000.0 if c == "SQ_VALU_MFMA_BUSY_CYCLES" else 1.0)
                w.writerow([did, k, c, v])
    md = bench.sq_summary(str(d), _bench_log(tmp_path / "b.log"), "sq command")
    assert "| MFMA busy | 50.0% | 50.0% |" in md
