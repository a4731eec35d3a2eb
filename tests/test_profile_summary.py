"""bench.py's rocprofv3 summary (--profile) on synthetic profiler output: the
figures it derives from a kernel trace and the counter runs (launch duration,
launches per step, shader clock, matrix-pipe and VALU busy, HBM bytes scaled
by the copy calibration, staging-copy overlap, the bench's own event timing
of the traced command) are recomputed here by hand from the same numbers."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from long_context_blockwise_amd import inputs  # noqa: E402

NAME = "prefill_bf16_h32_d128"
KERNEL = "void ra::(anonymous namespace)::fwd_bf16_kernel<128, 64, 4, 1, 2, 0>(ra::FwdArgs)"
STEPS = 2            # timed steps of the traced command (plus one warmup)
LAUNCHES = 4         # dominant-kernel launches per step
DUR_NS = [1_000_000, 1_200_000, 800_000, 1_000_000] * (STEPS + 1)
GRBM = 8 * 1_700_000.0  # GRBM_GUI_ACTIVE sums the 8 XCDs: 1.7 GHz over a 1 ms launch


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _runs(tmp, json_line):
    runs = {}
    # trace: the attention launches back to back, one staging copy per launch
    # overlapping its first half
    t = 0
    trace, copies = [], []
    for i, d in enumerate(DUR_NS):
        trace.append({"Kernel_Name": KERNEL, "Start_Timestamp": t, "End_Timestamp": t + d})
        copies.append({"Kernel_Name": "__amd_rocclr_copyBuffer", "Start_Timestamp": t, "End_Timestamp": t + d // 2})
        t += d + 10_000
    d = os.path.join(tmp, "trace")
    os.makedirs(d)
    _write_csv(os.path.join(d, "x_kernel_trace.csv"), trace + copies)
    _write_csv(os.path.join(d, "x_kernel_stats.csv"),
               [{"Name": KERNEL, "Calls": len(DUR_NS), "TotalDurationNs": sum(DUR_NS),
                 "AverageNs": sum(DUR_NS) / len(DUR_NS), "MinNs": min(DUR_NS), "MaxNs": max(DUR_NS)}])
    with open(os.path.join(d, "rocprof.log"), "w") as f:
        f.write("[bench] noise\n" + json_line + "\n---- stderr ----\n{not json on stderr}\n")
    runs["trace"] = (d, "trace-cmd")
    counters = {
        "pipes": {"GRBM_GUI_ACTIVE": GRBM, "SQ_VALU_MFMA_BUSY_CYCLES": 0.6 * 1_700_000 * 1024,
                  "SQ_ACTIVE_INST_VALU": 0.4 * 1_700_000 * 256, "SQ_VALU_MFMA_COEXEC_CYCLES": 0.2 * 1_700_000 * 1024,
                  "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1e9, "SQ_INSTS_VALU": 450.0, "SQ_INSTS_MFMA": 100.0},
        "lds": {"GRBM_GUI_ACTIVE": GRBM, "SQ_ACTIVE_INST_LDS": 0.1 * 1_700_000 * 256, "SQ_LDS_BANK_CONFLICT": 0.0,
                "SQ_INSTS_LDS": 10.0, "SQ_INSTS_VALU_TRANS_F32": 100.0, "SQ_WAVES": 1.0},
        "fetch": {"FETCH_SIZE": 1000.0},
        "write": {"WRITE_SIZE": 500.0},
    }
    for key, vals in counters.items():
        d = os.path.join(tmp, key)
        os.makedirs(d)
        rows = []
        for disp in range(len(DUR_NS)):
            for cname, v in vals.items():
                rows.append({"Dispatch_Id": disp, "Kernel_Name": KERNEL, "Counter_Name": cname, "Counter_Value": v})
            # another kernel's dispatch in the same run is not counted
            rows.append({"Dispatch_Id": 10_000 + disp, "Kernel_Name": "other_kernel",
                         "Counter_Name": next(iter(vals)), "Counter_Value": 1e12})
        _write_csv(os.path.join(d, "x_counter_collection.csv"), rows)
        runs[key] = (d, f"{key}-cmd")
    return runs


def test_profile_summary_figures(tmp_path):
    wl = inputs.WORKLOADS[NAME]
    flops, kv_bytes = bench.algorithmic(wl)
    avg_ns = sum(DUR_NS) / len(DUR_NS)
    ev_tflops = 1234.5
    runs = _runs(str(tmp_path), json.dumps({"metric": "m", "roofline": {"achieved": ev_tflops}}))
    calib = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    out = bench.write_profile_summary(NAME, runs, calib, str(tmp_path), STEPS)

    assert out["launches_per_step"] == pytest.approx(LAUNCHES)
    assert out["avg_us"] == pytest.approx(avg_ns / 1e3)
    assert out["clock_ghz"] == pytest.approx(GRBM / 8 / avg_ns)
    assert out["mfma_busy"] == pytest.approx(0.6)
    assert out["valu_busy"] == pytest.approx(0.4)
    assert out["coexec"] == pytest.approx(0.2)
    assert out["lds_busy"] == pytest.approx(0.1)
    assert out["fetch_bytes"] == pytest.approx(1000.0 * 1024 * 2.0)
    assert out["write_bytes"] == pytest.approx(500.0 * 1024 * 1.0)
    assert out["traffic_bytes"] == pytest.approx(1000.0 * 1024 * 2.0 + 500.0 * 1024)
    assert out["achieved_tflops"] == pytest.approx(flops / LAUNCHES / avg_ns / 1e3)
    assert out["achieved_gbs"] == pytest.approx(kv_bytes / LAUNCHES / avg_ns)
    st = out["staging"]
    timed = DUR_NS[-STEPS * LAUNCHES:]  # only the timed steps' launches (and their copies) are priced
    assert st["copies"] == len(timed)
    assert st["copy_ns"] == sum(d // 2 for d in timed)
    assert st["overlap_ns"] == st["copy_ns"]  # every copy lies inside its launch
    assert st["copy_frac_of_kernel_time"] == pytest.approx(0.5)

    text = open(out["file"]).read()
    assert "trace-cmd" in text and "fetch-cmd" in text
    # the bench's event timing of the traced command, converted back to a launch time
    ev_us = flops / LAUNCHES / ev_tflops * 1e-3 / 1e3
    assert "bench events in the traced command" in text
    assert f"({ev_tflops:.5g} TFLOP/s)" in text
    assert f"{ev_us:.5g} µs per launch" in text


def test_profile_summary_without_event_line(tmp_path):
    runs = _runs(str(tmp_path), "no json here")
    out = bench.write_profile_summary(NAME, runs, {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}, str(tmp_path), STEPS)
    text = open(out["file"]).read()
    assert "bench events in the traced command" not in text
    assert out["mfma_busy"] == pytest.approx(0.6)


def test_profile_summary_prices_only_timed_steps(tmp_path):
    """With the child's JSON line reporting 3 untimed steps (warmup and the
    step estimate), the summary keeps only the last STEPS steps' dispatches:
    here the untimed launches are made twice as long, and the average must
    not see them."""
    global DUR_NS
    saved = DUR_NS
    untimed = 3
    DUR_NS = [2 * d for d in [1_000_000, 1_200_000, 800_000, 1_000_000]] * untimed + \
        [1_000_000, 1_200_000, 800_000, 1_000_000] * STEPS
    try:
        line = json.dumps({"metric": "m", "run_info": {"untimed_steps": untimed}})
        runs = _runs(str(tmp_path), line)
        out = bench.write_profile_summary(NAME, runs, {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}, str(tmp_path), STEPS)
    finally:
        DUR_NS = saved
    assert out["launches_per_step"] == pytest.approx(LAUNCHES)
    assert out["avg_us"] == pytest.approx(1000.0)
    assert out["staging"]["copies"] == STEPS * LAUNCHES
    text = open(out["file"]).read()
    assert f"{STEPS} timed + {untimed} untimed steps" in text
