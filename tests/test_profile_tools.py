"""Host-side checks of the rocprofv3 summary tooling (no GPU): the derived
matrix-core figures and the bench's lookup of the committed summary."""
import csv
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from block_sparse_split_amd import rocprof_summary as rs  # noqa: E402


def _write_csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_counters_summary_derived_values(tmp_path, monkeypatch):
    # one warm-up dispatch (skipped) and two timed ones of a 1 ms kernel at
    # 2 GHz: 2e6 cycles per XCD, reported summed over 8 XCDs
    name = "void skv::(anonymous namespace)::bwd_dkdv_kernel<128>(skv::BwdArgs)"
    rows = []
    for did, busy in ((1, 9.9e9), (2, 1.024e9), (3, 1.024e9)):
        vals = {"SQ_VALU_MFMA_BUSY_CYCLES": busy, "SQ_VALU_MFMA_COEXEC_CYCLES": busy / 4,
                "SQ_INSTS_VALU_MFMA_MOPS_BF16": 2e9, "SQ_INSTS_MFMA": 1e7,
                "SQ_INSTS_VALU": 5e7, "SQ_INSTS_VALU_TRANS_F32": 5e6, "SQ_INSTS_LDS": 2e7,
                "SQ_LDS_BANK_CONFLICT": 0, "GRBM_GUI_ACTIVE": 8 * 2e6}
        for cn, v in vals.items():
            rows.append((did, name, cn, v, 1000, 1000 + 1_000_000))
    src = tmp_path / "c.csv"
    out = tmp_path / "s.txt"
    _write_csv(src, rows)
    rs.main(["counters", str(src), "--workload", "w", "--command", "cmd", "--skip-first", "1",
             "--out", str(out)])
    text = out.read_text()
    row = [l.split() for l in text.splitlines() if l.startswith("bwd_dkdv")][0]
    # busy = 1.024e9 / (2e6 cycles x 1024 SIMDs) = 50 %; co-issue = 25 %
    assert row[1] == "2" and row[2] == "50.0%" and row[3] == "25.0%"
    # 2e9 MOPS x 512 FLOP = 1.024 TFLOP in 1 ms at 2 GHz
    assert row[4] == "1.0240" and row[5] == "2.000" and row[6] == "1024.0"

    import bench
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    (tmp_path / "profiles" / "mfma_util_w.txt").write_text(text)
    got = bench.mfma_counters_for("bwd_dkdv", "w", rs.kernel_source_hash())
    assert got == {"mfma_busy": 0.5, "mfma_valu_coexec": 0.25, "clock_ghz": 2.0}
    # a summary taken on other kernel sources is not reported
    assert bench.mfma_counters_for("bwd_dkdv", "w", "0" * 64) is None


def test_kernels_summary_without_bench_figures(tmp_path):
    """Kernel statistics beside a bench record that has no per-kernel
    figures (the 1M merge workload's): the column shows '-'."""
    stats = tmp_path / "stats.csv"
    trace = tmp_path / "trace.csv"
    name = "void skv::(anonymous namespace)::fwd_bf16_kernel<128>(skv::FwdArgs)"
    with open(stats, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow([name, 3, 3_000_000, 1_000_000.0, 100.0, 900_000, 1_100_000, 1.0])
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, dur in enumerate((1_100_000, 1_000_000, 900_000)):
            w.writerow([name, 10_000_000 * i, 10_000_000 * i + dur])
    bench_json = tmp_path / "b.json"
    bench_json.write_text('{"metric": "m", "value": 1.0}\n')
    out = tmp_path / "k.txt"
    rs.main(["kernels", str(stats), "--trace", str(trace), "--skip-first", "1",
             "--bench-json", str(bench_json), "--command", "cmd", "--out", str(out)])
    row = [l.split() for l in out.read_text().splitlines() if l.startswith("fwd_bf16")][-1]
    assert row == ["fwd_bf16", "2", "0.9500", "-"]


def test_l2_summary(tmp_path):
    """Hits and misses summed over rows per dispatch; warm-up skipped."""
    name = "void skv::(anonymous namespace)::fwd_bf16_kernel<128>(skv::FwdArgs)"
    rows = []
    for did, (h, m) in ((1, (1.0, 1e9)), (2, (3e6, 1e6)), (3, (3e6, 1e6))):
        for part in range(2):  # two rows per counter
            rows.append((did, name, "TCC_HIT_sum", h / 2, 0, 1))
            rows.append((did, name, "TCC_MISS_sum", m / 2, 0, 1))
    src = tmp_path / "l2.csv"
    out = tmp_path / "l2.txt"
    _write_csv(src, rows)
    rs.main(["l2", str(src), "--workload", "w", "--command", "cmd", "--skip-first", "1",
             "--out", str(out)])
    row = [l.split() for l in out.read_text().splitlines() if l.startswith("fwd_bf16")][0]
    assert row == ["fwd_bf16", "2", "3000000", "1000000", "75.0%", "128.0"]


def _json_line(path, rec):
    import json
    path.write_text("some log line\n" + json.dumps(rec) + "\n")


def test_bench_tables(tmp_path):
    """The balance, sweep and plan tables read the last JSON line of a bench
    run and print its figures as percentages / relative XCD means."""
    k = {"planned_imbalance": 0.005, "realized_imbalance_median": 0.04,
         "mean_workgroup_us": 100.0, "kernel_span_us_median": 110.0,
         "xcd_mean_us": [101.0, 99.0] + [100.0] * 6, "on_xcd_w_plus_c_mod_8": 1.0,
         "xcd_rotation_per_run": [3, 3], "distinct_cus_per_run": 256}
    src = tmp_path / "wg.json"
    _json_line(src, {"workload": "w", "clock": "c", "workgroups": 256, "steps": 2,
                     "kernels": {"bwd_dq": k},
                     "kernels_xcd_plan": {"bwd_dq": dict(k, realized_imbalance_median=0.02)},
                     "kernels_calibrated_plan": {"bwd_dq": dict(
                         k, realized_imbalance_median=0.01,
                         decomposition={"if_xcd_speeds_matched": 0.008,
                                        "if_queue_residual_matched_too": 0.005,
                                        "queue_residual_rms": 0.002,
                                        "queue_residual_max": 0.006})},
                     "xcd_speed": [[1.0] * 8, [1.05] + [1.0] * 7, [0.9] * 8],
                     "cost_scale_range": [[0.95, 1.02], [0.9, 1.1]]})
    out = tmp_path / "b.txt"
    rs.main(["balance", str(src), "--command", "cmd", "--out", str(out)])
    lines = out.read_text().splitlines()
    uni, xcd, cal = [l.split() for l in lines if l.startswith("bwd_dq")]
    assert uni[1:5] == ["0.50%", "4.00%", "100.0", "110.0"]
    assert uni[5:7] == ["100.0%", "(c=3)"] and uni[7] == "256"
    assert uni[8:10] == ["+1.0%", "-1.0%"]
    assert xcd[1:3] == ["0.50%", "2.00%"] and cal[1:3] == ["0.50%", "1.00%"]
    assert [l.split()[2] for l in lines if l.startswith("speed")] == ["1.000", "1.050", "0.900"]
    assert [l.split()[3:] for l in lines if l.startswith("cost scales")] == [
        ["0.950", "..", "1.020"], ["0.900", "..", "1.100"]]
    # the spread decomposition, for the plans that carry one
    dec = [l.split() for l in lines if l.startswith("calibrated ")]
    assert dec == [["calibrated", "bwd_dq", "1.00%", "0.80%", "0.50%", "0.20%", "/", "0.60%"]]
    # a record without the per-XCD plan prints the uniform table only
    _json_line(src, {"workload": "w", "clock": "c", "workgroups": 256, "steps": 2,
                     "kernels": {"bwd_dq": k}})
    rs.main(["balance", str(src), "--command", "cmd", "--out", str(out)])
    assert sum(l.startswith("bwd_dq") for l in out.read_text().splitlines()) == 1

    src = tmp_path / "sw.json"
    _json_line(src, {"points": [{"context": 4096, "draft_queries": 512, "ms_per_step": 0.5,
                                 "tflops_fwd_bwd": 400.0, "frac_of_bf16_peak": 0.16,
                                 "tflops_fwd": 500.0, "fwd_ms": 0.1,
                                 "item_imbalance_256cu": 0.02, "plan_ms": 0.3}]})
    rs.main(["sweep", str(src), "--over", "context", "--command", "cmd", "--out", str(out)])
    text = out.read_text()
    assert text.startswith("# fwd+bwd throughput over context")
    row = [l.split() for l in text.splitlines() if l.startswith("   4096")][0]
    assert row == ["4096", "512", "0.500", "400.0", "0.160", "500.0", "0.100", "2.00%", "0.300"]

    src = tmp_path / "cmp.json"
    cmp = {"plan": "contiguous runs",
           "fwd_bf16": {"lpt_ms": 1.0, "contiguous_ms": 1.5, "gain": 1.5},
           "bwd_dq": {"lpt_ms": 2.0, "contiguous_ms": 3.0, "gain": 1.5}}
    _json_line(src, {"config": {"workload": "w", "seed": 1}, "in_gpu_plan_comparison": cmp})
    rs.main(["plans", str(src), "--command", "cmd", "--out", str(out)])
    rows = [l.split() for l in out.read_text().splitlines() if l.startswith(("fwd_", "bwd_"))]
    assert rows == [["fwd_bf16", "1.000", "1.500", "1.50x"], ["bwd_dq", "2.000", "3.000", "1.50x"]]
