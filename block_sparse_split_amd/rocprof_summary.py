"""Turn rocprofv3 CSV output into the short text summaries kept with the
sources.

  kernels  -- per-kernel call count / average / share from a
              `rocprofv3 --kernel-trace --stats --output-format csv` run
  traffic  -- HBM bytes per launch of one kernel from two `--pmc` runs
              (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by
              what the same counter reads for a plain elementwise copy of a
              known number of bytes
  counters -- matrix-core utilisation per kernel from one `--pmc` run of the
              SQ/GRBM counters listed in MFMA_COUNTERS
  l2       -- L2 (TCC) hits and misses per dispatch of each kernel from one
              `--pmc TCC_HIT_sum TCC_MISS_sum` run
  balance  -- the table of a `bench.py --wg-times` JSON line (planned against
              realised workgroup imbalance, placement and per-XCD means)
  sweep    -- the table of a `bench.py --sweep context|budget` JSON line
  plans    -- the table of a `bench.py --compare-plans` JSON line

Usage:
  python -m block_sparse_split_amd.rocprof_summary kernels STATS_CSV \\
      --command "..." [--trace TRACE_CSV --skip-first N --bench-json OUT] [--out FILE]
  python -m block_sparse_split_amd.rocprof_summary traffic KERNEL \\
      --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV \\
      --copy-bytes N --workload NAME --command "..." [--skip-first N] [--out FILE]
  python -m block_sparse_split_amd.rocprof_summary counters CSV \\
      --workload NAME --command "..." [--skip-first N] [--out FILE]
  python -m block_sparse_split_amd.rocprof_summary l2 CSV \\
      --workload NAME --command "..." [--skip-first N] [--out FILE]
  python -m block_sparse_split_amd.rocprof_summary balance|plans JSON \\
      --command "..." [--out FILE]
  python -m block_sparse_split_amd.rocprof_summary sweep JSON --over "..." \\
      --command "..." [--out FILE]
"""
import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# short names used by the library's own launch timing
SHORT = {
    "fwd_bf16_kernel": "fwd_bf16", "fwd_f32_kernel": "fwd_f32",
    "merge_split_kernel": "merge_split", "merge_kernel": "merge",
    "bwd_pre_kernel": "bwd_pre", "bwd_dq_kernel": "bwd_dq",
    "dq_reduce_kernel": "dq_reduce", "bwd_dkdv_kernel": "bwd_dkdv",
    "dq_finalize_kernel": "dq_finalize", "xcd_reset_kernel": "xcd_reset",
}


def short_name(kernel_name):
    for key, short in SHORT.items():
        if key in kernel_name:
            return short
    return None


def kernel_source_hash():
    """sha256 over the kernel sources (csrc/*.hip, csrc/*.h, sorted by name)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_split_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def counter_per_dispatch(path, counter, match, skip_first=0):
    """Mean over dispatches of `counter` (summed over its per-dimension rows)
    for kernels whose name satisfies `match`, without the first
    `skip_first` dispatches (in dispatch order)."""
    per_dispatch = defaultdict(float)
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] != counter or not match(row["Kernel_Name"]):
            continue
        per_dispatch[row["Dispatch_Id"]] += float(row["Counter_Value"])
    vals = [per_dispatch[d] for d in sorted(per_dispatch, key=int)][skip_first:]
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for the requested kernel")
    return sum(vals) / len(vals), len(vals)


def cmd_kernels(a):
    rows = list(csv.DictReader(open(a.stats)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"# rocprofv3 kernel statistics", f"command: {a.command}",
           f"kernel_source_sha256: {kernel_source_hash()}", "",
           "all dispatches:",
           f"{'kernel':<14} {'calls':>6} {'avg_ms':>9} {'min_ms':>9} {'max_ms':>9} {'share':>7}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = short_name(r["Name"]) or ("torch_elementwise" if "at::native" in r["Name"] else r["Name"][:40])
        out.append(f"{name:<14} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e6:>9.4f} "
                   f"{float(r['MinNs']) / 1e6:>9.4f} {float(r['MaxNs']) / 1e6:>9.4f} "
                   f"{100 * float(r['TotalDurationNs']) / total:>6.2f}%")
    if a.trace:
        # per-dispatch durations without the warm-up launches, beside the
        # bench's own HIP-event averages from the same run
        per = defaultdict(list)
        for r in csv.DictReader(open(a.trace)):
            name = short_name(r["Kernel_Name"])
            if name:
                per[name].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        bench = {}
        if a.bench_json:
            line = open(a.bench_json).read().strip().splitlines()[-1]
            bench = {k: v.get("avg_ms") for k, v in json.loads(line).get("kernels", {}).items()}
        out += ["", f"timed dispatches (first {a.skip_first} of each kernel skipped as warm-up):",
                f"{'kernel':<14} {'calls':>6} {'avg_ms':>9} {'bench_avg_ms':>13}"]
        for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            d = d[a.skip_first:]
            if not d:
                continue
            b = bench.get(name)
            out.append(f"{name:<14} {len(d):>6} {sum(d) / len(d) / 1e6:>9.4f} "
                       f"{'-' if b is None else f'{b:.4f}':>13}")
    emit("\n".join(out) + "\n", a.out)


def cmd_traffic(a):
    is_k = lambda n: short_name(n) == a.kernel
    is_copy = lambda n: "neg_kernel" in n
    f_kib, nf = counter_per_dispatch(a.fetch, "FETCH_SIZE", is_k, a.skip_first)
    w_kib, nw = counter_per_dispatch(a.write, "WRITE_SIZE", is_k, a.skip_first)
    cf_kib, _ = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", is_copy)
    cw_kib, _ = counter_per_dispatch(a.copy_write, "WRITE_SIZE", is_copy)
    f_scale = a.copy_bytes / (cf_kib * 1024.0)
    w_scale = a.copy_bytes / (cw_kib * 1024.0)
    lines = [
        f"# HBM traffic of {a.kernel} on workload {a.workload}",
        f"command: {a.command}",
        f"kernel: {a.kernel}",
        f"workload: {a.workload}",
        f"kernel_source_sha256: {kernel_source_hash()}",
        f"dispatches skipped as warm-up (each run): {a.skip_first}",
        f"dispatches_fetch: {nf}",
        f"dispatches_write: {nw}",
        f"fetch_kib_per_dispatch_raw: {f_kib:.1f}",
        f"write_kib_per_dispatch_raw: {w_kib:.1f}",
        f"copy_probe_bytes: {a.copy_bytes}",
        f"copy_fetch_kib_raw: {cf_kib:.1f}",
        f"copy_write_kib_raw: {cw_kib:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"fetch_bytes_per_launch: {f_kib * 1024.0 * f_scale:.0f}",
        f"write_bytes_per_launch: {w_kib * 1024.0 * w_scale:.0f}",
    ]
    emit("\n".join(lines) + "\n", a.out)


# one --pmc pass: 8 SQ counters and 1 GRBM counter (the per-block limits)
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                 "SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_LDS "
                 "SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE")
N_SIMD = 1024  # 256 CUs x 4 SIMDs
N_XCD = 8


def cmd_counters(a):
    """Matrix-core utilisation of each library kernel.

    Per dispatch, SQ counters are summed over their rows and GRBM_GUI_ACTIVE
    (GPU busy cycles) is the maximum over its rows.  Derived figures:
      mfma_busy   = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs)
      coexec      = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES, the
                    share of matrix-busy cycles in which a plain VALU
                    instruction also issued on that SIMD
      mfma_tflop  = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP (executed work)
      clock_ghz   = GRBM_GUI_ACTIVE / dispatch duration, when the CSV carries
                    timestamps
    """
    vals = defaultdict(lambda: defaultdict(list))   # kernel -> counter -> [per dispatch]
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(list)))
    durs = defaultdict(dict)
    for row in csv.DictReader(open(a.csv)):
        name = short_name(row["Kernel_Name"])
        if not name:
            continue
        did = row["Dispatch_Id"]
        per[name][did][row["Counter_Name"]].append(float(row["Counter_Value"]))
        if row.get("Start_Timestamp") and row.get("End_Timestamp"):
            durs[name][did] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    out = [f"# matrix-core utilisation per kernel on workload {a.workload}",
           f"command: {a.command}",
           f"kernel_source_sha256: {kernel_source_hash()}",
           f"counters: {MFMA_COUNTERS}",
           f"dispatches per kernel: first {a.skip_first} skipped as warm-up", ""]
    head = (f"{'kernel':<12} {'disp':>4} {'mfma_busy':>9} {'coexec':>7} {'mfma_TFLOP':>10} "
            f"{'clock_GHz':>9} {'exec_TFLOP/s':>12} {'valu/mfma':>9} {'trans/mfma':>10} "
            f"{'lds/mfma':>8} {'lds_conf':>8}")
    out.append(head)
    for name in sorted(per, key=lambda n: -sum(
            sum(c.get("SQ_VALU_MFMA_BUSY_CYCLES", [0])) for c in per[n].values())):
        dids = sorted(per[name], key=int)[a.skip_first:]
        if not dids:
            continue
        agg = defaultdict(float)
        dur = []
        for did in dids:
            for cn, v in per[name][did].items():
                agg[cn] += max(v) if cn.startswith("GRBM_") else sum(v)
            if did in durs[name]:
                dur.append(durs[name][did])
        n = len(dids)
        g = lambda cn: agg.get(cn, float("nan")) / n
        cyc = g("GRBM_GUI_ACTIVE")
        if not g("SQ_VALU_MFMA_BUSY_CYCLES") > 0:
            continue  # no matrix-core work (copies, reductions)
        # GRBM_GUI_ACTIVE arrives summed over the 8 XCDs of the GPU
        cyc /= N_XCD
        busy = g("SQ_VALU_MFMA_BUSY_CYCLES") / (cyc * N_SIMD)
        coex = g("SQ_VALU_MFMA_COEXEC_CYCLES") / g("SQ_VALU_MFMA_BUSY_CYCLES")
        flop = g("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
        mf = g("SQ_INSTS_MFMA")
        ns = sum(dur) / len(dur) if dur else float("nan")
        clock = cyc / ns
        out.append(f"{name:<12} {n:>4} {100 * busy:>8.1f}% {100 * coex:>6.1f}% {flop / 1e12:>10.4f} "
                   f"{clock:>9.3f} {flop / ns / 1e3:>12.1f} {g('SQ_INSTS_VALU') / mf:>9.2f} "
                   f"{g('SQ_INSTS_VALU_TRANS_F32') / mf:>10.2f} {g('SQ_INSTS_LDS') / mf:>8.2f} "
                   f"{g('SQ_LDS_BANK_CONFLICT') / cyc / 256:>8.4f}")
    out += ["", "valu/mfma, trans/mfma, lds/mfma: instructions per MFMA instruction "
            "(SQ_INSTS_VALU counts MFMAs too); lds_conf: LDS bank-conflict cycles per CU "
            "per GPU cycle"]
    emit("\n".join(out) + "\n", a.out)


def cmd_l2(a):
    """L2 requests of each library kernel: hits and misses per dispatch
    (each counter summed over its rows), the hit rate, and the miss count
    times the 128-byte L2 line as an upper bound on the bytes the misses
    bring in from beyond L2."""
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    for row in csv.DictReader(open(a.csv)):
        name = short_name(row["Kernel_Name"])
        if name:
            cn = row["Counter_Name"].replace("_sum", "")
            per[name][row["Dispatch_Id"]][cn] += float(row["Counter_Value"])
    out = [f"# L2 hits and misses per kernel on workload {a.workload}",
           f"command: {a.command}",
           f"kernel_source_sha256: {kernel_source_hash()}",
           f"dispatches per kernel: first {a.skip_first} skipped as warm-up", "",
           f"{'kernel':<12} {'disp':>4} {'hits/disp':>12} {'misses/disp':>12} {'hit_rate':>8} "
           f"{'miss_MB':>8}"]
    for name in sorted(per, key=lambda n: -sum(d.get("TCC_MISS", 0) for d in per[n].values())):
        dids = sorted(per[name], key=int)[a.skip_first:]
        if not dids:
            continue
        h = sum(per[name][d].get("TCC_HIT", 0.0) for d in dids) / len(dids)
        m = sum(per[name][d].get("TCC_MISS", 0.0) for d in dids) / len(dids)
        rate = h / (h + m) if h + m > 0 else float("nan")
        out.append(f"{name:<12} {len(dids):>4} {h:>12.0f} {m:>12.0f} {100 * rate:>7.1f}% "
                   f"{m * 128 / 1e6:>8.1f}")
    out += ["", "miss_MB = misses x 128 B per dispatch (an upper bound: a miss may fetch "
            "less than a line)"]
    emit("\n".join(out) + "\n", a.out)


def _last_json(path):
    return json.loads(open(path).read().strip().splitlines()[-1])


def cmd_balance(a):
    r = _last_json(a.json)
    out = [f"# per-workgroup balance of the forward, dQ and dK/dV kernels on workload "
           f"{r['workload']}",
           f"command: {a.command}",
           f"kernel_source_sha256: {kernel_source_hash()}",
           f"clock: {r['clock']}; workgroups: {r['workgroups']}; steps: {r['steps']}"]
    plans = [("uniform plan (skv_schedule_build)", r["kernels"])]
    if r.get("kernels_xcd_plan"):
        plans.append(("plan for per-XCD speeds (skv_schedule_build_xcd), speeds measured "
                      "on the uniform plan's steps", r["kernels_xcd_plan"]))
    if r.get("kernels_calibrated_plan"):
        plans.append(("plan for per-XCD speeds and cost scales (skv_schedule_build_xcd), "
                      "fitted to the stamps of the uniform and a first calibrated plan",
                      r["kernels_calibrated_plan"]))
    for title, kernels in plans:
        out += ["", f"## {title}"]
        if kernels is r.get("kernels_calibrated_plan"):
            for name, sp in zip(("forward", "dQ", "dK/dV"), r["xcd_speed"]):
                out.append(f"speed {name:<6} " + " ".join(f"{x:.3f}" for x in sp))
            for name, (lo, hi) in zip(("forward", "dQ"), r.get("cost_scale_range", [])):
                out.append(f"cost scales {name:<7} {lo:.3f} .. {hi:.3f}")
        out.append("kernel      planned  realised  mean_us  span_us  on XCD (w+c)%8  CUs   "
                   "mean time per XCD (XCC_ID register), relative")
        for k, v in kernels.items():
            m = v["mean_workgroup_us"]
            rel = " ".join(f"{(x / m - 1) * 100:+.1f}%" for x in v["xcd_mean_us"])
            out.append(f"{k:<10} {v['planned_imbalance'] * 100:7.2f}% "
                       f"{v['realized_imbalance_median'] * 100:8.2f}% {m:8.1f} "
                       f"{v['kernel_span_us_median']:8.1f}  "
                       f"{v['on_xcd_w_plus_c_mod_8'] * 100:5.1f}% "
                       f"(c={v['xcd_rotation_per_run'][0]})  {v['distinct_cus_per_run']:4d}   "
                       f"{rel}")
    dec = [(title, k, v["decomposition"]) for title, kernels in plans
           for k, v in kernels.items() if v.get("decomposition")]
    if dec:
        out += ["", "## what the realised spread is made of (forward and dQ)",
                "plan        kernel      realised  if XCD speeds matched  "
                "if queue residual matched too  queue residual rms / max"]
        for title, k, d in dec:
            tag = title.split(" (")[0].replace("plan for per-XCD speeds and cost scales",
                                                "calibrated").replace(
                "plan for per-XCD speeds", "per-XCD").replace("uniform plan", "uniform")
            real = next(v for t, kk in plans for kn, v in kk.items()
                        if t == title and kn == k)["realized_imbalance_median"]
            out.append(f"{tag:<11} {k:<10} {real * 100:8.2f}% "
                       f"{d['if_xcd_speeds_matched'] * 100:20.2f}% "
                       f"{d['if_queue_residual_matched_too'] * 100:29.2f}% "
                       f"{d['queue_residual_rms'] * 100:12.2f}% / {d['queue_residual_max'] * 100:.2f}%")
        out += ["(queue times divided by their XCD's mean time per unit of planned load in "
                "the same step,",
                "then by the per-queue factor that repeats in every step: what is left is "
                "step-to-step noise)"]
    out += ["", "planned = max/mean - 1 of the plan's workgroup loads (time units; in the "
            "per-XCD plan,",
            "each XCD's loads over its speed); realised = median over the steps of max/mean - 1 of "
            "the measured",
            "durations of the queues; span = last end - first start.",
            "on XCD (w+c)%8: share of queues v whose XCC_ID is (v + c) mod 8 for one rotation "
            "c per launch",
            "(c printed for the first step; in the per-XCD plan, queue v is planned for XCD "
            "v mod 8 and",
            "claimed there, so c = 0); CUs: distinct (XCD, SE, CU) triples per launch."]
    emit("\n".join(out) + "\n", a.out)


def cmd_sweep(a):
    r = _last_json(a.json)
    out = [f"# fwd+bwd throughput over {a.over} (bf16, 32 q-heads / 8 kv-heads, d 128, seed 1)",
           f"command: {a.command}",
           f"kernel_source_sha256: {kernel_source_hash()}", "",
           "context  draft_q  ms/step  TFLOP/s fwd+bwd  frac bf16  TFLOP/s fwd  fwd_ms  "
           "item imb  plan_ms"]
    for p in r["points"]:
        out.append(f"{p['context']:7d} {p['draft_queries']:8d} {p['ms_per_step']:8.3f} "
                   f"{p['tflops_fwd_bwd']:16.1f} {p['frac_of_bf16_peak']:10.3f} "
                   f"{p['tflops_fwd']:12.1f} {p['fwd_ms']:7.3f} "
                   f"{p['item_imbalance_256cu'] * 100:8.2f}% {p['plan_ms']:8.3f}")
    out += ["", "eager launches with one HIP event pair per kernel; the step is the forward "
            "partial, its",
            "split-tile merge and the backward; item imb = planned imbalance of the forward "
            "items (time units)."]
    emit("\n".join(out) + "\n", a.out)


def cmd_plans(a):
    r = _last_json(a.json)
    c = r["in_gpu_plan_comparison"]
    out = ["# in-GPU item plan: LPT with splitting against a contiguous equal-count plan of "
           "the same items",
           f"workload: {r['config']['workload']} (seed {r['config']['seed']})",
           f"command: {a.command}",
           f"kernel_source_sha256: {kernel_source_hash()}", "",
           "kernel     lpt_ms  contiguous_ms  gain"]
    for k in ("fwd_bf16", "bwd_dq"):
        out.append(f"{k:<9} {c[k]['lpt_ms']:7.3f} {c[k]['contiguous_ms']:14.3f} "
                   f"{c[k]['gain']:5.2f}x")
    out += ["", c["plan"] + "; items sorted by (kv head, query tile, first tile), one run per "
            "workgroup;", "both plans compute every item exactly once, only the queues differ."]
    emit("\n".join(out) + "\n", a.out)


def emit(text, out):
    if out:
        with open(out, "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("stats")
    k.add_argument("--command", required=True)
    k.add_argument("--trace", help="kernel trace CSV of the same run")
    k.add_argument("--skip-first", type=int, default=0)
    k.add_argument("--bench-json", help="bench.py output of the same run")
    k.add_argument("--out")
    t = sub.add_parser("traffic")
    t.add_argument("kernel")
    for opt in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--workload", "--command"):
        t.add_argument(opt, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--skip-first", type=int, default=0)
    t.add_argument("--out")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--workload", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--skip-first", type=int, default=0)
    c.add_argument("--out")
    l2 = sub.add_parser("l2")
    l2.add_argument("csv")
    l2.add_argument("--workload", required=True)
    l2.add_argument("--command", required=True)
    l2.add_argument("--skip-first", type=int, default=0)
    l2.add_argument("--out")
    for name in ("balance", "plans", "sweep"):
        b = sub.add_parser(name)
        b.add_argument("json")
        b.add_argument("--command", required=True)
        if name == "sweep":
            b.add_argument("--over", required=True, help="what the sweep varies, for the title")
        b.add_argument("--out")
    a = ap.parse_args(argv)
    {"kernels": cmd_kernels, "traffic": cmd_traffic, "counters": cmd_counters,
     "l2": cmd_l2, "balance": cmd_balance, "sweep": cmd_sweep, "plans": cmd_plans}[a.what](a)


if __name__ == "__main__":
    main()
