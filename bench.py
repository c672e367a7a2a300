#!/usr/bin/env python3
"""Benchmark of the Split-KV draft cross-attention hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input
already resident in HBM: forward partial attention with its in-library
merge of split query tiles, then the backward (rowsum(dO*O), dQ, dK/dV).
The schedule (chunk costs + LPT placement of work items on the persistent
workgroups) is built once per batch before the timed region, as the pages
describe the plan being built in advance; its host time is reported apart.

Workload: 32K-token context, 2048 draft queries (128 anchor blocks of 16,
anchors uniform in [8192, 32768)), GQA 32 query / 8 kv heads, d = 128,
bf16 N(0,1) inputs, KV chunks of 256, 256 CU bins.

FLOPs are realised-mask: every visible (query row, key) pair counts 4*d per
query head in the forward and 10*d in the backward (5 GEMMs), draft keys
included; masked-tile waste is not credited.

Prints ONE JSON line on stdout; progress goes to stderr.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
# unstamped steps run back to back before stamping the steps a plan is
# calibrated on (about 0.1 s of sustained load at 32K)
SUSTAIN_STEPS = 40

# System-level figures the Split-KV sources report for the whole method (the
# arXiv abstract of "Split-KV: Efficient Context Parallelism for Training
# Diffusion Drafters", and the rit.work blog post, section "Split-KV moves
# queries, not keys and values").  They name no hardware and no kernel
# figure: context for the records below, not targets.
PAGES_CONTEXT = {
    "note": "whole-method figures from the sources; hardware not stated; context, not targets",
    "weak_scaling_efficiency_cp64": "85-91 %",
    "speedup_over_fastest_cp_baseline": "up to 3.67x",
    "lpt_imbalance": "< 1 %",
    "planning_vs_dcp": "about three orders of magnitude faster",
    "step_gain_from_balancing_alone": "1.15-1.42x",
}
METRIC = "masked-attn TFLOP/s fwd & fwd+bwd, % of MFMA peak; LPT imbalance %"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def visible_elements(g, hq):
    """Visible (query row x head, key) pairs: context keys [lo, a) + 16 draft keys."""
    per_block = (g.anchors.astype(np.int64) - g.lo.astype(np.int64)) + 16
    return int(per_block.sum()) * 16 * hq


def shard_visible_elements(g, hq, chunk_ids, with_draft):
    """Visible pairs restricted to the keys of the given chunks (+ draft)."""
    a = g.anchors.astype(np.int64)[:, None]
    lo = g.lo.astype(np.int64)[:, None]
    cp = g.chunk_pos[chunk_ids].astype(np.int64)[None, :]
    ce = cp + g.chunk_len[chunk_ids].astype(np.int64)[None, :]
    keys = np.clip(np.minimum(a, ce) - np.maximum(lo, cp), 0, None).sum()
    return (int(keys) + (16 * len(g.anchors) if with_draft else 0)) * 16 * hq


def item_pair_loads(image, g, w):
    """Each workgroup's forward items counted in the chunk planner's unit,
    not the schedule's time units: the (anchor block, 64-key tile) pairs of
    the item's tiles that the block sees, plus one pair per anchor block of
    the query tile for its draft tile.  Returns the per-workgroup loads."""
    from block_sparse_split_amd.csrc_layout import H, I, T_WORDS, I_WORDS, QTILE, BLOCK
    h = {k: int(image[v]) for k, v in H.items()}
    tiles = image[h["OFF_TILES"]: h["OFF_TILES"] + h["NTILES"] * T_WORDS].reshape(-1, T_WORDS)
    items = image[h["OFF_ITEMS"]: h["OFF_ITEMS"] + h["NITEMS"] * I_WORDS].reshape(-1, I_WORDS)
    qoff = image[h["OFF_QOFF"]: h["OFF_QOFF"] + h["NWG"] + 1]
    queue = image[h["OFF_QUEUE"]: h["OFF_QUEUE"] + h["NITEMS"]]
    G = w.hq // w.hkv
    tpq = QTILE // G
    pos = tiles[:, 1].astype(np.int64)
    end = pos + tiles[:, 2]
    cum = {}
    pairs = np.zeros(len(items), np.int64)
    for i, it in enumerate(items):
        qt = int(it[I["QT"]])
        b0 = qt * tpq // BLOCK
        b1 = min(w.nb, -(-((qt + 1) * tpq) // BLOCK))
        if qt not in cum:
            a = g.anchors[b0:b1, None].astype(np.int64)
            lo = g.lo[b0:b1, None].astype(np.int64)
            seen = (np.maximum(lo, pos[None]) < np.minimum(a, end[None])).sum(0)
            cum[qt] = np.concatenate([[0], np.cumsum(seen)])
        pairs[i] = cum[qt][int(it[I["T1"]])] - cum[qt][int(it[I["T0"]])]
        if int(it[I["FLAGS"]]) & 1:
            pairs[i] += b1 - b0
    return np.array([pairs[queue[qoff[k]:qoff[k + 1]]].sum() for k in range(h["NWG"])])


def cpu_baseline(w, g, t, target_s=15.0):
    """The fp64 oracle (as it stands) on a bounded sample of anchor blocks,
    forward + backward, timed on this host's cores."""
    import oracle
    from block_sparse_split_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    scale = wl.softmax_scale(w.d)
    nb = len(g.anchors)
    pos = np.arange(g.ctx)

    def run(blocks):
        O = np.zeros((w.nq, w.hq, w.d))
        L = np.full((w.nq, w.hq), -np.inf)
        t0 = time.perf_counter()
        Ob, Lb = oracle.attention(t.Q, t.K, t.V, t.Kd, t.Vd, g.anchors, g.lo, scale,
                                  blocks=blocks)
        for k, b in enumerate(blocks):
            O[16 * b:16 * b + 16] = Ob[16 * k:16 * k + 16]
            L[16 * b:16 * b + 16] = Lb[16 * k:16 * k + 16]
        oracle.attention_bwd(t.Q, t.K, t.V, pos, g.anchors, g.lo, scale, O, t.dO, L, t.Kd,
                             t.Vd, blocks=blocks)
        return time.perf_counter() - t0

    probe = [nb // 2]
    t1 = run(probe)
    n = int(max(1, min(nb, target_s / max(t1, 1e-3))))
    blocks = sorted(set(np.linspace(0, nb - 1, n).astype(int).tolist()))
    dt = run(blocks)
    per_block = (g.anchors[blocks].astype(np.int64) - g.lo[blocks] + 16).sum() * 16 * w.hq
    flops = 14.0 * w.d * per_block
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 oracle forward+backward of {len(blocks)} of {nb} anchor blocks "
                      f"(all {w.hq} query heads), {dt:.1f} s wall"}


def traffic_for(kernel, workload, src_hash):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != src_hash:
        return None
    try:
        return float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def plan_imbalances(g, tile_k, bin_counts=(64, 256)):
    """Chunk-level balance of one workload: for each bin count, the
    max/mean - 1 of the bin loads under the library's LPT plan and under a
    contiguous equal-length split (chunk c to bin floor(c m / n)) of the same
    chunk costs."""
    from block_sparse_split_amd import splitkv as skv

    def imb(load):
        load = np.asarray(load, np.float64)
        return float(load.max() / load.mean() - 1.0) if load.mean() > 0 else 0.0

    out = {}
    for m in bin_counts:
        _, cost, load = skv.skv_plan_lpt(g.anchors, g.lo, g.chunk_pos, g.chunk_len, tile_k, m)
        cont = np.zeros(m, np.int64)
        np.add.at(cont, np.arange(len(cost), dtype=np.int64) * m // len(cost), cost)
        out[str(m)] = {"lpt": imb(load), "contiguous": imb(cont)}
    return out


def mfma_counters_for(kernel, workload, src_hash):
    """Matrix-core busy share, MFMA/VALU co-issue share and the settled
    clock of one kernel from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"mfma_util_{workload}.txt")
    if not os.path.exists(path):
        return None
    lines = open(path).read().splitlines()
    if f"kernel_source_sha256: {src_hash}" not in lines:
        return None
    for i, line in enumerate(lines):
        if line.startswith("kernel ") and "mfma_busy" in line:
            cols = line.split()
            for row in lines[i + 1:]:
                f = row.split()
                if f and f[0] == kernel:
                    rec = dict(zip(cols, f))
                    return {"mfma_busy": float(rec["mfma_busy"].rstrip("%")) / 100,
                            "mfma_valu_coexec": float(rec["coexec"].rstrip("%")) / 100,
                            "clock_ghz": float(rec["clock_GHz"])}
    return None


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_split_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def bench_tiny(args):
    """1K-context fp32 job: the forward partials of the 4 LPT shards (draft
    keys on shard 0), then their 4-way LSE merge.  A latency figure (us per
    step); value = TFLOP/s of the visible pairs over that time."""
    import torch
    from block_sparse_split_amd import splitkv as skv
    from block_sparse_split_amd import shards
    from block_sparse_split_amd import workloads as wl

    w, g, t = wl.make("tiny_f32_ctx1k", args.seed)
    ids, _, _, load = shards.lpt_shards(w, g, w.n_shards)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().float()
    Q, Kd, Vd = dev(t.Q), dev(t.Kd), dev(t.Vd)
    parts = []
    for r in range(w.n_shards):
        rows = shards.shard_rows(g, ids[r])
        parts.append((skv.Shard(shards.shard_problem(w, g, ids[r], r == 0)), dev(t.K[rows]),
                      dev(t.V[rows])))
    Op = torch.empty((w.n_shards, w.nq, w.hq, w.d), dtype=torch.float32, device="cuda")
    Lp = torch.empty((w.n_shards, w.nq, w.hq), dtype=torch.float32, device="cuda")
    Om = torch.empty((w.nq, w.hq, w.d), dtype=torch.float32, device="cuda")
    Lm = torch.empty((w.nq, w.hq), dtype=torch.float32, device="cuda")

    # the shards are independent (on a real job, different ranks): their
    # forwards run concurrently on streams of their own, then the merge
    side = [torch.cuda.Stream() for _ in parts]

    def step():
        main = torch.cuda.current_stream()
        start = torch.cuda.Event()
        start.record(main)
        done = []
        for r, (sh, K, V) in enumerate(parts):
            side[r].wait_event(start)
            kd, vd = (Kd, Vd) if r == 0 else (None, None)
            sh.fwd(Q, K, V, kd, vd, Op[r], Lp[r], side[r])
            ev = torch.cuda.Event()
            ev.record(side[r])
            done.append(ev)
        for ev in done:
            main.wait_event(ev)
        skv.skv_merge_lse(Op, Lp, Om, Lm)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    ref_O, ref_L = Om.clone(), Lm.clone()

    def timed(run):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    eager_ms = timed(step)
    # The job is a handful of small launches: the host's launch path bounds
    # it.  One HIP graph of the whole step removes that; every replay is
    # checked against the eager result before its time counts.
    graph_ms = None
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        ok = True
        for _ in range(3):
            Om.zero_()
            Lm.zero_()
            graph.replay()
            torch.cuda.synchronize()
            ok &= bool(torch.equal(Om, ref_O)) and bool(torch.equal(Lm, ref_L))
        if ok:
            graph_ms = timed(graph.replay)
        else:
            log("graph replay differs from the eager step; reporting eager time")
    except Exception as exc:  # capture not available: eager time only
        log(f"graph capture failed ({exc}); reporting eager time")
    ms = graph_ms if graph_ms is not None else eager_ms
    E = sum(shard_visible_elements(g, w.hq, ids[r], r == 0) for r in range(w.n_shards))
    flops = 4.0 * w.d * E
    value = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "us_per_step": ms * 1e3, "eager_us_per_step": eager_ms * 1e3,
        "timed_as": "hip graph replay" if graph_ms is not None else "eager launches",
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "context": g.ctx, "draft_queries": w.nq,
                   "anchor_blocks": w.nb, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.d,
                   "chunk": w.chunk, "shards": w.n_shards, "seed": args.seed,
                   "step": "4 shard forwards (fp32, concurrent streams) + 4-way merge"},
        "lpt": {"shard_imbalance_4": float(load.max() / load.mean() - 1)},
        "roofline": {"bound": "latency", "achieved": value, "peak": PEAK_F32_TFLOPS,
                     "unit": "TFLOP/s", "frac": value / PEAK_F32_TFLOPS, "kernel": "step",
                     "avg_ms": ms, "traffic": None},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_tiny(w, g, t, ids, flops),
        "context_from_pages": PAGES_CONTEXT,
    }
    return out


def cpu_baseline_tiny(w, g, t, ids, flops):
    """The fp64 oracle (as it stands) on the whole 1K-context job: the four
    shard partials and their merge."""
    import oracle
    from block_sparse_split_amd import shards
    from block_sparse_split_amd import workloads as wl
    scale = wl.softmax_scale(w.d)
    t0 = time.perf_counter()
    Os, Ls = [], []
    for r in range(w.n_shards):
        rows = shards.shard_rows(g, ids[r])
        O, L = oracle.attention_partial(t.Q, t.K[rows], t.V[rows], rows, g.anchors, g.lo, scale,
                                        t.Kd if r == 0 else None, t.Vd if r == 0 else None)
        Os.append(O)
        Ls.append(L)
    oracle.merge_lse(np.stack(Os), np.stack(Ls))
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"fp64 oracle, the whole job (4 partials + merge), {dt:.2f} s wall"}


def bench_merge64(args):
    """1M-context job: the forward partial of each of the 64 LPT shards (draft
    keys on shard 0) into one partial buffer, then the 64-way LSE merge.
    value = forward TFLOP/s over the 64 partials; the merge is reported in
    GB/s against HBM."""
    import torch
    from block_sparse_split_amd import splitkv as skv
    from block_sparse_split_amd import shards
    from block_sparse_split_amd import workloads as wl

    w, g, _ = wl.make("ctx1m_merge64", args.seed, tensors=False)
    w32 = wl.scaled(w, dtype="f32")
    ids, _, _, load = shards.lpt_shards(w, g, w.n_shards)
    t = wl.draw_tensors(w, g, args.seed, chunk_ids=[])
    dev = lambda x: torch.from_numpy(x).cuda().to(torch.bfloat16)
    Q, Kd, Vd = dev(t.Q), dev(t.Kd), dev(t.Vd)
    Op = torch.empty((w.n_shards, w.nq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    Lp = torch.empty((w.n_shards, w.nq, w.hq), dtype=torch.float32, device="cuda")
    Om = torch.empty((w.nq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    Lm = torch.empty((w.nq, w.hq), dtype=torch.float32, device="cuda")
    def run_shards(plan, label):
        """Forward partial of every shard of a plan into Op/Lp; per-shard ms."""
        times = []
        for r in range(w.n_shards):
            if r % 16 == 0:
                log(f"{label} shard {r}")
            sh = skv.Shard(shards.shard_problem(w, g, plan[r], r == 0))
            # K/V drawn in fp32, rounded to bf16 on the device (round to nearest even)
            K = dev(wl.draw_kv_chunks(w32, g, args.seed, plan[r], "K"))
            V = dev(wl.draw_kv_chunks(w32, g, args.seed, plan[r], "V"))
            kd, vd = (Kd, Vd) if r == 0 else (None, None)
            sh.fwd(Q, K, V, kd, vd, Op[r], Lp[r])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                sh.fwd(Q, K, V, kd, vd, Op[r], Lp[r])
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / args.steps)
            del K, V, sh
        return np.array(times)

    # simulated context-parallel step: every rank runs its share; the
    # slowest one sets the step time.  Contiguous equal-length split first,
    # then the LPT plan (whose partials stay in Op/Lp for the merge).
    n = len(g.chunk_pos)
    contiguous = [np.arange(r * n // w.n_shards, (r + 1) * n // w.n_shards)
                  for r in range(w.n_shards)]
    t_cont = run_shards(contiguous, "contiguous")
    t_lpt = run_shards(ids, "lpt")
    fwd_ms = float(t_lpt.sum())
    E = sum(shard_visible_elements(g, w.hq, ids[r], r == 0) for r in range(w.n_shards))
    for _ in range(args.warmup):
        skv.skv_merge_lse(Op, Lp, Om, Lm)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        skv.skv_merge_lse(Op, Lp, Om, Lm)
    e1.record()
    torch.cuda.synchronize()
    merge_ms = e0.elapsed_time(e1) / args.steps
    merge_bytes = Op.numel() * 2 + Lp.numel() * 4 + Om.numel() * 2 + Lm.numel() * 4
    flops = 4.0 * w.d * E
    ms = fwd_ms + merge_ms
    out = {
        "metric": METRIC, "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "context": g.ctx, "draft_queries": w.nq,
                   "anchor_blocks": w.nb, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.d,
                   "chunk": w.chunk, "shards": w.n_shards, "seed": args.seed,
                   "step": "64 shard forwards + 64-way merge"},
        "fwd_ms_all_shards": fwd_ms,
        "fwd_tflops": flops / (fwd_ms * 1e-3) / 1e12,
        "merge_ms": merge_ms,
        "merge_gbs": merge_bytes / (merge_ms * 1e-3) / 1e9,
        "merge_frac_of_hbm_peak": merge_bytes / (merge_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "lpt": {"shard_imbalance_64": float(load.max() / load.mean() - 1),
                "chunk_imbalance_by_bins": plan_imbalances(g, w.tile_k)},
        "simulated_cp_step": {
            "ranks": w.n_shards,
            "lpt_max_ms": float(t_lpt.max()), "lpt_mean_ms": float(t_lpt.mean()),
            "contiguous_max_ms": float(t_cont.max()), "contiguous_mean_ms": float(t_cont.mean()),
            "step_gain_from_balancing": float(t_cont.max() / t_lpt.max())},
        "roofline": {"bound": "hbm", "achieved": merge_bytes / (merge_ms * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": merge_bytes / (merge_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "kernel": "merge", "avg_ms": merge_ms, "traffic": None},
        "cpu_baseline": None,
        "context_from_pages": PAGES_CONTEXT,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ctx32k_q2k")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", choices=("context", "budget"),
                    help="throughput over context length (2K-32K at 2048 draft queries) or over "
                         "the draft-query budget (512-4096 at 32K context), fwd+bwd")
    ap.add_argument("--compare-plans", action="store_true",
                    help="also time the forward and dQ kernels with a contiguous (cost-blind) "
                         "item plan of the same items")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time the forward alone (diagnostic; not the benchmark step)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain elementwise copy of this many "
                         "MiB (read once, written once) three times; used to calibrate HBM "
                         "byte counters")
    ap.add_argument("--wg-times", action="store_true",
                    help="instead of the benchmark: per-workgroup start/end stamps of the "
                         "forward, dQ and dK/dV kernels over --steps steps; realised against "
                         "planned imbalance")
    ap.add_argument("--uniform-plan", action="store_true",
                    help="plan the in-GPU work without per-XCD speeds (by default the bench "
                         "measures each XCD's speed on the uniform plan and times the plan "
                         "made for them)")
    ap.add_argument("--no-subrecords", action="store_true",
                    help="with the default workload, skip the sub-records of the varlen, "
                         "512K rank-share and 1M merge workloads")
    ap.add_argument("--plan-sweep", action="store_true",
                    help="host only: time the chunk-level LPT plan (costs + placement) for "
                         "1K-4M chunks of 256 keys on 64 and 256 bins")
    args = ap.parse_args()
    if args.plan_sweep:
        return plan_sweep()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_split_amd import splitkv as skv
    from block_sparse_split_amd import shards
    from block_sparse_split_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                          "launches": 3}), flush=True)
        return
    skv.lib()  # fail loudly if the HIP library is not built

    if args.workload == "ctx1m_merge64":
        return bench_merge64(args)
    if args.workload == "tiny_f32_ctx1k":
        print(json.dumps(bench_tiny(args)), flush=True)
        return
    if args.sweep:
        return run_sweep(args)
    if args.wg_times:
        return wg_balance(args)
    rec = run_workload(args, args.workload)
    if args.workload == "ctx32k_q2k" and not args.fwd_only and not args.no_subrecords:
        rec["other_configs"] = other_configs(args)
    print(json.dumps(rec), flush=True)


def _summary(r):
    """The figures of a workload record that a sub-record keeps."""
    keep = ("value", "unit", "ms_per_step", "frac_of_bf16_peak", "fwd_tflops",
            "fwd_frac_of_bf16_peak", "fwd_ms", "algorithmic_tflop_per_step", "config", "lpt",
            "roofline", "hip_graph")
    out = {k: r[k] for k in keep if k in r}
    out["kernels_avg_ms"] = {k: v["avg_ms"] for k, v in r["kernels"].items()}
    return out


def other_configs(args):
    """Sub-records for the other workloads, timed in the same run: the tiny
    fp32 job (4 shard forwards and their merge, seed 0), the varlen fwd+bwd
    job, the 512K-context rank-0 share (forward) and the 64-way merge of the
    1M-context job (the merge alone, on N(0,1) bf16 partials and N(0, 4)
    LSEs drawn on the device, seeded)."""
    import argparse as _ap
    import torch
    from block_sparse_split_amd import splitkv as skv
    from block_sparse_split_amd import workloads as wl
    sub = _ap.Namespace(**vars(args))
    sub.steps = max(3, args.steps // 2)
    sub.no_cpu_baseline = True
    sub.compare_plans = False
    out = {}
    sub.seed = 0
    log("sub-record tiny_f32_ctx1k")
    r = bench_tiny(sub)
    out["tiny_f32_ctx1k"] = {k: r[k] for k in ("value", "unit", "ms_per_step", "us_per_step",
                                               "eager_us_per_step", "timed_as", "dtype", "config",
                                               "lpt")}
    for name, seed in (("varlen8_fwdbwd", 3), ("cp64_rank0_ctx512k", 2)):
        sub.seed = seed
        sub.fwd_only = False
        log(f"sub-record {name}")
        out[name] = _summary(run_workload(sub, name))
        torch.cuda.empty_cache()
    w, g, _ = wl.make("ctx1m_merge64", 4, tensors=False)
    log("sub-record ctx1m_merge64 (64-way merge)")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    Op = torch.randn((w.n_shards, w.nq, w.hq, w.d), device="cuda", generator=gen,
                     dtype=torch.bfloat16)
    Lp = 2.0 * torch.randn((w.n_shards, w.nq, w.hq), device="cuda", generator=gen)
    Om = torch.empty((w.nq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    Lm = torch.empty((w.nq, w.hq), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        skv.skv_merge_lse(Op, Lp, Om, Lm)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(sub.steps):
        skv.skv_merge_lse(Op, Lp, Om, Lm)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / sub.steps
    nbytes = Op.numel() * 2 + Lp.numel() * 4 + Om.numel() * 2 + Lm.numel() * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    from block_sparse_split_amd import shards
    _, _, _, load = shards.lpt_shards(w, g, w.n_shards)
    out["ctx1m_merge64"] = {"step": "64-way LSE merge", "partials": w.n_shards,
                            "rows": w.nq * w.hq, "head_dim": w.d, "ms": ms,
                            "algorithmic_bytes": nbytes, "gbs": gbs,
                            "frac_of_hbm_peak": gbs / PEAK_HBM_GBS, "launches": sub.steps,
                            "lpt": {"shard_imbalance_64": float(load.max() / load.mean() - 1),
                                    "chunk_imbalance_by_bins": plan_imbalances(g, w.tile_k)}}
    del Op, Lp, Om, Lm
    torch.cuda.empty_cache()
    return out


def run_workload(args, workload):
    """One workload (a name or a Workload): plan, time `steps` steps, and
    return the JSON record."""
    import torch
    from block_sparse_split_amd import splitkv as skv
    from block_sparse_split_amd import shards
    from block_sparse_split_amd import workloads as wl

    w, g, _ = wl.make(workload, args.seed, tensors=False)
    # the 512K workload is one rank's share of a 64-way LPT split: its chunks
    # (no draft keys) against all queries, forward only
    rank_share = w.n_shards > 1
    rank_load = None
    if rank_share:
        ids_all, _, _, rank_load = shards.lpt_shards(w, g, w.n_shards)
        chunk_ids = ids_all[0]
    else:
        chunk_ids = None
    t = wl.draw_tensors(w, g, args.seed, with_grad=True, chunk_ids=chunk_ids)
    if rank_share:
        args.fwd_only = True
    log(f"workload {w.name}: ctx {g.ctx}, nb {w.nb}, hq {w.hq}, hkv {w.hkv}, d {w.d}"
        + (f", rank 0 of {w.n_shards}: {len(chunk_ids)} chunks" if rank_share else ""))
    prob = (shards.shard_problem(w, g, chunk_ids, False) if rank_share
            else shards.whole_context_problem(w, g))
    plan_times = []
    for _ in range(5):
        t0 = time.perf_counter()
        image, info = skv.skv_schedule_build(prob, 0)
        plan_times.append(time.perf_counter() - t0)
    sh = skv.Shard(prob)
    n_wg = sh.info.n_workgroups
    chunk_bins, chunk_cost, chunk_load = skv.skv_plan_lpt(g.anchors, g.lo, g.chunk_pos,
                                                          g.chunk_len, w.tile_k, n_wg)
    dev = "cuda"
    to = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
    Q, K, V, Kd, Vd, dO = (to(x) for x in (t.Q, t.K, t.V, t.Kd, t.Vd, t.dO))
    O = torch.empty((w.nq, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((w.nq, w.hq), dtype=torch.float32, device=dev)
    dQ = torch.empty((w.nq, w.hq, w.d), dtype=torch.float32, device=dev)
    dK = torch.empty_like(K)
    dV = torch.empty_like(V)
    dKd = torch.empty_like(Kd)
    dVd = torch.empty_like(Vd)
    stream = torch.cuda.current_stream()

    def step(s=stream):
        sh.fwd(Q, K, V, Kd, Vd, O, LSE, s)
        if not args.fwd_only:
            sh.bwd(Q, K, V, Kd, Vd, O, dO, LSE, dQ, dK, dV, dKd, dVd, skv.SKV_BF16, s)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    xcd = None
    # (--compare-plans reorders the uniform plan's queues: it keeps that plan)
    if not args.uniform_plan and not args.compare_plans and n_wg % 8 == 0:
        # per-XCD speeds and measured cost scales from stamps of the uniform
        # plan, a plan made for them, then a refit over the stamps of both
        # plans and the plan the step below uses (all outside the timed
        # region)
        runs = stamp_runs(step, n_wg, 6, torch, SUSTAIN_STEPS)
        uni_realized = {k: v["realized_imbalance_median"] for k, v in
                        realized_balance(step, sh.info, 0, torch, args.fwd_only,
                                         runs=runs).items()}
        data = [(sh.image, runs, None)]
        for rnd in range(2):
            speed, scale = calibrate(data, args.fwd_only)
            sh = skv.Shard(prob, n_workgroups=n_wg, xcd_speed=speed, cost_scale=scale)
            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            if rnd == 0:
                data.append((sh.image, stamp_runs(step, n_wg, 6, torch, SUSTAIN_STEPS), scale))
        xcd = {"speed": np.round(speed, 4).tolist(),
               "cost_scale_range": [[round(float(x.min()), 4), round(float(x.max()), 4)]
                                    for x in scale],
               "calibration": f"two rounds of 6 stamped steps after {SUSTAIN_STEPS} unstamped "
                              "ones, back to back (uniform plan, then the first calibrated "
                              "plan)",
               "uniform_plan_realized": uni_realized}
    skv.skv_timing_collect()  # discard anything recorded before
    skv.skv_timing_enable(True)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    skv.skv_timing_enable(False)
    kernels = skv.skv_timing_collect()
    ms = start.elapsed_time(stop) / args.steps
    log(f"{ms:.3f} ms/step")
    graph = graph_step(step, (O, LSE) if args.fwd_only else (O, LSE, dQ, dK, dV, dKd, dVd),
                       args, torch)

    E = (shard_visible_elements(g, w.hq, chunk_ids, False) if rank_share
         else visible_elements(g, w.hq))
    fwd_flops = 4.0 * w.d * E
    bwd_flops = 10.0 * w.d * E
    step_flops = fwd_flops + (0 if args.fwd_only else bwd_flops)
    algo = {"fwd_bf16": ("mfma", fwd_flops), "bwd_dkdv": ("mfma", 8.0 * w.d * E),
            "bwd_dq": ("mfma", 2.0 * w.d * E)}
    per_kernel = {}
    for name, (cnt, tot) in kernels.items():
        per_kernel[name] = {"launches": cnt, "avg_ms": tot / cnt,
                            "share_of_step": (tot / args.steps) / ms}
        if name in algo:
            per_kernel[name]["tflops"] = algo[name][1] / (tot / cnt * 1e-3) / 1e12
    dom = max(kernels, key=lambda k: kernels[k][1])
    cnt, tot = kernels[dom]
    avg_s = tot / cnt * 1e-3
    if dom in algo:
        achieved = algo[dom][1] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": None}
    roof["kernel"] = dom
    roof["avg_ms"] = avg_s * 1e3
    roof["traffic"] = traffic_for(dom, w.name, kernel_source_hash())
    roof["counters"] = mfma_counters_for(dom, w.name, kernel_source_hash())

    realized = realized_balance(step, sh.info, 5, torch, args.fwd_only, image=sh.image,
                                plan_speed=None if xcd is None else speed)
    pair_loads = item_pair_loads(sh.image, g, w)
    fwd_ms = sum(kernels[k][1] for k in ("fwd_bf16", "merge_split") if k in kernels) / args.steps
    # the headline step time: the HIP-graph replay of the same step (no
    # per-kernel events, no host launch gaps) when capture works and every
    # checked replay is bit-equal to the eager step; else the eager time
    eager_ms = ms
    if graph is not None:
        ms = graph
    value = step_flops / (ms * 1e-3) / 1e12
    item_imb = sh.info.item_cost_max_bin / (sh.info.item_cost_total / n_wg) - 1
    kv_imb = sh.info.kv_cost_max_bin / (sh.info.kv_cost_total / n_wg) - 1
    chunk_imb = float(chunk_load.max() / chunk_load.mean() - 1)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "context": g.ctx, "draft_queries": w.nq,
                   "anchor_blocks": w.nb, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.d,
                   "chunk": w.chunk, "seed": args.seed,
                   "step": "fwd" if args.fwd_only else "fwd+bwd"},
        "frac_of_bf16_peak": value / PEAK_BF16_TFLOPS,
        "fwd_tflops": fwd_flops / (fwd_ms * 1e-3) / 1e12,
        "fwd_frac_of_bf16_peak": fwd_flops / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "fwd_ms": fwd_ms,
        "algorithmic_tflop_per_step": step_flops / 1e12,
        "timed_as": ("hip graph replay of the step (replays checked bit-equal to the eager "
                     "step); per-kernel times from the eager pass" if graph is not None else
                     "eager launches, one HIP event pair around each kernel"),
        "eager_ms_per_step": eager_ms,
        "eager_tflops": step_flops / (eager_ms * 1e-3) / 1e12,
        "hip_graph": (None if graph is None else
                      {"ms_per_step": graph, "tflops": step_flops / (graph * 1e-3) / 1e12,
                       "replays_checked": "bit-equal to the eager step"}),
        "lpt": {"work_items": sh.info.n_items, "item_imbalance_256cu": item_imb,
                "item_cost_unit": "time units fitted to measured workgroup times",
                "item_pair_imbalance_256cu": float(pair_loads.max() / pair_loads.mean() - 1),
                "kv_items": sh.info.n_kv_items, "kv_item_imbalance_256cu": kv_imb,
                "chunk_imbalance_256bins": chunk_imb, "plan_ms": 1e3 * float(np.median(plan_times)),
                "workgroups": n_wg,
                "plan": ("per-XCD speeds and per-(kv head, query tile group) cost scales "
                         "fitted to clock stamps (skv_schedule_build_xcd)" if xcd
                         else "uniform (skv_schedule_build)"),
                "xcd": xcd,
                "realized": {k: {"imbalance_median": v["realized_imbalance_median"],
                                 "on_xcd_w_plus_c_mod_8": v["on_xcd_w_plus_c_mod_8"],
                                 "xcd_rotation_per_run": v["xcd_rotation_per_run"],
                                 "distinct_cus": v["distinct_cus_per_run"],
                                 "xcd_mean_us": v["xcd_mean_us"],
                                 "decomposition": v.get("decomposition")}
                             for k, v in realized.items()}},
        "kernels": per_kernel,
        "roofline": roof,
        "cpu_baseline": None,
        "context_from_pages": PAGES_CONTEXT,
    }
    if rank_share:
        out["config"]["rank"] = f"0 of {w.n_shards} (LPT), {len(chunk_ids)} chunks"
        out["lpt"]["rank_imbalance"] = float(rank_load.max() / rank_load.mean() - 1)
    if args.compare_plans and not rank_share:
        out["in_gpu_plan_comparison"] = compare_item_plans(sh, step, kernels, args, torch)
    if not args.no_cpu_baseline and not rank_share:
        log("timing the fp64 oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(w, g, t)
    return out


def graph_step(step, outs, args, torch):
    """The same step captured once in a HIP graph and replayed: the time of
    `steps` replays without per-kernel events or host launch gaps.  Every
    output is cleared before each of three checked replays and must come back
    bit-equal to the eager step's (the kernels are deterministic); None when
    capture fails or a replay differs."""
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]
    try:
        side = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                step(side)
        torch.cuda.synchronize()
        for _ in range(3):
            for x in outs:
                x.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(x, r) for x, r in zip(outs, ref)):
                log("graph replay differs from the eager step")
                return None
        for _ in range(args.warmup):
            graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
    except RuntimeError as exc:
        log(f"graph capture failed ({exc})")
        return None
    ms = e0.elapsed_time(e1) / args.steps
    log(f"{ms:.3f} ms/step as one HIP graph")
    return ms


def compare_item_plans(sh, step, kernels_lpt, args, torch):
    """Kernel times with the library's LPT item plan against a contiguous
    plan of the same items: items sorted by (kv head, query tile, first
    tile) and cut into equal-count runs, one per workgroup (no cost model).
    Both plans compute every item exactly once; only the queues differ."""
    from block_sparse_split_amd import splitkv as skv
    from block_sparse_split_amd.csrc_layout import H
    img = sh.image.copy()
    n_items, n_wg = int(img[H["NITEMS"]]), int(img[H["NWG"]])
    off_items, off_qoff, off_queue = (int(img[H["OFF_ITEMS"]]), int(img[H["OFF_QOFF"]]),
                                      int(img[H["OFF_QUEUE"]]))
    # the comparison reorders the forward's queues, which dQ shares in a
    # plan made without per-XCD speeds
    assert int(img[H["OFF_DQ_QUEUE"]]) == off_queue
    items = img[off_items:off_items + 8 * n_items].reshape(n_items, 8)
    order = np.lexsort((items[:, 2], items[:, 1], items[:, 0])).astype(np.int32)
    img[off_queue:off_queue + n_items] = order
    img[off_qoff:off_qoff + n_wg + 1] = np.linspace(0, n_items, n_wg + 1).astype(np.int32)
    lpt_sched = sh.schedule
    sh.schedule = torch.from_numpy(img).to(lpt_sched.device)
    try:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        skv.skv_timing_collect()
        skv.skv_timing_enable(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        skv.skv_timing_enable(False)
        kernels_cont = skv.skv_timing_collect()
    finally:
        sh.schedule = lpt_sched
    res = {"plan": "contiguous equal-count runs of the same items"}
    for name in ("fwd_bf16", "bwd_dq"):
        if name in kernels_lpt and name in kernels_cont:
            a = kernels_lpt[name][1] / kernels_lpt[name][0]
            b = kernels_cont[name][1] / kernels_cont[name][0]
            res[name] = {"lpt_ms": a, "contiguous_ms": b, "gain": b / a}
    log("in-GPU item plan, LPT vs contiguous: " + ", ".join(
        f"{k} {v['lpt_ms']:.3f} vs {v['contiguous_ms']:.3f} ms" for k, v in res.items() if k != "plan"))
    return res




SWEEPS = {
    # fixed draft-query budget (2048 queries), context 2K -> 32K; anchors
    # uniform on [L/4, L) as in the 32K workload
    "context": [dict(ctx=L, anchor_lo=L // 4, anchor_hi=L) for L in (2048, 4096, 8192, 16384, 32768)],
    # fixed 32K context, draft-query budget 512 -> 4096
    "budget": [dict(blocks_per_seq=nb) for nb in (32, 64, 128, 256)],
}


def spread_decomposition(dur, xcc, load, plan_speed=None):
    """What the realised spread of one kernel is made of, from its stamped
    runs (dur, xcc: [runs, n_wg]) and the plan's queue loads (load: [n_wg];
    queue v planned at plan_speed[v % 8], 1 without one): the spread left
    if each XCD's mean speed were what the plan assumed (queue times
    divided by their XCD's mean ratio of measured to planned time in the
    same run), then if the per-queue residual that repeats in every run
    (the cost model's error on that queue's items) were matched too; what
    is still left then is step-to-step noise.  Queues without load are
    left out."""
    ok = load > 0
    sp = np.ones(8) if plan_speed is None else np.asarray(plan_speed, np.float64)
    planned = load.astype(np.float64) / sp[np.arange(len(load)) % 8]
    d, x, ld = dur[:, ok], xcc[:, ok], planned[ok]
    ratio = d / ld[None, :]
    fac = np.ones_like(ratio)
    for r in range(len(d)):
        for c in range(8):
            m = x[r] == c
            if m.any():
                fac[r, m] = ratio[r, m].mean()
    q = ratio / fac                        # per queue, XCD speed removed
    stable = q.mean(0) / q.mean()          # the part that repeats every run
    no_xcd = d / fac
    no_model = no_xcd / stable[None, :]
    med = lambda a: float(np.median(a.max(1) / a.mean(1) - 1))
    return {"if_xcd_speeds_matched": med(no_xcd),
            "if_queue_residual_matched_too": med(no_model),
            "queue_residual_rms": float(np.sqrt(np.mean((stable - 1) ** 2))),
            "queue_residual_max": float(stable.max() - 1)}


def balance_stats(runs, planned, names=("fwd_bf16", "bwd_dq", "bwd_dkdv"), loads=None,
                  plan_speed=None):
    """Per kernel (forward, dQ, dK/dV = index 0, 1, 2 of each run's
    [3, n_wg, 4] array of (start, end, XCC_ID, HW_ID) words, stamps in
    100 MHz ticks): workgroup durations in us, max/mean - 1 per run and its
    median, the span from the first start to the last end, the mean
    duration per XCD as the XCC_ID register reports it, the share of
    workgroups w that ran on XCD w mod 8 and on XCD (w + c) mod 8 for the
    best single rotation c of each run (the plan only needs workgroups
    w = w' mod 8 to share an XCD), and the number of distinct compute units
    (XCD, SE, CU) used.  With the plan's queue loads, the forward and dQ
    also get spread_decomposition (dK/dV workgroups take items of other
    queues at run time, so their times are not their queues')."""
    out = {}
    n = runs[0].shape[1]
    for k, name in enumerate(("fwd_bf16", "bwd_dq", "bwd_dkdv")):
        if name not in names:
            continue
        dur = np.stack([r[k, :, 1] - r[k, :, 0] for r in runs]).astype(np.float64) / 100.0
        span = np.array([r[k, :, 1].max() - r[k, :, 0].min() for r in runs]) / 100.0
        imb = dur.max(1) / dur.mean(1) - 1
        xcc = np.stack([r[k, :, 2] & 15 for r in runs])
        hw = np.stack([r[k, :, 3] for r in runs])
        cu = (xcc << 8) | (((hw >> 13) & 7) << 4) | ((hw >> 8) & 15)
        xcd_mean = [float(dur[xcc == x].mean()) if np.any(xcc == x) else None for x in range(8)]
        out[name] = {"planned_imbalance": planned[name],
                     "realized_imbalance_median": float(np.median(imb)),
                     "realized_imbalance_runs": [float(x) for x in imb],
                     "mean_workgroup_us": float(dur.mean()),
                     "kernel_span_us_median": float(np.median(span)),
                     "xcd_mean_us": xcd_mean,
                     "on_xcd_w_mod_8": float(np.mean(xcc == (np.arange(n) % 8)[None, :])),
                     # the dispatcher's round robin may start a launch on any
                     # XCD: workgroup w on XCD (w + c) mod 8 for one c per run
                     "xcd_rotation_per_run": [int(np.bincount(o, minlength=8).argmax())
                                              for o in (xcc - np.arange(n)[None, :]) % 8],
                     "on_xcd_w_plus_c_mod_8": float(np.mean([
                         np.bincount(o, minlength=8).max() / n
                         for o in (xcc - np.arange(n)[None, :]) % 8])),
                     "distinct_cus_per_run": int(np.median([len(np.unique(c)) for c in cu]))}
        if loads is not None and k < 2 and len(runs) > 1:
            out[name]["decomposition"] = spread_decomposition(
                dur, xcc, np.asarray(loads[k]), None if plan_speed is None else plan_speed[k])
    return out


def stamp_runs(step, n, steps, torch, sustain=0):
    """Per-workgroup stamps of `steps` steps (outside any timed region): a
    list of [3, n, 4] arrays (forward, dQ, dK/dV).  The steps run back to
    back like the timed ones (each launch writes its own buffer; one
    synchronisation at the end), after `sustain` unstamped steps that bring
    the GPU to the clocks and temperatures of a sustained run: the per-XCD
    speeds differ between a GPU that idles between steps and one that does
    not."""
    from block_sparse_split_amd import splitkv as skv
    clk = torch.zeros((steps, 3 * n * 4), dtype=torch.int64, device="cuda")
    for _ in range(sustain):
        step()
    try:
        for i in range(steps):
            skv.skv_timing_wg_clock(clk[i])
            step()
    finally:
        skv.skv_timing_wg_clock(None)
    torch.cuda.synchronize()
    host = clk.cpu().numpy()
    return [host[i].reshape(3, n, 4).copy() for i in range(steps)]


def planned_imbalance(info):
    n = info.n_workgroups
    return {"fwd_bf16": info.item_cost_max_bin / (info.item_cost_total / n) - 1,
            "bwd_dq": info.dq_cost_max_bin / (info.dq_cost_total / n) - 1,
            "bwd_dkdv": info.kv_cost_max_bin / (info.kv_cost_total / n) - 1}


def realized_balance(step, info, steps, torch, fwd_only=False, runs=None, image=None,
                     plan_speed=None):
    """Stamp every workgroup for `steps` steps (or take `runs`) and return
    balance_stats for the forward, dQ and dK/dV kernels (the forward only
    with fwd_only); with the schedule image (and the per-XCD speeds it was
    planned at, if any), the spread decomposition too."""
    from block_sparse_split_amd import splitkv as skv
    if runs is None:
        runs = stamp_runs(step, info.n_workgroups, steps, torch)
    loads = skv.queue_loads(image) if image is not None else None
    return balance_stats(runs, planned_imbalance(info), ("fwd_bf16",) if fwd_only else
                         ("fwd_bf16", "bwd_dq", "bwd_dkdv"), loads, plan_speed)


def calibrate(data, fwd_only):
    """Per-XCD speeds and cost scales fitted to stamped runs of one or more
    plans (skv.calibrate_from_stamps); a forward-only run gives dQ the
    forward's and dK/dV equal speeds."""
    from block_sparse_split_amd import splitkv as skv
    sp, sc = skv.calibrate_from_stamps(data)
    if fwd_only:
        sp[1], sc[1] = sp[0], sc[0]
        sp[2] = 1.0
    return sp, sc


def wg_balance(args):
    """Realised balance of the in-GPU plan: every workgroup of the forward,
    dQ and dK/dV kernels stamps its start and end (100 MHz clock); per
    kernel and step, max(duration) / mean(duration) - 1 against the plan's
    max(load) / mean(load) - 1, and the mean duration per XCD (workgroup
    w runs on XCD w mod 8)."""
    import torch
    from block_sparse_split_amd import splitkv as skv
    from block_sparse_split_amd import shards
    from block_sparse_split_amd import workloads as wl
    w, g, t = wl.make(args.workload, args.seed, with_grad=True)
    sh = skv.Shard(shards.whole_context_problem(w, g))
    n = sh.info.n_workgroups
    to = lambda x: torch.from_numpy(x).cuda().to(torch.bfloat16)
    Q, K, V, Kd, Vd, dO = (to(x) for x in (t.Q, t.K, t.V, t.Kd, t.Vd, t.dO))
    O = torch.empty((w.nq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    LSE = torch.empty((w.nq, w.hq), device="cuda")
    dQ = torch.empty((w.nq, w.hq, w.d), device="cuda")
    dK, dV, dKd, dVd = (torch.empty_like(x) for x in (K, V, Kd, Vd))

    def step():
        sh.fwd(Q, K, V, Kd, Vd, O, LSE)
        sh.bwd(Q, K, V, Kd, Vd, O, dO, LSE, dQ, dK, dV, dKd, dVd, skv.SKV_BF16)

    for _ in range(max(1, args.warmup)):
        step()
    prob = shards.whole_context_problem(w, g)
    runs = stamp_runs(step, n, args.steps, torch, SUSTAIN_STEPS)
    plans = {"uniform": realized_balance(step, sh.info, 0, torch, runs=runs, image=sh.image)}
    data = [(sh.image, runs, None)]
    speed, scale = calibrate(data, False)
    if n % 8 == 0:
        # the same steps with the plan made for the XCD speeds just measured
        # (no cost scales), then with speeds and cost scales fitted to the
        # uniform plan's stamps and, in a second round, to those of the first
        # calibrated plan as well
        sh = skv.Shard(prob, n_workgroups=n, xcd_speed=speed)
        plans["xcd"] = realized_balance(step, sh.info, 0, torch, runs=stamp_runs(
            step, n, args.steps, torch, SUSTAIN_STEPS), image=sh.image, plan_speed=speed)
        for rnd in range(2):
            speed, scale = calibrate(data, False)
            sh = skv.Shard(prob, n_workgroups=n, xcd_speed=speed, cost_scale=scale)
            runs = stamp_runs(step, n, args.steps, torch, SUSTAIN_STEPS)
            data.append((sh.image, runs, scale))
        plans["calibrated"] = realized_balance(step, sh.info, 0, torch, runs=runs,
                                               image=sh.image, plan_speed=speed)
    for plan, out in plans.items():
        for name, v in out.items():
            log(f"{plan} {name}: planned {v['planned_imbalance'] * 100:.2f} %, realised "
                f"{v['realized_imbalance_median'] * 100:.2f} % (median of {args.steps}), "
                f"mean {v['mean_workgroup_us']:.1f} us")
    print(json.dumps({"metric": "workgroup_balance", "workload": w.name, "workgroups": n,
                      "clock": "s_memrealtime, 100 MHz", "steps": args.steps,
                      "xcd_speed": np.round(speed, 4).tolist(),
                      "cost_scale_range": [[round(float(x.min()), 4), round(float(x.max()), 4)]
                                           for x in scale],
                      "kernels": plans["uniform"], "kernels_xcd_plan": plans.get("xcd"),
                      "kernels_calibrated_plan": plans.get("calibrated")}),
          flush=True)


def plan_sweep():
    """Host time of `skv_plan_lpt` (realised tile costs of every chunk, then
    LPT) against the chunk count: chunks of 256 keys, 512 anchor blocks
    uniform on [L/4, L), tile 64; one JSON line."""
    from block_sparse_split_amd import splitkv as skv
    rng = np.random.default_rng(1)
    points = []
    for n in (1024, 4096, 16384, 65536, 262144, 1048576, 4194304):
        ctx = min(n * 256, (1 << 31) - 256)
        n = ctx // 256
        nb = 512
        a = np.sort(rng.choice(np.arange(ctx // 4, ctx), nb, replace=False)).astype(np.int32)
        lo = np.zeros(nb, np.int32)
        pos = (np.arange(n, dtype=np.int64) * 256).astype(np.int32)
        ln = np.full(n, 256, np.int32)
        for m in (64, 256):
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                _, _, load = skv.skv_plan_lpt(a, lo, pos, ln, 64, m)
                ts.append(time.perf_counter() - t0)
            points.append({"chunks": n, "bins": m, "plan_ms": 1e3 * float(np.median(ts)),
                           "imbalance": float(load.max() / load.mean() - 1)})
            log(f"plan: {n} chunks on {m} bins: {points[-1]['plan_ms']:.2f} ms, "
                f"imbalance {points[-1]['imbalance']:.2e}")
    print(json.dumps({"metric": "lpt_plan_time", "unit": "ms", "host_threads": 1,
                      "points": points}), flush=True)


def run_sweep(args):
    """Throughput over context length at a fixed query budget, or over the
    query budget at a fixed context (the regime the pages study: a short
    draft-query set against a long context)."""
    from block_sparse_split_amd import workloads as wl
    base = wl.WORKLOADS["ctx32k_q2k"]
    points = []
    for over in SWEEPS[args.sweep]:
        w = wl.scaled(base, name=f"sweep_{args.sweep}", **over)
        args.no_cpu_baseline = True
        r = run_workload(args, w)
        points.append({"context": r["config"]["context"], "draft_queries": r["config"]["draft_queries"],
                       "ms_per_step": r["ms_per_step"], "tflops_fwd_bwd": r["value"],
                       "tflops_fwd": r["fwd_tflops"], "fwd_ms": r["fwd_ms"],
                       "frac_of_bf16_peak": r["frac_of_bf16_peak"],
                       "item_imbalance_256cu": r["lpt"]["item_imbalance_256cu"],
                       "plan_ms": r["lpt"]["plan_ms"]})
        log(f"sweep {args.sweep}: ctx {points[-1]['context']}, queries {points[-1]['draft_queries']}: "
            f"{points[-1]['ms_per_step']:.3f} ms, {points[-1]['tflops_fwd_bwd']:.0f} TFLOP/s")
    last = points[-1]
    print(json.dumps({"metric": METRIC, "value": last["tflops_fwd_bwd"], "unit": "TFLOP/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                      "sweep": args.sweep, "points": points}), flush=True)


if __name__ == "__main__":
    main()
