"""Host-side figures of bench.py checked against the oracle's planner (no
GPU): the chunk-level LPT and contiguous-split imbalances reported for the
1M-context job follow the oracle's independent LPT scan and contiguous split
exactly."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_sparse_split_amd import workloads as wl  # noqa: E402
from oracle import planner  # noqa: E402


@pytest.mark.parametrize("name,scale", [
    ("tiny_f32_ctx1k", None),
    # the 1M-context job's anchor and chunk structure at 1/16 of its length
    ("ctx1m_merge64", dict(ctx=65536, anchor_lo=16384, anchor_hi=65536, blocks_per_seq=64)),
])
def test_plan_imbalances_match_oracle(name, scale):
    w = wl.WORKLOADS[name]
    if scale:
        w = wl.scaled(w, **scale)
    w, g, _ = wl.make(w, 4, tensors=False)
    got = bench.plan_imbalances(g, w.tile_k, bin_counts=(4, 64, 256))
    costs = planner.chunk_costs(g.anchors, g.lo, g.chunk_pos, g.chunk_len, w.tile_k)
    n = len(costs)
    for m in (4, 64, 256):
        bins, load = planner.plan_lpt(costs, m)
        cont = planner.loads_of(costs, planner.plan_contiguous(n, m), m)
        assert got[str(m)]["lpt"] == planner.imbalance(load)
        assert got[str(m)]["contiguous"] == planner.imbalance(cont)
        # LPT never does worse than the contiguous split here
        assert got[str(m)]["lpt"] <= got[str(m)]["contiguous"]


def test_balance_stats_from_workgroup_stamps():
    """Synthetic stamps: 16 workgroups, XCD class 3 runs 10 % longer; the
    realised imbalance, span and per-XCD means follow by hand."""
    import bench
    n = 16
    runs = []
    for shift in (0, 1000):
        r = np.zeros((3, n, 2), np.int64)
        for k in range(3):
            for w in range(n):
                d = 1100 if w % 8 == 3 else 1000          # ticks (10 / 11 us)
                r[k, w] = (shift + 5 * w, shift + 5 * w + d)
        runs.append(r)
    planned = {"fwd_bf16": 0.01, "bwd_dq": 0.02, "bwd_dkdv": 0.03}
    out = bench.balance_stats(runs, planned)
    mean = (14 * 10.0 + 2 * 11.0) / 16
    for name in planned:
        v = out[name]
        assert v["planned_imbalance"] == planned[name]
        assert abs(v["realized_imbalance_median"] - (11.0 / mean - 1)) < 1e-12
        assert abs(v["mean_workgroup_us"] - mean) < 1e-12
        # last end: workgroup 11 (class 3) at 5 * 11 + 1100 ticks
        assert abs(v["kernel_span_us_median"] - (55 + 1100) / 100.0) < 1e-12
        assert v["xcd_mean_us"] == [10.0, 10.0, 10.0, 11.0, 10.0, 10.0, 10.0, 10.0]
