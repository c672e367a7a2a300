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
