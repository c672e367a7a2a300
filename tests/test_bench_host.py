"""Host-side figures of bench.py (no GPU): the chunk-level LPT and
contiguous-split imbalances reported for the 1M-context job follow the
oracle's independent LPT scan and contiguous split exactly, and the
realised-spread decomposition separates per-XCD, per-queue and per-run
parts of synthetic queue times."""
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
    """Synthetic stamps: 16 workgroups, XCD 3 runs 10 % longer; the realised
    imbalance, span, per-XCD means (by the stamped XCC_ID), placement share
    and CU count follow by hand."""
    import bench
    n = 16
    runs = []
    for shift in (0, 1000):
        r = np.zeros((3, n, 4), np.int64)
        for k in range(3):
            for w in range(n):
                d = 1100 if w % 8 == 3 else 1000          # ticks (10 / 11 us)
                # XCC_ID w mod 8, except workgroup 5 which reports XCD 3;
                # HW_ID: CU w // 8, SE 1
                xcc = 3 if w == 5 else w % 8
                r[k, w] = (shift + 5 * w, shift + 5 * w + d, 0x100 | xcc,
                           (1 << 13) | ((w // 8) << 8))
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
        # XCD 3 holds workgroups 3, 11 (11 us) and 5 (10 us); XCD 5 only 13
        assert v["xcd_mean_us"] == [10.0, 10.0, 10.0, 32.0 / 3, 10.0, 10.0, 10.0, 10.0]
        assert v["on_xcd_w_mod_8"] == 15 / 16
        assert v["xcd_rotation_per_run"] == [0, 0]
        assert v["on_xcd_w_plus_c_mod_8"] == 15 / 16
        # (XCD, SE, CU): workgroups 5 and 3 share (3, 1, 0)
        assert v["distinct_cus_per_run"] == 15
    only = bench.balance_stats(runs, planned, ("fwd_bf16",))
    assert list(only) == ["fwd_bf16"]
    # every workgroup one XCD further on: rotation 1, all consistent
    for r in runs:
        r[:, :, 2] = 0x100 | ((np.arange(n) + 1) % 8)
    v = bench.balance_stats(runs, planned)["bwd_dq"]
    assert v["on_xcd_w_mod_8"] == 0.0
    assert v["xcd_rotation_per_run"] == [1, 1] and v["on_xcd_w_plus_c_mod_8"] == 1.0


def test_item_pair_loads_by_hand():
    """Two anchor blocks (G = 16: one block per 256-row query tile), one kv
    head, three 64-key tiles; block 0 sees keys [0, 100), block 1 [0, 200).
    Pair counts: query tile 0 sees tiles 0, 1 (2 pairs), query tile 1 sees
    tiles 0, 1, 2 (3 pairs), plus one draft pair per block."""
    import bench
    from block_sparse_split_amd import splitkv as skv
    from block_sparse_split_amd import workloads as wl

    class G_:
        anchors = np.array([100, 200], np.int32)
        lo = np.array([0, 0], np.int32)
    w = wl.scaled(wl.WORKLOADS["ctx32k_q2k"], hq=16, hkv=1, d=64, blocks_per_seq=2)
    prob = skv.Problem(nb=2, hq=16, hkv=1, d=64, scale=0.125, dtype=skv.SKV_BF16,
                       anchors=G_.anchors, lo=G_.lo, chunk_pos=[0], chunk_off=[0, 192],
                       with_draft=True)
    for n_wg in (1, 2, 5):
        image, info = skv.skv_schedule_build(prob, n_wg)
        loads = bench.item_pair_loads(image, G_, w)
        assert len(loads) == n_wg
        assert loads.sum() == (2 + 1) + (3 + 1)
    image, info = skv.skv_schedule_build(prob, 1)
    assert bench.item_pair_loads(image, G_, w).tolist() == [7]


def test_spread_decomposition_separates_its_parts():
    """Queue times built from a plan's loads times known per-XCD factors,
    known per-queue factors that repeat every run, and small per-run noise:
    the decomposition's spread without the XCD part is that of the queue
    factors and noise, without both that of the noise, and the queue
    residual it reports is the queue factors'.  Queues planned at per-XCD
    speeds (load / speed) count as on time."""
    rng = np.random.default_rng(3)
    n, runs = 64, 8
    load = rng.uniform(900, 1100, n)
    speed = 1 + 0.05 * np.sin(np.arange(8))
    xfac = 1 + 0.04 * np.cos(np.arange(8))           # per-XCD deviation from the plan
    qfac = 1 + 0.02 * rng.standard_normal(n)         # per-queue model error
    qfac /= qfac.mean()
    dur = np.zeros((runs, n))
    xcc = np.zeros((runs, n), np.int64)
    for r in range(runs):
        x = (np.arange(n) + r) % 8                   # a rotation of queues to XCDs
        xcc[r] = x
        noise = 1 + 0.002 * rng.standard_normal(n)
        dur[r] = load / speed[np.arange(n) % 8] * xfac[x] * qfac * noise
    d = bench.spread_decomposition(dur, xcc, load, speed)
    planned = load / speed[np.arange(n) % 8]
    imb = lambda a: a.max() / a.mean() - 1
    assert abs(d["if_xcd_speeds_matched"] - imb(planned * qfac)) < 0.01
    assert d["if_queue_residual_matched_too"] < imb(planned) + 0.01
    assert abs(d["queue_residual_rms"] - np.sqrt(np.mean((qfac - 1) ** 2))) < 0.002
    # with the XCD factors, the realised spread is clearly larger
    assert imb(dur[0]) > d["if_xcd_speeds_matched"] + 0.02
