"""Pins for the oracle's cost model and LPT planner (CPU only).

Hand-traced fixtures (tests/golden), brute force key by key, closed forms,
exhaustive optimum on tiny instances with Graham's 4/3 - 1/(3m) bound, and
Graham's tight instance.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import planner as opl
from block_sparse_split_amd import workloads as wl


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_cost_hand_fixtures(golden_dir):
    for c in load(golden_dir, "cost_hand.json")["cases"]:
        got = oracle.chunk_costs(c["anchors"], c["lo"], c["chunk_pos"],
                                 c["chunk_len"], c["tile_k"])
        assert got.tolist() == c["costs"], c["name"]


def _costs_key_by_key(anchors, lo, chunk_pos, chunk_len, tile_k):
    out = []
    for p, n in zip(chunk_pos, chunk_len):
        total = 0
        for u in range(math.ceil(n / tile_k)):
            keys = range(p + u * tile_k, min(p + (u + 1) * tile_k, p + n))
            for a, l in zip(anchors, lo):
                total += any(l <= j < a for j in keys)
        out.append(total)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_costs_match_key_by_key_enumeration(seed):
    rng = np.random.default_rng(seed)
    w = wl.scaled(wl.WORKLOADS["varlen8_fwdbwd"], n_seq=3, blocks_per_seq=5,
                  len_median=300, len_min=40, len_max=900, chunk=int(rng.integers(7, 50)))
    _, g, _ = wl.make(w, seed, tensors=False)
    tk = int(rng.integers(1, 20))
    got = oracle.chunk_costs(g.anchors, g.lo, g.chunk_pos, g.chunk_len, tk)
    want = _costs_key_by_key(g.anchors.tolist(), g.lo.tolist(),
                             g.chunk_pos.tolist(), g.chunk_len.tolist(), tk)
    assert got.tolist() == want


def test_cost_closed_forms():
    # A chunk below every anchor costs nb * ceil(len / T).
    anchors = np.array([300, 410, 999], np.int32)
    lo = np.zeros(3, np.int32)
    c = oracle.chunk_costs(anchors, lo, [0, 100], [100, 130], 64)
    assert c.tolist() == [3 * 2, 3 * math.ceil(130 / 64)]
    # Single sequence, T-aligned chunks covering [0, L): the total is
    # sum_i ceil(a_i / T).
    _, g, _ = wl.make("ctx32k_q2k", 1, tensors=False)
    c = oracle.chunk_costs(g.anchors, g.lo, g.chunk_pos, g.chunk_len, 64)
    assert int(c.sum()) == int(np.ceil(g.anchors / 64).sum())
    # Tiny fp32 workload, T = 64: chunks 0 and 1 lie below every anchor
    # (anchors >= 256), so they cost 2 tiles x 4 blocks.
    _, g0, _ = wl.make("tiny_f32_ctx1k", 0, tensors=False)
    c0 = oracle.chunk_costs(g0.anchors, g0.lo, g0.chunk_pos, g0.chunk_len, 64)
    assert c0[0] == 8 and c0[1] == 8


def test_lpt_hand_fixtures(golden_dir):
    for c in load(golden_dir, "lpt_hand.json")["cases"]:
        bins, load_ = oracle.plan_lpt(c["costs"], c["m"])
        assert bins.tolist() == c["bins"], c["name"]
        assert load_.tolist() == c["load"], c["name"]


def _opt_makespan(costs, m):
    best = math.inf
    for assign in itertools.product(range(m), repeat=len(costs)):
        if assign and assign[0] != 0:
            continue  # bins are symmetric: fix the first job's bin
        ld = [0] * m
        for c, b in zip(costs, assign):
            ld[b] += c
        best = min(best, max(ld))
    return best


@pytest.mark.parametrize("seed", range(40))
def test_lpt_within_graham_bound_of_exhaustive_optimum(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(1, 4))
    n = int(rng.integers(1, 9))
    costs = rng.integers(0, 20, size=n).tolist()
    bins, ld = oracle.plan_lpt(costs, m)
    assert oracle.makespan(costs, bins, m) == ld.max()
    assert sorted(bins.tolist()) == sorted(bins.tolist()) and ld.sum() == sum(costs)
    opt = _opt_makespan(costs, m)
    assert opt <= ld.max() <= (4 / 3 - 1 / (3 * m)) * opt + 1e-9


@pytest.mark.parametrize("m", [2, 3, 4, 5, 6])
def test_graham_tight_instance(m):
    costs = []
    for v in range(2 * m - 1, m, -1):
        costs += [v, v]
    costs += [m, m, m]
    bins, ld = oracle.plan_lpt(costs, m)
    assert ld.max() == 4 * m - 1
    assert sum(costs) == 3 * m * m  # so the optimum is at least 3m
    if m <= 3:
        assert _opt_makespan(costs, m) == 3 * m


def test_lpt_degenerate_cases():
    bins, ld = oracle.plan_lpt([5, 1, 9, 0], 1)
    assert bins.tolist() == [0, 0, 0, 0] and ld.tolist() == [15]
    costs = [4, 11, 7, 2]
    bins, _ = oracle.plan_lpt(costs, 6)
    rank = np.argsort(-np.array(costs), kind="stable")
    for k, c in enumerate(rank):
        assert bins[c] == k
    bins, ld = oracle.plan_lpt([], 3)
    assert bins.size == 0 and ld.tolist() == [0, 0, 0]


def test_imbalance_and_contiguous():
    assert oracle.imbalance([10, 10, 10]) == 0.0
    assert oracle.imbalance([12, 9, 9]) == pytest.approx(0.2)
    assert oracle.imbalance([4, 0, 0, 0]) == pytest.approx(3.0)
    assert oracle.plan_contiguous(8, 4).tolist() == [0, 0, 1, 1, 2, 2, 3, 3]
    assert oracle.plan_contiguous(5, 2).tolist() == [0, 0, 0, 1, 1]


def test_mutation_highest_bin_tie_break_is_caught(golden_dir, monkeypatch):
    """Planting 'ties go to the highest bin' must break a hand fixture."""
    def bad(costs, m):
        costs = [int(c) for c in costs]
        order = sorted(range(len(costs)), key=lambda c: (-costs[c], c))
        load_ = np.zeros(m, np.int64)
        bins = np.zeros(len(costs), np.int32)
        for c in order:
            b = m - 1 - int(np.argmin(load_[::-1]))
            bins[c] = b
            load_[b] += costs[c]
        return bins, load_
    monkeypatch.setattr(opl, "plan_lpt", bad)
    cases = load(golden_dir, "lpt_hand.json")["cases"]
    assert any(opl.plan_lpt(c["costs"], c["m"])[0].tolist() != c["bins"]
               for c in cases)
