"""CPU pins of skv_plan_lpt_split, the LPT-with-splitting placement of the
in-GPU forward / dQ work items: hand-traced fixtures, equality with the
oracle's plain LPT when cuts are off, and a decision-by-decision check of
every plan against the rule the header states (LPT order from the rit.work
blog on Split-KV, section "Split-KV moves queries, not keys and values")."""
import json
import os

import numpy as np
import pytest

import oracle
from block_sparse_split_amd import splitkv as skv

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "lpt_split_hand.json")


def _target(x):
    return skv.NO_CUT if x == "no_cut" else int(x)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_traced_cases(case):
    pieces, cost, target, load = skv.skv_plan_lpt_split(
        case["extra"], case["steps"], case["item_cost"], case["step_cost"], case["n_bins"],
        _target(case["target"]))
    assert target == _target(case["expect_target"])
    got = [list(map(int, p)) + [int(c)] for p, c in zip(pieces, cost)]
    assert got == case["pieces"]
    assert load.tolist() == case["load"]


def _unit_cost(extra, steps, item_cost, step_cost, u, k0):
    return item_cost + (extra[u] if k0 == 0 else 0) + step_cost * (steps[u] - k0)


def check_plan(extra, steps, item_cost, step_cost, m, target, pieces, cost, load):
    """Every placement decision against the stated rule, replayed in order."""
    n_units = len(steps)
    assert len(pieces) <= n_units + m
    cur = np.zeros(m, np.int64)
    last_pending = None
    next_k0 = np.zeros(n_units, np.int64)   # each unit's pieces come in step order
    cuts = np.zeros(m, np.int64)
    for (u, k0, k1, b), c in zip(pieces.tolist(), cost.tolist()):
        assert 0 <= u < n_units and 0 <= b < m
        assert k0 == next_k0[u], "pieces of a unit must tile its steps in order"
        pending = _unit_cost(extra, steps, item_cost, step_cost, u, k0)
        # largest pending first; ties lower unit, then lower k0
        key = (-pending, u, k0)
        if last_pending is not None:
            assert key > last_pending
        last_pending = key
        # least-loaded bin, ties to the lower bin
        assert cur[b] == cur.min() and b == int(np.argmin(cur))
        head = item_cost + (extra[u] if k0 == 0 else 0)
        whole_end = max(steps[u], k0)
        assert c == head + step_cost * (k1 - k0)
        can_cut = (cur[b] + pending > target and steps[u] - k0 > 1
                   and target - cur[b] >= head + step_cost)
        if k1 < whole_end:                      # a cut
            assert can_cut
            assert k1 > k0
            # the longest prefix that fits: one more step would not
            assert cur[b] + c <= target < cur[b] + c + step_cost
            cuts[b] += 1
        else:
            # taken whole: it fits, has fewer than two steps, or the bin has
            # no room for its fixed part and one step
            assert k1 == whole_end
            assert not can_cut
        cur[b] += c
        next_k0[u] = k1
    assert np.all(next_k0 == np.asarray(steps)), "every step of every unit placed once"
    assert np.all(cuts <= 1), "a bin is cut at most once"
    assert np.array_equal(cur, load)
    return cuts.sum()


def _random_instance(rng):
    n = int(rng.integers(0, 60))
    m = int(rng.integers(1, 17))
    steps = rng.integers(0, int(rng.integers(1, 40)), size=n)
    extra = np.where(rng.random(n) < 0.3, rng.integers(0, 30, size=n), 0)
    item_cost = int(rng.choice([0, 1, 5, 44]))
    step_cost = int(rng.choice([0, 1, 3, 8]))
    return extra, steps, item_cost, step_cost, m


def test_never_cut_equals_oracle_lpt():
    """target = INT64_MAX: every unit is one piece and the placement is the
    oracle's O(n*m) LPT scan on the unit costs."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        extra, steps, ic, sc, m = _random_instance(rng)
        pieces, cost, target, load = skv.skv_plan_lpt_split(extra, steps, ic, sc, m, skv.NO_CUT)
        costs = np.array([ic + e + sc * s for e, s in zip(extra, steps)], np.int64)
        bins, lo = oracle.plan_lpt(costs, m)
        order = sorted(range(len(costs)), key=lambda j: (-int(costs[j]), j))
        assert pieces[:, 0].tolist() == order
        assert np.all(pieces[:, 1] == 0) and np.array_equal(pieces[:, 2], steps[order])
        assert np.array_equal(pieces[:, 3], bins[order])
        assert np.array_equal(cost, costs[order])
        assert np.array_equal(load, lo)


def test_every_decision_follows_the_rule():
    rng = np.random.default_rng(12)
    n_cuts = 0
    for i in range(300):
        extra, steps, ic, sc, m = _random_instance(rng)
        total = int(sum(ic + e + sc * s for e, s in zip(extra, steps)))
        tgt = 0 if i % 3 else int(rng.integers(1, max(2, total // m + 50)))
        pieces, cost, target, load = skv.skv_plan_lpt_split(extra, steps, ic, sc, m, tgt)
        if tgt == 0:
            assert target >= -(-total // m)   # the automatic target starts at the mean
        else:
            assert target == tgt
        n_cuts += check_plan(extra, steps, ic, sc, m, target, pieces, cost, load)
    assert n_cuts > 100   # the instances do exercise cuts


def test_checker_rejects_a_planted_mistake():
    """The decision checker itself: a plan whose cut overshoots the target
    by a step must fail it."""
    extra, steps, ic, sc, m = [0, 0], [10, 2], 2, 1, 2
    pieces, cost, target, load = skv.skv_plan_lpt_split(extra, steps, ic, sc, m, 0)
    check_plan(extra, steps, ic, sc, m, target, pieces, cost, load)
    bad_p, bad_c, bad_l = pieces.copy(), cost.copy(), load.copy()
    bad_p[0, 2] += 1   # the cut keeps one step too many
    bad_p[1, 1] += 1
    bad_c[0] += 1
    bad_c[1] -= 1
    with pytest.raises(AssertionError):
        check_plan(extra, steps, ic, sc, m, target, bad_p, bad_c, bad_l)


def test_invalid_arguments():
    with pytest.raises(skv.SplitKVError):
        skv.skv_plan_lpt_split([0], [-1], 1, 1, 2)
    with pytest.raises(skv.SplitKVError):
        skv.skv_plan_lpt_split([0], [1], 1, 1, 0)
    with pytest.raises(skv.SplitKVError):
        skv.skv_plan_lpt_split([0], [1], -1, 1, 2)
    with pytest.raises(skv.SplitKVError):
        skv.skv_plan_lpt_split([0], [1], 1, 1, 2, target=-5)
    with pytest.raises(skv.SplitKVError):
        skv.skv_plan_lpt_split([2 ** 61], [1], 1, 1, 2)
    p, c, t, ld = skv.skv_plan_lpt_split([], [], 3, 1, 4)
    assert len(p) == 0 and ld.tolist() == [0, 0, 0, 0]
