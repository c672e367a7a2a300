"""CPU checks of the schedule planned for XCDs of unequal speed
(skv_schedule_build_xcd): the forward, dQ and dK/dV plans each cover the
same work once, balance time rather than load at their own kernel's
speeds, keep work in its kv head's XCD class unless moving it saves time,
and the speed estimate inverts the stamps it is made from.  No device call
is made."""
import numpy as np
import pytest

import oracle
from block_sparse_split_amd import splitkv as skv
from block_sparse_split_amd import workloads as wl
from block_sparse_split_amd import shards
from block_sparse_split_amd.csrc_layout import H, I, K, T_WORDS, I_WORDS, K_WORDS, QTILE, BLOCK

STEP_COST, ITEM_COST = 8, 44


def _case(name, seed, shard_of=None, **over):
    w = wl.scaled(wl.WORKLOADS[name], **over) if over else wl.WORKLOADS[name]
    w, g, _ = wl.make(w, seed, tensors=False)
    if shard_of is None:
        return w, g, shards.whole_context_problem(w, g)
    ids, _, _, _ = shards.lpt_shards(w, g, w.n_shards)
    return w, g, shards.shard_problem(w, g, ids[shard_of], shard_of == 0)


def _queues(image, off_key, q_key, n):
    h = {k: int(image[v]) for k, v in H.items()}
    off = image[h[off_key]: h[off_key] + h["NWG"] + 1]
    q = image[h[q_key]: h[q_key] + n]
    return [q[off[v]:off[v + 1]].tolist() for v in range(h["NWG"])]


def _decode(image):
    h = {k: int(image[v]) for k, v in H.items()}
    tiles = image[h["OFF_TILES"]: h["OFF_TILES"] + h["NTILES"] * T_WORDS].reshape(-1, T_WORDS)
    items = image[h["OFF_ITEMS"]: h["OFF_ITEMS"] + h["NITEMS"] * I_WORDS].reshape(-1, I_WORDS)
    kv = image[h["OFF_KV"]: h["OFF_KV"] + h["NKV"] * K_WORDS].reshape(-1, K_WORDS)
    return (h, tiles, items, kv, _queues(image, "OFF_QOFF", "OFF_QUEUE", h["NITEMS"]),
            _queues(image, "OFF_KVQOFF", "OFF_KVQUEUE", h["NKV"]))


def _decode_dq(image, info):
    """dQ's items, queues and split records (dQ's own sections)."""
    h = {k: int(image[v]) for k, v in H.items()}
    n = info.n_dq_items
    items = image[h["OFF_DQ_ITEMS"]: h["OFF_DQ_ITEMS"] + n * I_WORDS].reshape(-1, I_WORDS)
    split = image[h["OFF_DQ_SPLIT"]: h["OFF_DQ_SPLIT"] + 4 * info.n_dq_split_qtiles]
    return items, _queues(image, "OFF_DQ_QOFF", "OFF_DQ_QUEUE", n), split.reshape(-1, 4)


def _speeds(seed, spread):
    rng = np.random.default_rng(seed)
    return (1.0 + spread * rng.uniform(-1, 1, (3, 8))).astype(np.float32)


CASES = [
    ("ctx32k_q2k", 1, None, 256, {}),
    ("varlen8_fwdbwd", 3, None, 256, dict(len_median=2048, len_min=512, len_max=8192)),
    ("ctx32k_q2k", 3, None, 64, dict(ctx=4096, anchor_lo=512, anchor_hi=4096, blocks_per_seq=24,
                                     hq=32, hkv=2)),
    ("cp64_rank0_ctx512k", 2, 5, 256, {}),
    ("tiny_f32_ctx1k", 0, 0, 8, {}),
]


@pytest.mark.parametrize("case", CASES)
def test_xcd_plan_covers_the_work_once(case):
    """Every (kv head, query tile, visible tile) in exactly one item, item
    costs as in the uniform plan, every item in exactly one forward/dQ
    queue and every dK/dV item in exactly one dK/dV queue."""
    name, seed, shard_of, n_wg, over = case
    w, g, prob = _case(name, seed, shard_of, **over)
    image, info = skv.skv_schedule_build_xcd(prob, n_wg, _speeds(seed, 0.1))
    assert info.xcd_mode == 1
    h, tiles, items_f, kv, fq_f, kq = _decode(image)
    assert h["XCD"] == 1 and h["NWG"] == n_wg
    items_d, fq_d, split_d = _decode_dq(image, info)
    # dQ has sections of its own, after the forward's
    assert h["OFF_DQ_ITEMS"] > h["OFF_ITEMS"] and h["OFF_DQ_SPLIT"] > h["OFF_SPLIT"]
    G = w.hq // w.hkv
    qtph = -(-w.nq * G // QTILE)
    for items, fq, n_slots in ((items_f, fq_f, info.n_partial_slots),
                               (items_d, fq_d, info.n_dq_partial_slots)):
        seen = np.zeros((w.hkv, qtph, len(tiles)), np.int32)
        draft = np.zeros((w.hkv, qtph), np.int32)
        for it in items:
            hd, qt, t0, t1 = it[I["HEAD"]], it[I["QT"]], it[I["T0"]], it[I["T1"]]
            seen[hd, qt, t0:t1] += 1
            draft[hd, qt] += it[I["FLAGS"]] & 1
            b0 = qt * (QTILE // G) // BLOCK
            b1 = min(w.nb, -(-((qt + 1) * (QTILE // G)) // BLOCK))
            want = ITEM_COST + STEP_COST * (t1 - t0)
            if it[I["FLAGS"]] & 1:
                want += STEP_COST * -(-((b1 - b0) * BLOCK) // 64)
            assert it[I["COST"]] == want
        for qt in range(qtph):
            b0 = qt * (QTILE // G) // BLOCK
            b1 = min(w.nb, -(-((qt + 1) * (QTILE // G)) // BLOCK))
            vis = np.array([oracle.tile_pairs_visible(g.anchors[b0:b1], g.lo[b0:b1], t[1],
                                                      t[1] + t[2]) > 0 for t in tiles], bool)
            for hd in range(w.hkv):
                assert np.array_equal(seen[hd, qt] > 0, vis)
                assert seen[hd, qt].max(initial=0) <= 1
                assert draft[hd, qt] == int(prob.c.with_draft)
        assert sorted(i for q in fq for i in q) == list(range(len(items)))
        # partial slots: a query tile cut into several items numbers them
        # consecutively, a single item writes its rows directly
        per_qt = {}
        for it in items:
            per_qt.setdefault((it[0], it[1]), []).append(it[I["SLOT"]])
        slots = sorted(s for v in per_qt.values() if len(v) > 1 for s in v)
        assert slots == list(range(n_slots))
        assert all(v == [-1] for v in per_qt.values() if len(v) == 1)
    assert sorted(i for q in kq for i in q) == list(range(len(kv)))
    # dQ's split records: one per cut query tile, naming its slots
    recs = sorted(((int(r[0]), int(r[1])), int(r[2]), int(r[3])) for r in split_d)
    cut = {}
    for it in items_d:
        if it[I["SLOT"]] >= 0:
            cut.setdefault((int(it[0]), int(it[1])), []).append(int(it[I["SLOT"]]))
    assert recs == sorted((k, min(v), len(v)) for k, v in cut.items())
    assert info.n_dq_items == len(items_d) and info.n_dq_split_qtiles == len(split_d)
    # the backward workspace holds dQ's slots, the forward's holds the forward's
    assert info.bwd_workspace_bytes >= info.n_dq_partial_slots * QTILE * w.d * 4
    assert info.fwd_workspace_bytes >= info.n_partial_slots * QTILE * (w.d + 1) * 4


def _times(loads, speed8):
    n = len(loads)
    return loads / np.array([speed8[v % 8] for v in range(n)], np.float64)


@pytest.mark.parametrize("name,seed,over", [("ctx32k_q2k", 1, {}),
                                            ("varlen8_fwdbwd", 3, {}),
                                            ("cp64_rank0_ctx512k", 2, {})])
def test_xcd_plan_balances_time_at_unequal_speeds(name, seed, over):
    """With XCD speeds 0.95-1.05 (different in each kernel) the slowest
    queue of each kernel never finishes later than in the uniform plan
    timed at the same speeds; where the items are fine enough (the uniform
    plan balances equal speeds within 2 %), queue time is balanced within
    2.5 % while the uniform plan, at these speeds, is off by several per
    cent.  The forward, dQ and dK/dV are each planned at their own speeds.
    info reports each plan's speed-normalised maximum."""
    w, g, prob = _case(name, seed, 0 if name.startswith("cp64") else None, **over)
    sp = _speeds(seed + 10, 0.05)
    base, _ = skv.skv_schedule_build(prob, 256)
    bloads = skv.queue_loads(base).astype(np.float64)
    image, info = skv.skv_schedule_build_xcd(prob, 256, sp)
    loads = skv.queue_loads(image).astype(np.float64)
    for k in range(3):
        t, tb, lu = _times(loads[k], sp[k]), _times(bloads[k], sp[k]), bloads[k]
        # never slower than the uniform plan at these speeds (the builder
        # keeps whichever finishes first) ...
        assert t.max() <= tb.max() * (1 + 1e-9), (k, t.max(), tb.max())
        # ... and where the items are fine enough for the uniform plan to
        # balance equal speeds within 2 %, within 2.5 % here and clearly
        # better than the uniform plan
        grain = lu.max() / lu.mean() - 1
        if grain < 0.02:
            imb = t.max() / t.mean() - 1
            imb_base = tb.max() / tb.mean() - 1
            assert imb < 0.025, (k, imb, grain)
            assert imb < imb_base - 0.01, (k, imb, imb_base)
    for k, mx, tot in ((0, info.item_cost_max_bin, info.item_cost_total),
                       (1, info.dq_cost_max_bin, info.dq_cost_total),
                       (2, info.kv_cost_max_bin, info.kv_cost_total)):
        norm = loads[k] * sp[k].mean() / np.array([sp[k][v % 8] for v in range(256)])
        assert abs(mx - norm.max()) <= 1, k
        assert tot == int(loads[k].sum()), k


def test_xcd_plan_keeps_heads_home_at_equal_speeds():
    """Eight kv heads on eight XCDs with equal work and equal speeds: no
    forward/dQ or dK/dV work leaves its kv head's XCD class; at unequal
    speeds only a few per cent of it does."""
    w, g, prob = _case("ctx32k_q2k", 1)
    for spread, bound in ((0.0, 0.0), (0.05, 0.08)):
        image, info = skv.skv_schedule_build_xcd(prob, 256, np.ones((3, 8)) + spread *
                                                 np.sin(np.arange(24)).reshape(3, 8))
        h, tiles, items, kv, fq, kq = _decode(image)
        items_d, fq_d, _ = _decode_dq(image, info)
        ncls = h["NCLASS"]
        for qs, heads, cost in ((fq, items[:, I["HEAD"]], items[:, I["COST"]]),
                                (fq_d, items_d[:, I["HEAD"]], items_d[:, I["COST"]]),
                                (kq, kv[:, K["HEAD"]], kv[:, K["COST"]])):
            away = sum(int(cost[i]) for v, q in enumerate(qs) for i in q
                       if heads[i] % ncls != v % ncls)
            assert away <= bound * cost.sum(), (spread, away / cost.sum())


def test_xcd_plan_arguments():
    w, g, prob = _case("tiny_f32_ctx1k", 0, 0)
    ok = np.ones((3, 8), np.float32)
    with pytest.raises(skv.SplitKVError, match="divisible by 8"):
        skv.skv_schedule_build_xcd(prob, 12, ok)
    for bad in (0.0, -1.0, np.nan, np.inf):
        sp = ok.copy()
        sp[1, 3] = bad
        with pytest.raises(skv.SplitKVError, match="finite and > 0"):
            skv.skv_schedule_build_xcd(prob, 8, sp)
    with pytest.raises(ValueError):
        skv.skv_schedule_build_xcd(prob, 8, np.ones(8))
    # the C entry point refuses a NULL speed table
    info = skv.SkvScheduleInfo()
    import ctypes
    st = skv.lib().skv_schedule_build_xcd(ctypes.byref(prob.c), 8, None, None, None, 0,
                                          ctypes.byref(info))
    assert skv.STATUS_NAMES[st] == "SKV_ERR_INVALID_ARG"
    # without speeds the image keeps one queue set, shared by the forward
    # and dQ, and no XCD claim
    image, info = skv.skv_schedule_build(prob, 8)
    h = {k: int(image[v]) for k, v in H.items()}
    assert info.xcd_mode == 0 and h["XCD"] == 0
    for f in ("ITEMS", "QOFF", "QUEUE", "SPLIT"):
        assert h["OFF_DQ_" + f] == h["OFF_" + f]
    assert (info.n_dq_items, info.n_dq_split_qtiles, info.n_dq_partial_slots,
            info.dq_cost_total, info.dq_cost_max_bin) == (
        info.n_items, info.n_split_qtiles, info.n_partial_slots, info.item_cost_total,
        info.item_cost_max_bin)


def test_speeds_from_stamps_invert_a_known_speed():
    """Stamps made from a known per-XCD speed (queue time = planned load /
    speed of the XCD it ran on, under any rotation of queues to XCDs, with
    a workgroup missing its stamp) give that speed back, scaled to mean 1."""
    w, g, prob = _case("ctx32k_q2k", 2, None, ctx=4096, anchor_lo=512, anchor_hi=4096,
                       blocks_per_seq=16)
    image, info = skv.skv_schedule_build(prob, 64)
    loads = skv.queue_loads(image)
    assert loads.shape == (3, 64) and loads[0].sum() == info.item_cost_total
    assert loads[2].sum() == info.kv_cost_total
    true = np.array([[1.0, 1.1, 0.9, 1.0, 1.05, 0.95, 1.0, 1.0]] * 3)
    true[2] = true[2][::-1]
    runs = []
    for c in (0, 3, 5):
        r = np.zeros((3, 64, 4), np.int64)
        for k in range(3):
            for v in range(64):
                x = (v + c) % 8
                r[k, v, 0] = 1000
                r[k, v, 1] = 1000 + int(round(1e4 * loads[k, v] / true[k, x]))
                r[k, v, 2] = x | 0x100   # high bits of XCC_ID are ignored
        r[1, 7] = 0                      # a queue without stamps is skipped
        runs.append(r)
    got = skv.xcd_speeds_from_stamps(image, runs)
    np.testing.assert_allclose(got, true / true.mean(1, keepdims=True), rtol=1e-3)


def test_cost_scales_scale_the_plan():
    """Cost scales of 1 give the plan without them, word for word; other
    scales multiply each unit's cost (item costs are the scaled, rounded
    base costs of their (kv head, query tile)), every plan still covers the
    work once, and scales are refused without speeds, with bad values or
    with the wrong size."""
    name, seed, shard_of, n_wg, over = CASES[1]
    w, g, prob = _case(name, seed, shard_of, **over)
    sp = _speeds(seed, 0.05)
    qtph = prob.qt_per_head
    base, binfo = skv.skv_schedule_build_xcd(prob, n_wg, sp)
    ones, oinfo = skv.skv_schedule_build_xcd(prob, n_wg, sp, np.ones((2, w.hkv, qtph)))
    assert np.array_equal(base, ones) and oinfo.item_cost_total == binfo.item_cost_total
    rng = np.random.default_rng(5)
    scale = rng.uniform(0.8, 1.25, (2, w.hkv, qtph)).astype(np.float32)
    image, info = skv.skv_schedule_build_xcd(prob, n_wg, sp, scale)
    h, tiles, items_f, kv, fq_f, kq = _decode(image)
    items_d, fq_d, _ = _decode_dq(image, info)
    G = w.hq // w.hkv
    for k, items, fq in ((0, items_f, fq_f), (1, items_d, fq_d)):
        seen = np.zeros((w.hkv, qtph, len(tiles)), np.int32)
        for it in items:
            hd, qt, t0, t1 = it[I["HEAD"]], it[I["QT"]], it[I["T0"]], it[I["T1"]]
            seen[hd, qt, t0:t1] += 1
            b0 = qt * (QTILE // G) // BLOCK
            b1 = min(w.nb, -(-((qt + 1) * (QTILE // G)) // BLOCK))
            want = ITEM_COST + STEP_COST * (t1 - t0)
            if it[I["FLAGS"]] & 1:
                want += STEP_COST * -(-((b1 - b0) * BLOCK) // 64)
            assert abs(it[I["COST"]] - float(scale[k, hd, qt]) * want) <= 0.5 + 1e-6
        assert seen.max() <= 1
        assert sorted(i for q in fq for i in q) == list(range(len(items)))
    loads = skv.queue_loads(image)
    assert info.item_cost_total == loads[0].sum() and info.dq_cost_total == loads[1].sum()
    with pytest.raises(skv.SplitKVError, match="finite and > 0"):
        bad = scale.copy()
        bad[1, 0, 3] = np.nan
        skv.skv_schedule_build_xcd(prob, n_wg, sp, bad)
    with pytest.raises(ValueError, match="cost_scale must hold"):
        skv.skv_schedule_build_xcd(prob, n_wg, sp, scale[:, :, :-1])
    import ctypes
    info = skv.SkvScheduleInfo()
    cs = np.ascontiguousarray(scale.reshape(-1))
    st = skv.lib().skv_schedule_build(ctypes.byref(prob.c), n_wg, None, 0, ctypes.byref(info))
    assert skv.STATUS_NAMES[st] == "SKV_OK"
    # the uniform builder takes no scales; the per-XCD builder needs speeds
    st = skv.lib().skv_schedule_build_xcd(ctypes.byref(prob.c), n_wg, None,
                                          cs.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                          None, 0, ctypes.byref(info))
    assert skv.STATUS_NAMES[st] == "SKV_ERR_INVALID_ARG"


def test_calibration_recovers_known_costs():
    """Stamps made from known per-XCD speeds and known per-(kv head, query
    tile group) cost scales, over two plans (the second built with scales,
    whose item costs the fit divides back out), give those speeds and
    scales back; a plan built with them balances the true queue times
    better than the plan without them."""
    w, g, prob = _case("varlen8_fwdbwd", 3, None, len_median=2048, len_min=512, len_max=8192)
    qtph, hkv = prob.qt_per_head, w.hkv
    per = -(-qtph // 8)
    ng = -(-qtph // per)
    rng = np.random.default_rng(11)
    true_sig = rng.uniform(0.9, 1.12, (2, hkv, ng))
    # each head's scales have a cost-weighted mean near 1 only after the
    # fit's normalisation, so compare shapes: normalise per head below
    true_scale = np.repeat(true_sig, per, axis=2)[:, :, :qtph]
    true_speed = np.ones((3, 8)) + 0.04 * np.sin(np.arange(24)).reshape(3, 8)

    def stamps(image, used):
        _, plans = skv._plan_sections(image)
        loads_kv = skv.queue_loads(image)[2]
        n = len(plans[0][1]) - 1
        runs = []
        for c in (0, 5):
            r = np.zeros((3, n, 4), np.int64)
            for k, (items, off, q) in enumerate(plans):
                cost = items[:, I["COST"]].astype(float)
                hd, qt = items[:, I["HEAD"]], items[:, I["QT"]]
                if used is not None:
                    cost = cost / used[k, hd, qt]
                t = cost * true_scale[k, hd, qt]
                for v in range(n):
                    x = (v + c) % 8
                    r[k, v, 0] = 100
                    r[k, v, 1] = 100 + int(round(t[q[off[v]:off[v + 1]]].sum() / true_speed[k, x]))
                    r[k, v, 2] = x
            for v in range(n):
                x = (v + c) % 8
                r[2, v, :3] = (100, 100 + int(round(loads_kv[v] / true_speed[2, x])), x)
            runs.append(r)
        return runs

    base, _ = skv.skv_schedule_build(prob, 64)
    sp1, sc1 = skv.calibrate_from_stamps([(base, stamps(base, None), None)], ridge=1e-4)
    second, _ = skv.skv_schedule_build_xcd(prob, 64, sp1, sc1)
    data = [(base, stamps(base, None), None), (second, stamps(second, sc1), sc1)]
    sp, sc = skv.calibrate_from_stamps(data, ridge=1e-4)
    # dK/dV (whose stamps include items taken from other queues) gets dQ's
    assert np.array_equal(sp[2], sp[1])
    for k in (0, 1):
        # the scales' pattern (here each head ran on four XCDs, so heads and
        # XCDs are told apart) ...
        np.testing.assert_allclose(sc[k] / sc[k].mean(), true_scale[k] / true_scale[k].mean(),
                                   rtol=0.01)
        np.testing.assert_allclose(sp[k], true_speed[k] / true_speed[k].mean(), rtol=0.01)
        # ... and, with the speeds, every stamped queue time of both plans
        # up to one overall factor
        for image, runs, used in data:
            _, plans = skv._plan_sections(image)
            items, off, q = plans[k]
            cost = items[:, I["COST"]].astype(float)
            hd, qt = items[:, I["HEAD"]], items[:, I["QT"]]
            if used is not None:
                cost = cost / used[k, hd, qt]
            c_fit = cost * sc[k, hd, qt]
            for r in runs:
                x = r[k, :, 2] & 15
                pred = np.array([c_fit[q[off[v]:off[v + 1]]].sum() for v in range(len(x))])
                pred = pred / sp[k][x]
                got_t = (r[k, :, 1] - r[k, :, 0]).astype(float)
                ratio = got_t / pred
                assert ratio.max() / ratio.min() - 1 < 0.03, (k, ratio.min(), ratio.max())
    # the calibrated plan balances the true times at least as well
    def true_max(image, used):
        runs = stamps(image, used)[0]
        d = (runs[:2, :, 1] - runs[:2, :, 0]).astype(float)
        return d.max(1) / d.mean(1) - 1
    cal, _ = skv.skv_schedule_build_xcd(prob, 64, sp, sc)
    plain, _ = skv.skv_schedule_build_xcd(prob, 64, sp)
    assert np.all(true_max(cal, sc) <= true_max(plain, None) + 0.002)


def test_calibration_without_backward_stamps():
    """Stamps of forward-only steps (the dQ and dK/dV regions stay zero)
    calibrate the forward and leave dQ and dK/dV at speed 1 and scale 1,
    with no NaN."""
    w, g, prob = _case("ctx32k_q2k", 2, None, ctx=4096, anchor_lo=512, anchor_hi=4096,
                       blocks_per_seq=16)
    image, _ = skv.skv_schedule_build(prob, 64)
    loads = skv.queue_loads(image)
    true = 1.0 + 0.05 * np.cos(np.arange(8))
    r = np.zeros((3, 64, 4), np.int64)
    for v in range(64):
        r[0, v] = (10, 10 + int(round(1e3 * loads[0, v] / true[v % 8])), v % 8, 0)
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        sp, sc = skv.calibrate_from_stamps([(image, [r, r], None)])
    assert np.all(np.isfinite(sp)) and np.all(np.isfinite(sc))
    np.testing.assert_allclose(sp[0], true / true.mean(), rtol=0.01)
    assert np.all(sp[1:] == 1.0) and np.all(sc[1] == 1.0)


@pytest.mark.parametrize("xcd", [False, True])
def test_kv_suffix_costs_and_claim_counters(xcd):
    """The dK/dV kernel claims its items at run time by the image's suffix
    costs: per queue position, the summed cost of that position and the rest
    of its queue; the backward workspace holds one claim counter per queue
    beyond the statistics and dQ's slots."""
    w, g, prob = _case("varlen8_fwdbwd", 3, None, len_median=2048, len_min=512, len_max=8192)
    if xcd:
        image, info = skv.skv_schedule_build_xcd(prob, 64, _speeds(4, 0.05))
    else:
        image, info = skv.skv_schedule_build(prob, 64)
    h, tiles, items, kv, fq, kq = _decode(image)
    suf = image[h["OFF_KVSUF"]: h["OFF_KVSUF"] + h["NKV"]]
    qoff = image[h["OFF_KVQOFF"]: h["OFF_KVQOFF"] + h["NWG"] + 1]
    cost = kv[:, K["COST"]].astype(np.int64)
    for v, q in enumerate(kq):
        want = np.cumsum(cost[q][::-1])[::-1]
        assert np.array_equal(suf[qoff[v]:qoff[v + 1]], want)
    G = w.hq // w.hkv
    stat = -(-(w.hkv * (w.nq * G + 64) * 4) // 256) * 256
    dq = -(-(info.n_dq_partial_slots * QTILE * w.d * 4) // 256) * 256
    front = -(-(64 * 4) // 256) * 256
    assert info.bwd_workspace_bytes == 4 * stat + dq + front + (256 if xcd else 0)
