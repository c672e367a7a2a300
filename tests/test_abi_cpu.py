"""CPU checks of the C-ABI library: exports, argument errors, the planner
(bit-exact against the oracle) and the in-GPU schedule (coverage checked
with the oracle's tile visibility; placement re-derived from units built
with it).  No device call is made here."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from block_sparse_split_amd import splitkv as skv
from block_sparse_split_amd import workloads as wl
from block_sparse_split_amd import shards
from block_sparse_split_amd.csrc_layout import (H, T_WORDS, I_WORDS, S_WORDS, K_WORDS,
                                                QTILE, TILE_K, BLOCK)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "splitkv.h")


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const char\*|int32_t|skv_status)\s+(skv_\w+)\(",
                              text, re.M))
    assert {"skv_plan_lpt", "skv_attn_fwd_partial", "skv_merge_lse",
            "skv_attn_bwd"} <= declared
    out = subprocess.run(["nm", "-D", "--defined-only", skv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (skv_\w+)$", out, re.M))
    assert declared <= exported, declared - exported
    L = skv.lib()
    for name in declared:
        assert hasattr(L, name)
    assert L.skv_abi_version() == 4


def test_invalid_arguments_return_status_codes():
    L = skv.lib()
    assert L.skv_plan_lpt_costs(None, 3, 2, None, None) == -1
    assert b"NULL" in L.skv_last_error()
    with pytest.raises(skv.SplitKVError) as e:
        skv.skv_plan_lpt_costs([1, -2, 3], 2)
    assert e.value.status == -1
    with pytest.raises(skv.SplitKVError):
        skv.skv_plan_lpt_costs([1, 2], 0)
    with pytest.raises(skv.SplitKVError):
        skv.skv_chunk_costs([5], [0], [0], [0], 4)  # empty chunk
    with pytest.raises(skv.SplitKVError):
        skv.skv_chunk_costs([5], [6], [0], [4], 4)  # lo > anchor
    # problem validation
    base = dict(nb=1, hq=4, hkv=2, d=128, scale=0.1, dtype=skv.SKV_BF16, anchors=[10],
                lo=[0], chunk_pos=[0], chunk_off=[0, 64])
    for bad, status in [(dict(hq=3), -1), (dict(hq=6, hkv=2), -2), (dict(d=96), -2),
                        (dict(scale=0.0), -1), (dict(dtype=7), -2),
                        (dict(chunk_off=[1, 64]), -1),
                        # a chunk whose last key lies past INT32_MAX
                        (dict(chunk_pos=[2**31 - 32]), -1),
                        (dict(chunk_pos=[0, 32], chunk_off=[0, 64, 128]), -1)]:
        kw = dict(base, **bad)
        with pytest.raises(skv.SplitKVError) as e:
            skv.skv_schedule_build(skv.Problem(**kw), 8)
        assert e.value.status == status, bad
    # merge argument checks need no device
    assert L.skv_merge_lse(0, 4, 128, None, 1, None, None, 1, None, None) == -1
    assert L.skv_merge_lse(2, 4, 96, None, 1, None, None, 1, None, None) == -2
    assert L.skv_merge_lse(2, 0, 128, None, 1, None, None, 1, None, None) == 0
    # dQ finalize argument checks need no device either
    V = ctypes.c_void_p
    assert L.skv_dq_finalize(0, 64, V(4096), 64, V(8192), 1, None) == -1       # no shares
    assert L.skv_dq_finalize(2, 64, V(4096), 64, V(8192), 9, None) == -2       # out dtype
    assert L.skv_dq_finalize(2, 64, V(4096), 66, V(1 << 20), 1, None) == -1    # stride % 4
    assert L.skv_dq_finalize(2, 64, V(4096), 32, V(1 << 20), 1, None) == -1    # stride < elems
    assert L.skv_dq_finalize(2, 64, V(4100), 64, V(1 << 20), 1, None) == -1    # misaligned
    assert L.skv_dq_finalize(2, 64, V(4096), 64, V(4096 + 256), 1, None) == -1  # overlap
    assert L.skv_dq_finalize(2, 64, V(4096), 64, V(4096), 1, None) == -1       # bf16 in place
    assert L.skv_dq_finalize(2, 64, None, 64, V(8192), 1, None) == -1          # NULL
    assert L.skv_dq_finalize(3, 0, None, 0, None, 1, None) == 0                # nothing to do


def test_error_text_clears_after_success():
    L = skv.lib()
    L.skv_plan_lpt_costs(None, 3, 2, None, None)
    skv.skv_plan_lpt_costs([1, 2, 3], 2)
    assert L.skv_last_error() == b""


@pytest.mark.parametrize("name,seed", [("tiny_f32_ctx1k", 0), ("tiny_f32_ctx1k", 5),
                                       ("ctx32k_q2k", 1), ("cp64_rank0_ctx512k", 2),
                                       ("varlen8_fwdbwd", 3), ("ctx1m_merge64", 4)])
def test_chunk_costs_and_lpt_bit_exact_vs_oracle(name, seed):
    w, g, _ = wl.make(name, seed, tensors=False)
    bins_list = [w.n_shards, 256] if w.n_shards > 1 else [256, 64]
    c_lib = skv.skv_chunk_costs(g.anchors, g.lo, g.chunk_pos, g.chunk_len, w.tile_k)
    c_or = oracle.chunk_costs(g.anchors, g.lo, g.chunk_pos, g.chunk_len, w.tile_k)
    np.testing.assert_array_equal(c_lib, c_or)
    for m in bins_list:
        b_lib, cost, load = skv.skv_plan_lpt(g.anchors, g.lo, g.chunk_pos, g.chunk_len,
                                            w.tile_k, m)
        b_or, load_or = oracle.plan_lpt(c_or, m)
        np.testing.assert_array_equal(b_lib, b_or)
        np.testing.assert_array_equal(load, load_or)
        np.testing.assert_array_equal(cost, c_or)


def test_chunk_costs_random_blocks_bit_exact_vs_oracle():
    """Random visible intervals, including empty ones (lo = anchor), ones
    that start inside a tile and unsorted blocks, against chunks of random
    lengths and positions (overlapping, ragged) and several tile sizes."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        nb = int(rng.integers(0, 40))
        L = int(rng.integers(1, 2000))
        lo = rng.integers(0, L, size=nb)
        an = np.minimum(lo + rng.integers(0, L // 2 + 1, size=nb), L)
        empty = rng.random(nb) < 0.2
        an[empty] = lo[empty]
        n = int(rng.integers(0, 30))
        pos = rng.integers(0, L + 50, size=n)
        ln = rng.integers(1, 300, size=n)
        tk = int(rng.choice([1, 7, 16, 64, 100]))
        got = skv.skv_chunk_costs(an, lo, pos, ln, tk)
        want = oracle.chunk_costs(an, lo, pos, ln, tk)
        np.testing.assert_array_equal(got, want)


def test_workgroup_clock_buffer_arguments():
    L = skv.lib()
    assert L.skv_timing_wg_clock(ctypes.c_void_p(8 * 1000 + 4), 64) == -1  # misaligned
    assert L.skv_timing_wg_clock(ctypes.c_void_p(8 * 1000), -1) == -1
    assert L.skv_timing_wg_clock(None, 0) == 0  # off (no device access either way)
    # a host pointer is refused (the kernels would store to it)
    host = (ctypes.c_uint64 * 64)()
    assert L.skv_timing_wg_clock(ctypes.cast(host, ctypes.c_void_p), 512) == -1
    assert L.skv_timing_wg_clock(None, 0) == 0
    import torch
    with pytest.raises(ValueError):
        skv.skv_timing_wg_clock(torch.zeros(64, dtype=torch.int64))  # not a device tensor


def test_lpt_costs_random_bit_exact():
    rng = np.random.default_rng(0)
    for _ in range(50):
        n = int(rng.integers(0, 300))
        m = int(rng.integers(1, 40))
        costs = rng.integers(0, int(rng.integers(1, 50)), size=n)  # many ties
        b, ld = skv.skv_plan_lpt_costs(costs, m)
        bo, lo_ = oracle.plan_lpt(costs, m)
        np.testing.assert_array_equal(b, bo)
        np.testing.assert_array_equal(ld, lo_)


def test_lpt_deterministic_across_calls():
    w, g, _ = wl.make("ctx1m_merge64", 4, tensors=False)
    a = skv.skv_plan_lpt(g.anchors, g.lo, g.chunk_pos, g.chunk_len, 64, 256)
    b = skv.skv_plan_lpt(g.anchors, g.lo, g.chunk_pos, g.chunk_len, 64, 256)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ------------------------------------------------------------------ schedule

def _decode(image):
    h = {k: int(image[v]) for k, v in H.items()}
    tiles = image[h["OFF_TILES"]: h["OFF_TILES"] + h["NTILES"] * T_WORDS].reshape(-1, T_WORDS)
    items = image[h["OFF_ITEMS"]: h["OFF_ITEMS"] + h["NITEMS"] * I_WORDS].reshape(-1, I_WORDS)
    qoff = image[h["OFF_QOFF"]: h["OFF_QOFF"] + h["NWG"] + 1]
    queue = image[h["OFF_QUEUE"]: h["OFF_QUEUE"] + h["NITEMS"]]
    split = image[h["OFF_SPLIT"]: h["OFF_SPLIT"] + h["NSPLIT"] * S_WORDS].reshape(-1, S_WORDS)
    kv = image[h["OFF_KV"]: h["OFF_KV"] + h["NKV"] * K_WORDS].reshape(-1, K_WORDS)
    kvqoff = image[h["OFF_KVQOFF"]: h["OFF_KVQOFF"] + h["NWG"] + 1]
    kvqueue = image[h["OFF_KVQUEUE"]: h["OFF_KVQUEUE"] + h["NKV"]]
    return h, tiles, items, qoff, queue, split, kv, kvqoff, kvqueue


def _check_lpt_per_class(costs, heads, qoff, queue, n_wg, n_cls):
    """Re-derive the per-XCD-class LPT with the oracle and compare queues."""
    per = n_wg // n_cls
    for c in range(n_cls):
        ids = np.nonzero(heads % n_cls == c)[0]
        bins, _ = oracle.plan_lpt(costs[ids], per)
        order = sorted(range(len(ids)), key=lambda j: (-int(costs[ids[j]]), j))
        want = {c + b * n_cls: [] for b in range(per)}
        for j in order:
            want[c + int(bins[j]) * n_cls].append(int(ids[j]))
        for wgi, lst in want.items():
            assert queue[qoff[wgi]:qoff[wgi + 1]].tolist() == lst


STEP_COST, ITEM_COST = 8, 44  # time units of a key step and of an item's fixed part


def _fwd_items_via_split_plan(w, g, tiles, n_wg, n_cls, with_draft):
    """The forward item plan re-derived from its parts: units from the
    oracle's tile visibility (per kv head and query tile, runs of
    consecutive tiles that some anchor block of the query tile sees; a query
    tile that sees none still makes one empty unit; the first run carries
    the draft steps, one per 64 draft keys), placed per XCD class by
    skv_plan_lpt_split, which tests/test_plan_split_cpu.py pins on its own.
    Returns the items (head, qt, t0, t1, flags, cost) in emission order, the
    per-workgroup queues and each class's target."""
    G = w.hq // w.hkv
    tpq = QTILE // G
    qtph = -(-w.nq * G // QTILE)
    units = []  # (head, qt, tiles of the run, draft cost)
    for h in range(w.hkv):
        for qt in range(qtph):
            b0 = qt * tpq // BLOCK
            b1 = min(w.nb, -(-((qt + 1) * tpq) // BLOCK))
            vis = [i for i, t in enumerate(tiles)
                   if oracle.tile_pairs_visible(g.anchors[b0:b1], g.lo[b0:b1], t[1],
                                                t[1] + t[2]) > 0]
            dc = STEP_COST * -(-((b1 - b0) * BLOCK) // 64) if with_draft else 0
            runs = np.split(np.array(vis, np.int64),
                            np.nonzero(np.diff(vis) != 1)[0] + 1) if vis else [[]]
            for j, r in enumerate(runs):
                units.append((h, qt, list(r), dc if j == 0 else 0))
    per = n_wg // n_cls
    items, queues, targets = [], [[] for _ in range(n_wg)], []
    for c in range(n_cls):
        ids = [i for i, u in enumerate(units) if u[0] % n_cls == c]
        pieces, cost, target, _ = skv.skv_plan_lpt_split(
            [units[i][3] for i in ids], [len(units[i][2]) for i in ids], ITEM_COST, STEP_COST,
            per, 0)
        targets.append(target)
        for (u, k0, k1, b), cst in zip(pieces.tolist(), cost.tolist()):
            h, qt, run, dc = units[ids[u]]
            t0, t1 = (run[k0], run[k1 - 1] + 1) if k1 > k0 else (0, 0)
            flags = 1 if (k0 == 0 and with_draft and dc > 0) else 0
            queues[c + b * n_cls].append(len(items))
            items.append((h, qt, t0, t1, flags, cst))
    return items, queues, targets


def _schedule_case(name, seed, shard_of=None, n_wg=256, **over):
    w = wl.scaled(wl.WORKLOADS[name], **over) if over else wl.WORKLOADS[name]
    w, g, _ = wl.make(w, seed, tensors=False)
    if shard_of is None:
        prob = shards.whole_context_problem(w, g)
        pos = np.arange(g.ctx)
    else:
        ids, _, _, _ = shards.lpt_shards(w, g, w.n_shards)
        chunk_ids = ids[shard_of]
        prob = shards.shard_problem(w, g, chunk_ids, shard_of == 0)
        pos = shards.shard_rows(g, chunk_ids)
    image, info = skv.skv_schedule_build(prob, n_wg)
    return w, g, prob, pos, image, info


@pytest.mark.parametrize("case", [
    ("ctx32k_q2k", 1, None, 256, {}),
    ("ctx32k_q2k", 2, None, 40, dict(ctx=4096, anchor_lo=512, anchor_hi=4096, blocks_per_seq=16)),
    ("varlen8_fwdbwd", 3, None, 256, dict(len_median=2048, len_min=512, len_max=8192)),
    # G = 16 (one anchor block per query tile) and G = 2 (eight)
    ("ctx32k_q2k", 3, None, 64, dict(ctx=4096, anchor_lo=512, anchor_hi=4096, blocks_per_seq=24,
                                     hq=32, hkv=2)),
    ("ctx32k_q2k", 4, None, 48, dict(ctx=4096, anchor_lo=512, anchor_hi=4096, blocks_per_seq=24,
                                     hq=16, hkv=8)),
    ("cp64_rank0_ctx512k", 2, 0, 256, {}),
    ("cp64_rank0_ctx512k", 2, 5, 256, {}),
    ("tiny_f32_ctx1k", 0, 1, 8, {}),
    ("tiny_f32_ctx1k", 0, 0, 3, {}),
])
def test_whole_row_tiles_of_dkdv_items_need_no_mask(case):
    """Each context dK/dV item marks the run of its 64-row tiles [w0, w1)
    whose rows all see every key of the item, so the kernel skips the
    per-row intervals and masks there: each such tile must lie inside the
    item's rows, and every anchor block it covers must see the item's whole
    key range."""
    name, seed, shard_of, n_wg, over = case
    w, g, prob, pos, image, info = _schedule_case(name, seed, shard_of, n_wg, **over)
    h, tiles, items, qoff, queue, split, kv, kvqoff, kvqueue = _decode(image)
    G = w.hq // w.hkv
    rpb = BLOCK * G
    n_whole = n_rt_all = 0
    for k in kv:
        hd, t0, nt, dtok0, nd, b0, b1, cost, whole = (int(x) for x in k)
        w0, w1 = whole & 0xFFFF, whole >> 16
        r_begin, r_end = b0 * rpb, b1 * rpb
        n_rt = -(-max(0, r_end - r_begin) // TILE_K)
        assert w0 <= w1 <= n_rt
        if nd > 0:
            assert whole == 0
            continue
        if w1 > w0:
            kmin = int(tiles[t0][1])
            kend = int(tiles[t0 + nt - 1][1]) + int(tiles[t0 + nt - 1][2])
            for rt in range(w0, w1):
                r0 = r_begin + TILE_K * rt
                assert r0 + TILE_K <= r_end
                for b in range(r0 // rpb, (r0 + TILE_K - 1) // rpb + 1):
                    assert g.lo[b] <= kmin and g.anchors[b] >= kend
        n_whole += w1 - w0
        n_rt_all += n_rt
    if name == "ctx32k_q2k" and not over:
        assert n_whole > 0.8 * n_rt_all


@pytest.mark.parametrize("case", [
    ("ctx32k_q2k", 1, None, 256, {}),
    ("ctx32k_q2k", 2, None, 40, dict(ctx=4096, anchor_lo=512, anchor_hi=4096, blocks_per_seq=16)),
    ("varlen8_fwdbwd", 3, None, 256, dict(len_median=2048, len_min=512, len_max=8192)),
    # G = 16 (one anchor block per query tile) and G = 2 (eight)
    ("ctx32k_q2k", 3, None, 64, dict(ctx=4096, anchor_lo=512, anchor_hi=4096, blocks_per_seq=24,
                                     hq=32, hkv=2)),
    ("ctx32k_q2k", 4, None, 48, dict(ctx=4096, anchor_lo=512, anchor_hi=4096, blocks_per_seq=24,
                                     hq=16, hkv=8)),
    ("cp64_rank0_ctx512k", 2, 0, 256, {}),
    ("cp64_rank0_ctx512k", 2, 5, 256, {}),
    ("tiny_f32_ctx1k", 0, 1, 8, {}),
    ("tiny_f32_ctx1k", 0, 0, 3, {}),
    # one workgroup, one anchor block near the end of a 2.1M-key context:
    # each item has more than 2^15 steps, too many to mark
    ("ctx32k_q2k", 5, None, 1, dict(ctx=2162688, anchor_lo=2162600, anchor_hi=2162688,
                                    blocks_per_seq=1, hq=1, hkv=1)),
])
def test_whole_step_ranges_need_no_mask(case):
    """Each item marks the run of its steps [s0, s1) that every row of its
    query tile sees whole, so the kernels skip bounds and masks there: each
    such step must be a full 64-key context tile inside every anchor block's
    interval [lo, anchor)."""
    name, seed, shard_of, n_wg, over = case
    w, g, prob, pos, image, info = _schedule_case(name, seed, shard_of, n_wg, **over)
    h, tiles, items, *_ = _decode(image)
    G = w.hq // w.hkv
    tpq = QTILE // G
    n_whole = 0
    for it in items:
        hd, qt, t0, t1, slot, flags, cost, whole = (int(x) for x in it)
        # the kernels decode the high half with a signed shift
        assert 0 <= whole < 2 ** 31
        s0, s1 = whole & 0xFFFF, whole >> 16
        if t1 - t0 >= 2 ** 15:
            assert whole == 0
        b0 = qt * tpq // BLOCK
        b1 = min(w.nb, -(-((qt + 1) * tpq) // BLOCK))
        dtok0 = b0 * BLOCK
        dtok1 = min(w.nq, b1 * BLOCK)
        nd = -(-(dtok1 - dtok0) // TILE_K) if flags & 1 else 0
        assert s0 <= s1 <= nd + t1 - t0
        if s1 > s0:
            assert s0 >= nd
        for s in range(s0, s1):
            t = t0 + s - nd
            p0, n = int(tiles[t][1]), int(tiles[t][2])
            assert n == TILE_K
            assert all(g.lo[b] <= p0 and p0 + n <= g.anchors[b] for b in range(b0, b1))
        n_whole += s1 - s0
    # most steps of the long-context workloads are whole
    if name in ("ctx32k_q2k", "cp64_rank0_ctx512k") and not over:
        n_ctx = sum(int(it[3]) - int(it[2]) for it in items)
        assert n_whole > 0.8 * n_ctx


@pytest.mark.parametrize("case", [
    ("ctx32k_q2k", 1, None, 256, {}),
    ("ctx32k_q2k", 2, None, 40, dict(ctx=4096, anchor_lo=512, anchor_hi=4096, blocks_per_seq=16)),
    ("varlen8_fwdbwd", 3, None, 256, dict(len_median=2048, len_min=512, len_max=8192)),
    # G = 16 (one anchor block per query tile) and G = 2 (eight)
    ("ctx32k_q2k", 3, None, 64, dict(ctx=4096, anchor_lo=512, anchor_hi=4096, blocks_per_seq=24,
                                     hq=32, hkv=2)),
    ("ctx32k_q2k", 4, None, 48, dict(ctx=4096, anchor_lo=512, anchor_hi=4096, blocks_per_seq=24,
                                     hq=16, hkv=8)),
    ("cp64_rank0_ctx512k", 2, 0, 256, {}),
    ("cp64_rank0_ctx512k", 2, 5, 256, {}),
    ("tiny_f32_ctx1k", 0, 1, 8, {}),
    ("tiny_f32_ctx1k", 0, 0, 3, {}),
])
def test_schedule_covers_visible_work_once_and_is_lpt(case):
    name, seed, shard_of, n_wg, over = case
    w, g, prob, pos, image, info = _schedule_case(name, seed, shard_of, n_wg, **over)
    h, tiles, items, qoff, queue, split, kv, kvqoff, kvqueue = _decode(image)
    assert h["MAGIC"] == 0x314B5653 and h["NWG"] == n_wg
    G = w.hq // w.hkv
    # tiles: sorted, non-overlapping, rows map to the right absolute keys
    assert np.all(np.diff(tiles[:, 1]) > 0)
    for t in tiles:
        assert np.array_equal(pos[t[0]:t[0] + t[2]], np.arange(t[1], t[1] + t[2]))
    assert tiles[:, 2].sum() == len(pos)
    # every (kv head, query tile, visible tile) appears in exactly one item
    rows = w.nq * G
    qtph = -(-rows // QTILE)
    seen = np.zeros((w.hkv, qtph, len(tiles)), np.int32)
    draft_seen = np.zeros((w.hkv, qtph), np.int32)
    for it in items:
        hd, qt, t0, t1, slot, flags, cost = it[:7]
        seen[hd, qt, t0:t1] += 1
        draft_seen[hd, qt] += flags & 1
        # the item cost: its fixed part plus one step per tile and per 64
        # draft keys; every tile of the run is one some block sees
        b0 = qt * (QTILE // G) // BLOCK
        b1 = min(w.nb, -(-((qt + 1) * (QTILE // G)) // BLOCK))
        assert all(oracle.tile_pairs_visible(g.anchors[b0:b1], g.lo[b0:b1], tiles[t, 1],
                                             tiles[t, 1] + tiles[t, 2]) > 0 for t in range(t0, t1))
        want = ITEM_COST + STEP_COST * (t1 - t0)
        want += STEP_COST * -(-((b1 - b0) * BLOCK) // 64) if flags & 1 else 0
        assert cost == want
    for qt in range(qtph):
        b0 = qt * (QTILE // G) // BLOCK
        b1 = min(w.nb, -(-((qt + 1) * (QTILE // G)) // BLOCK))
        vis = np.array([oracle.tile_pairs_visible(g.anchors[b0:b1], g.lo[b0:b1], t[1],
                                                  t[1] + t[2]) > 0 for t in tiles], bool)
        for hd in range(w.hkv):
            assert np.array_equal(seen[hd, qt] > 0, vis)
            assert seen[hd, qt].max(initial=0) <= 1
            assert draft_seen[hd, qt] == int(prob.c.with_draft)
    # every query tile has at least one item; split tiles own consecutive slots
    per_qt = {}
    for it in items:
        per_qt.setdefault((it[0], it[1]), []).append(it[4])
    assert len(per_qt) == w.hkv * qtph
    nsl = 0
    for s in split:
        slots = sorted(per_qt[(s[0], s[1])])
        assert slots == list(range(s[2], s[2] + s[3]))
        nsl += s[3]
    assert nsl == info.n_partial_slots
    for k, v in per_qt.items():
        if len(v) == 1:
            assert v[0] == -1
    # queues: each item once, LPT per XCD class re-derived by the oracle
    assert sorted(queue.tolist()) == list(range(len(items)))
    want_items, want_q, _ = _fwd_items_via_split_plan(w, g, tiles, n_wg, h["NCLASS"],
                                                      prob.c.with_draft)
    assert len(want_items) == len(items)
    for got, want in zip(items, want_items):
        assert (got[0], got[1], got[2], got[3], got[5], got[6]) == want
    for wgi in range(n_wg):
        assert queue[qoff[wgi]:qoff[wgi + 1]].tolist() == want_q[wgi]
    _check_lpt_per_class(kv[:, 7].astype(np.int64), kv[:, 0], kvqoff, kvqueue, n_wg,
                         h["NCLASS"])
    loads = np.zeros(n_wg, np.int64)
    for wgi in range(n_wg):
        loads[wgi] = items[queue[qoff[wgi]:qoff[wgi + 1]], 6].sum()
    assert loads.max() == info.item_cost_max_bin and loads.sum() == info.item_cost_total
    # dK/dV items cover every tile once per kv head (+ draft groups)
    for hd in range(w.hkv):
        cover = np.zeros(len(tiles), np.int32)
        dcover = np.zeros(w.nq, np.int32)
        for k in kv[kv[:, 0] == hd]:
            cover[k[1]:k[1] + k[2]] += 1
            dcover[k[3]:k[3] + k[4]] += 1
            for t in range(k[1], k[1] + k[2]):
                vb = np.nonzero((np.maximum(g.lo, tiles[t, 1]) <
                                 np.minimum(g.anchors, tiles[t, 1] + tiles[t, 2])))[0]
                if vb.size:
                    assert k[5] <= vb.min() and vb.max() < k[6]
        assert np.all(cover == 1)
        assert np.all(dcover == int(prob.c.with_draft))


@pytest.mark.parametrize("name,seed", [("ctx32k_q2k", 1), ("ctx32k_q2k", 2),
                                       ("varlen8_fwdbwd", 1)])
def test_in_gpu_item_plan_imbalance_below_one_percent(name, seed):
    """Forward items and dK/dV items over 256 workgroups: max/mean - 1 < 1%."""
    w, g, prob, pos, image, info = _schedule_case(name, seed, None, 256)
    imb = info.item_cost_max_bin / (info.item_cost_total / 256) - 1
    kv_imb = info.kv_cost_max_bin / (info.kv_cost_total / 256) - 1
    assert imb < 0.01 and kv_imb < 0.01, (imb, kv_imb)


def test_device_calls_reject_misaligned_tensors_before_launch():
    """Tensors must be 16-byte aligned (LSE arrays 4-byte): a misaligned
    pointer is refused before any launch (the fake pointers are never
    dereferenced)."""
    import ctypes
    w, g, _ = wl.make("tiny_f32_ctx1k", 0, tensors=False)
    prob = shards.whole_context_problem(w, g)
    image, info = skv.skv_schedule_build(prob, 8)
    L = skv.lib()
    ok, bad8, bad2 = ctypes.c_void_p(256), ctypes.c_void_p(264), ctypes.c_void_p(258)
    # forward: K at an 8-byte boundary
    st = L.skv_attn_fwd_partial(ctypes.byref(prob.c), ctypes.byref(info), ok, ok, bad8, ok,
                                ok, ok, ok, 1, ok, ok, 1 << 30, None)
    assert st == -1 and b"16-byte aligned" in L.skv_last_error()
    # forward: LSE off a 4-byte boundary
    st = L.skv_attn_fwd_partial(ctypes.byref(prob.c), ctypes.byref(info), ok, ok, ok, ok,
                                ok, ok, ok, 1, bad2, ok, 1 << 30, None)
    assert st == -1 and b"4-byte aligned" in L.skv_last_error()
    # merge: O_out misaligned
    st = L.skv_merge_lse(2, 16, 64, ok, 1, ok, ctypes.c_void_p(1 << 20 | 8), 1, ok, None)
    assert st == -1 and b"16-byte aligned" in L.skv_last_error()
    # backward (bf16 problem): dK misaligned
    wb, gb, _ = wl.make("ctx32k_q2k", 1, tensors=False)
    wb = wl.scaled(wb, ctx=2048, anchor_lo=512, anchor_hi=2048, blocks_per_seq=8)
    wb, gb, _ = wl.make(wb, 0, tensors=False)
    pb = shards.whole_context_problem(wb, gb)
    _, ib = skv.skv_schedule_build(pb, 8)
    st = L.skv_attn_bwd(ctypes.byref(pb.c), ctypes.byref(ib), ok, ok, ok, ok, ok, ok, ok, ok,
                        ok, ok, bad8, ok, ok, ok, 0, ok, 1 << 40, None)
    assert st == -1 and b"16-byte aligned" in L.skv_last_error()


def test_device_calls_reject_bad_dtypes_before_launch():
    """Argument errors are returned before anything touches a device (the
    fake pointers below are never dereferenced)."""
    import ctypes
    w, g, _ = wl.make("tiny_f32_ctx1k", 0, tensors=False)
    prob = shards.whole_context_problem(w, g)
    image, info = skv.skv_schedule_build(prob, 8)
    L = skv.lib()
    fake = ctypes.c_void_p(256)
    st = L.skv_attn_fwd_partial(ctypes.byref(prob.c), ctypes.byref(info), fake, fake, fake, fake,
                                fake, fake, fake, 7, fake, fake, 1 << 30, None)
    assert st == -2 and b"o_dtype" in L.skv_last_error()
    # backward takes bf16 inputs only
    st = L.skv_attn_bwd(ctypes.byref(prob.c), ctypes.byref(info), fake, fake, fake, fake, fake,
                        fake, fake, fake, fake, fake, fake, fake, fake, fake, 0, fake, 1 << 30,
                        None)
    assert st == -2 and b"bf16" in L.skv_last_error()
    # a schedule built for another problem is refused
    prob2 = shards.shard_problem(w, g, [0, 1], False)
    st = L.skv_attn_fwd_partial(ctypes.byref(prob2.c), ctypes.byref(info), fake, fake, fake,
                                fake, fake, fake, fake, 1, fake, fake, 1 << 30, None)
    assert st == -1 and b"different problem" in L.skv_last_error()
    # workspace too small
    w1, g1, _ = wl.make("ctx32k_q2k", 1, tensors=False)
    p1 = shards.whole_context_problem(w1, g1)
    _, i1 = skv.skv_schedule_build(p1, 256)
    assert i1.fwd_workspace_bytes > 0
    st = L.skv_attn_fwd_partial(ctypes.byref(p1.c), ctypes.byref(i1), fake, fake, fake, fake,
                                fake, fake, fake, 1, fake, fake, 16, None)
    assert st == -4


def test_noalloc_forward_refuses_oversized_workspace_before_any_device_call():
    """The allocation-free forward holds 64 MiB of scratch; a schedule that
    needs more is refused with SKV_ERR_WORKSPACE and a message that names both
    sizes, before the library touches the device."""
    w, g, _ = wl.make("ctx32k_q2k", 1, tensors=False)
    prob = shards.whole_context_problem(w, g)
    _, info = skv.skv_schedule_build(prob, 256)
    assert info.fwd_workspace_bytes <= 64 << 20
    info.fwd_workspace_bytes = (64 << 20) + 256
    L = skv.lib()
    st = L.skv_attn_fwd_partial_noalloc(ctypes.byref(prob.c), ctypes.byref(info), None, None,
                                        None, None, None, None, None, skv.SKV_BF16, None, None)
    assert st == -4
    msg = L.skv_last_error().decode()
    assert str((64 << 20) + 256) in msg and str(64 << 20) in msg
