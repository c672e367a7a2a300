"""GPU checks of schedules planned for per-XCD speeds and measured cost
scales (skv_schedule_build_xcd): workgroups claim queues by the XCD they
run on, every queue runs exactly once, and the forward, backward (through
dQ's own plan) and allocation-free forward match the oracle as with the
uniform plan."""
import numpy as np
import pytest
import torch

from block_sparse_split_amd import splitkv as skv
from block_sparse_split_amd import shards
from block_sparse_split_amd import workloads as wl
from gpu_util import announce, compare, gpu_fwd, oracle_partial, to_dev
from test_bwd_gpu import check_grad, oracle_fwd_bwd

pytestmark = pytest.mark.gpu


def _small(seed, **over):
    base = dict(ctx=4096, anchor_lo=1024, anchor_hi=4096, blocks_per_seq=16)
    base.update(over)
    return wl.make(wl.scaled(wl.WORKLOADS["ctx32k_q2k"], **base), seed, with_grad=True)


def _speeds(seed):
    rng = np.random.default_rng(seed)
    return (1.0 + 0.08 * rng.uniform(-1, 1, (3, 8))).astype(np.float32)


def _run(w, t, sh, noalloc=False):
    dt = w.dtype
    Q, K, V = to_dev(t.Q, dt), to_dev(t.K, dt), to_dev(t.V, dt)
    Kd, Vd, dO = to_dev(t.Kd, dt), to_dev(t.Vd, dt), to_dev(t.dO, dt)
    O = torch.full((w.nq, w.hq, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    LSE = torch.full((w.nq, w.hq), float("nan"), device="cuda")
    dQ = torch.full((w.nq, w.hq, w.d), float("nan"), device="cuda")
    dK, dV = torch.full_like(K, float("nan")), torch.full_like(V, float("nan"))
    dKd, dVd = torch.full_like(Kd, float("nan")), torch.full_like(Vd, float("nan"))
    if noalloc:
        sh.fwd_noalloc(Q, K, V, Kd, Vd, O, LSE)
    else:
        sh.fwd(Q, K, V, Kd, Vd, O, LSE)
    sh.bwd(Q, K, V, Kd, Vd, O, dO, LSE, dQ, dK, dV, dKd, dVd, skv.SKV_BF16)
    torch.cuda.synchronize()
    return O, LSE, dQ, dK, dV, dKd, dVd


@pytest.mark.parametrize("seed,n_wg,scaled", [(1, 256, False), (2, 64, True), (3, 8, True)])
def test_xcd_plan_forward_backward_parity(seed, n_wg, scaled):
    """Forward (and its allocation-free form) and backward through an XCD
    plan (with cost scales: other cuts and queues) against the oracle;
    every queue of the three kernels is stamped exactly once (each
    workgroup stamps the queue it claimed), so none was skipped."""
    w, g, t = _small(seed)
    prob = shards.whole_context_problem(w, g)
    scale = None
    if scaled:
        rng = np.random.default_rng(seed + 100)
        scale = rng.uniform(0.7, 1.4, (2, w.hkv, prob.qt_per_head))
    sh = skv.Shard(prob, n_workgroups=n_wg, xcd_speed=_speeds(seed), cost_scale=scale)
    assert sh.info.xcd_mode == 1
    announce("xcd plan parity", seed, n_wg, scaled)
    clk = torch.zeros(3 * n_wg * 4, dtype=torch.int64, device="cuda")
    skv.skv_timing_wg_clock(clk)
    try:
        got = _run(w, t, sh)
    finally:
        skv.skv_timing_wg_clock(None)
    st = clk.view(3, n_wg, 4).cpu().numpy()
    assert np.all(st[:, :, 0] > 0) and np.all(st[:, :, 1] >= st[:, :, 0])
    print("[xcd] queues run on their own XCD:",
          float(np.mean((st[:, :, 2] & 15) == np.arange(n_wg) % 8)), flush=True)
    Oo, Lo, want = oracle_fwd_bwd(w, g, t, np.arange(len(g.chunk_pos)), True)
    compare(got[0], got[1], Oo, Lo, "bf16", "xcd plan forward")
    for name, a, b in zip(("dQ", "dK", "dV", "dKd", "dVd"), got[2:], want):
        check_grad(a, b, f"xcd plan {name}")
    # twice in a row (the counters are zeroed before every launch), and the
    # allocation-free forward, give the same bits
    again = _run(w, t, sh)
    free = _run(w, t, sh, noalloc=True)
    for x, y, z in zip(got, again, free):
        assert torch.equal(x, y) and torch.equal(x, z)


def test_xcd_plan_shard_partials():
    """A context-parallel shard (no draft keys) planned per XCD: its
    partial output and LSE against the oracle's partial attention."""
    w = wl.scaled(wl.WORKLOADS["cp64_rank0_ctx512k"], ctx=8192, anchor_lo=2048,
                  anchor_hi=8192, blocks_per_seq=8, chunk=512, n_shards=4)
    w, g, t = wl.make(w, 6)
    ids, _, _, _ = shards.lpt_shards(w, g, w.n_shards)
    prob = shards.shard_problem(w, g, ids[2], False)
    sh = skv.Shard(prob, n_workgroups=32, xcd_speed=_speeds(7))
    announce("xcd plan shard partial")
    O, L, _ = gpu_fwd(w, g, t, ids[2], False, shard=sh)
    Oo, Lo = oracle_partial(w, g, t, ids[2], False)
    compare(O, L, Oo, Lo, "bf16", "xcd shard")


@pytest.mark.parametrize("layout", ["one_queue", "reversed"])
def test_dkdv_items_claimed_across_queues(layout):
    """The dK/dV kernel claims items of other queues once its own is done,
    and an item's outputs do not depend on the workgroup that runs it: with
    every dK/dV item moved into queue 0 (the other workgroups find their
    queues empty at once and take everything from it) or with the queues
    reversed, dK, dV, dKd, dVd and dQ are bit-identical to the planned
    queues'."""
    from block_sparse_split_amd.csrc_layout import H, K as KW, K_WORDS
    w, g, t = _small(4)
    prob = shards.whole_context_problem(w, g)
    sh = skv.Shard(prob, n_workgroups=16)
    announce("dkdv claims across queues", layout)
    ref = _run(w, t, sh)
    img = sh.image.copy()
    h = {k: int(img[v]) for k, v in H.items()}
    n, nkv = h["NWG"], h["NKV"]
    qoff = img[h["OFF_KVQOFF"]: h["OFF_KVQOFF"] + n + 1].copy()
    queue = img[h["OFF_KVQUEUE"]: h["OFF_KVQUEUE"] + nkv].copy()
    cost = img[h["OFF_KV"]: h["OFF_KV"] + nkv * K_WORDS].reshape(-1, K_WORDS)[:, KW["COST"]]
    qs = [list(queue[qoff[v]:qoff[v + 1]]) for v in range(n)]
    if layout == "one_queue":
        qs = [[i for q in qs for i in q]] + [[] for _ in range(n - 1)]
    else:
        qs = qs[::-1]
    pos = 0
    for v in range(n):
        img[h["OFF_KVQOFF"] + v] = pos
        for i in qs[v]:
            img[h["OFF_KVQUEUE"] + pos] = i
            pos += 1
        # suffix costs of the new queue
        rest = 0
        for j in range(pos - 1, img[h["OFF_KVQOFF"] + v] - 1, -1):
            rest += int(cost[img[h["OFF_KVQUEUE"] + j]])
            img[h["OFF_KVSUF"] + j] = rest
    img[h["OFF_KVQOFF"] + n] = pos
    assert pos == nkv
    sh.schedule = torch.from_numpy(img).to(sh.schedule.device)
    got = _run(w, t, sh)
    for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV", "dKd", "dVd"), ref, got):
        assert torch.equal(x, y), name


def test_xcd_plan_empty_and_draft_only_shards():
    """Per-XCD plans of shards without context keys: the empty shard has no
    dK/dV item at all (every workgroup finds nothing to claim) and adds
    nothing to dQ; the draft-only shard's dQ share and draft-key gradients
    match the oracle."""
    from test_bwd_gpu import gpu_bwd, oracle_fwd_bwd as ofb
    w, g, t = _small(9, blocks_per_seq=4)
    allc = np.arange(len(g.chunk_pos))
    O, L, _ = ofb(w, g, t, allc, True)
    Od = to_dev(wl.round_to_bf16(O.astype(np.float32)), "bf16")
    Ld = torch.from_numpy(L.astype(np.float32)).cuda()
    announce("xcd plan empty shard")
    dQ, dK, dV, _, _ = gpu_bwd(w, g, t, [], False, Od, Ld, n_wg=16, xcd_speed=_speeds(9))
    assert dK.shape[0] == 0 and torch.all(dQ == 0)
    announce("xcd plan draft-only shard")
    dQ, _, _, dKd, dVd = gpu_bwd(w, g, t, [], True, Od, Ld, n_wg=16, xcd_speed=_speeds(10))
    _, _, (wq, _, _, wkd, wvd) = ofb(w, g, t, [], True)
    check_grad(dQ, wq, "xcd draft-only dQ share")
    check_grad(dKd, wkd, "xcd draft-only dKd")
    check_grad(dVd, wvd, "xcd draft-only dVd")
