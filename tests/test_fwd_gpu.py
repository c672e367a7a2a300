"""GPU parity of the forward partial and the LSE merge against the fp64
oracle, element by element, through the C ABI (tolerances: fp32 path
max-abs 1e-5; bf16 path 2e-2 on O and 1e-3 on LSE)."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_split_amd import splitkv as skv
from block_sparse_split_amd import shards
from block_sparse_split_amd import workloads as wl
from gpu_util import (announce, block_rows, compare, gpu_fwd, measured_like_plan,
                      oracle_partial, rows_of, to_dev)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_f32_lpt_shards_then_merge(seed):
    """1K context, 8 chunks over 4 LPT shards (draft keys on shard 0); every
    partial and the 4-way merge against the oracle at 1e-5."""
    w, g, t = wl.make("tiny_f32_ctx1k", seed)
    ids, bins, cost, load = shards.lpt_shards(w, g, w.n_shards)
    b_or, _ = oracle.plan_lpt(oracle.chunk_costs(g.anchors, g.lo, g.chunk_pos, g.chunk_len,
                                                 w.tile_k), w.n_shards)
    np.testing.assert_array_equal(bins, b_or)
    Os, Ls = [], []
    for r in range(w.n_shards):
        announce("tiny_f32 shard", r, "seed", seed)
        O, L, _ = gpu_fwd(w, g, t, ids[r], r == 0)
        Oo, Lo = oracle_partial(w, g, t, ids[r], r == 0)
        compare(O, L, Oo, Lo, "f32", f"shard {r}")
        Os.append(O)
        Ls.append(L)
    Om = torch.empty_like(Os[0])
    Lm = torch.empty_like(Ls[0])
    announce("tiny_f32 merge")
    skv.skv_merge_lse(torch.stack(Os), torch.stack(Ls), Om, Lm)
    torch.cuda.synchronize()
    Of, Lf = oracle.attention(t.Q, t.K, t.V, t.Kd, t.Vd, g.anchors, g.lo,
                              wl.softmax_scale(w.d))
    compare(Om, Lm, Of, Lf, "f32", "merged")


def _small32k(seed, **over):
    base = dict(ctx=4096, anchor_lo=1024, anchor_hi=4096, blocks_per_seq=16)
    base.update(over)
    return wl.make(wl.scaled(wl.WORKLOADS["ctx32k_q2k"], **base), seed)


@pytest.mark.parametrize("seed,n_wg", [(0, 256), (1, 13), (2, 1), (3, 64)])
def test_bf16_whole_context_small(seed, n_wg):
    """4K context, 16 blocks, 32q/8kv, d=128: all rows, several workgroup
    counts (so query tiles are cut into items and merged in the library)."""
    w, g, t = _small32k(seed)
    allc = np.arange(len(g.chunk_pos))
    announce("bf16 small whole", seed, n_wg)
    O, L, sh = gpu_fwd(w, g, t, allc, True, n_wg=n_wg)
    Oo, Lo = oracle_partial(w, g, t, allc, True)
    compare(O, L, Oo, Lo, "bf16", "whole")
    # fp32 output of the same problem, and determinism across calls
    O2, L2, _ = gpu_fwd(w, g, t, allc, True, o_dtype=torch.float32, shard=sh)
    compare(O2, L2, Oo, Lo, "bf16", "whole fp32 out")
    O3, L3, _ = gpu_fwd(w, g, t, allc, True, o_dtype=torch.float32, shard=sh)
    assert torch.equal(O2, O3) and torch.equal(L2, L3)


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 64), (8, 4, 128), (16, 2, 64), (16, 1, 128),
                                       (6, 6, 128)])
def test_bf16_gqa_and_head_dims(hq, hkv, d):
    w, g, t = _small32k(7, hq=hq, hkv=hkv, d=d, ctx=2048, anchor_lo=100, anchor_hi=2048,
                        blocks_per_seq=9)
    allc = np.arange(len(g.chunk_pos))
    announce("bf16 gqa", hq, hkv, d)
    O, L, _ = gpu_fwd(w, g, t, allc, True, n_wg=32)
    Oo, Lo = oracle_partial(w, g, t, allc, True)
    compare(O, L, Oo, Lo, "bf16", f"G={hq // hkv} d={d}")


def test_f32_d128_and_ragged():
    w = wl.scaled(wl.WORKLOADS["tiny_f32_ctx1k"], hq=4, hkv=2, d=128, ctx=1000, chunk=100,
                  blocks_per_seq=5, anchor_lo=0, anchor_hi=1000)
    w, g, t = wl.make(w, 11)
    ids, _, _, _ = shards.lpt_shards(w, g, 3)
    for r in range(3):
        announce("f32 d128 ragged shard", r)
        O, L, _ = gpu_fwd(w, g, t, ids[r], r == 1, n_wg=5)
        Oo, Lo = oracle_partial(w, g, t, ids[r], r == 1)
        compare(O, L, Oo, Lo, "f32", f"shard {r}")


@pytest.mark.parametrize("d,n_wg", [(64, 1), (128, 7)])
def test_f32_wide_logits(d, n_wg):
    """The fp32 path under logits that grow along the context (key rows at
    position p scaled by 2^min(5, p // 300), exact in fp32), so each row's
    running maximum rises by tens of units (log2) inside one work item and
    the rescale of O runs mid-item.  The bar follows from the arithmetic:
    S sums d fp32 products, each rounded once, so it errs by at most eps_s =
    (d + 1) 2^-24 max|q| max|k|, a factor of at most 2^(c eps_s) on each
    weight in numerator and denominator; O and the sum add n fp32 terms
    each (n visible keys, at most (n - 1) 2^-24 of the sum of magnitudes);
    LSE errs by at most scale eps_s plus the sum's relative error.  A missed
    or wrong rescale is off by O(1)."""
    w = wl.scaled(wl.WORKLOADS["tiny_f32_ctx1k"], hq=4, hkv=2, d=d, ctx=2048, chunk=128,
                  blocks_per_seq=6, anchor_lo=256, anchor_hi=2048)
    w, g, t = wl.make(w, 12)
    pos = shards.shard_rows(g, t.chunk_ids)
    t.K *= (2.0 ** np.minimum(5, pos // 300)).astype(np.float32)[:, None, None]
    allc = np.arange(len(g.chunk_pos))
    announce("f32 wide logits", d, n_wg)
    O, L, _ = gpu_fwd(w, g, t, allc, True, n_wg=n_wg)
    Oo, Lo = oracle_partial(w, g, t, allc, True)
    assert np.nanmax(Lo) > 100.0
    scale = wl.softmax_scale(d)
    c = scale * np.log2(np.e)
    kmax = max(np.linalg.norm(t.K, axis=-1).max(), np.linalg.norm(t.Kd, axis=-1).max())
    eps_s = (d + 1) * 2.0 ** -24 * np.linalg.norm(t.Q, axis=-1).max() * kmax
    n = g.ctx + 16
    vmax = max(np.abs(t.V).max(), np.abs(t.Vd).max())
    sum_rel = (n - 1) * 2.0 ** -24
    o_bar = vmax * (2 * np.log(2) * c * eps_s + 2 * sum_rel) + 1e-6
    l_bar = scale * eps_s + sum_rel + 1e-6
    Og = O.cpu().numpy().astype(np.float64)
    Lg = L.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(Lg), np.isneginf(Lo))
    fin = np.isfinite(Lo)
    dl = np.abs(Lg[fin] - Lo[fin]).max()
    do = np.abs(Og - Oo).max()
    announce("O err", do, "bar", o_bar, "LSE err", dl, "bar", l_bar)
    assert dl <= l_bar, f"LSE max-abs {dl:.3g} > {l_bar:.3g}"
    assert do <= o_bar, f"O max-abs {do:.3g} > {o_bar:.3g}"


@pytest.mark.parametrize("seed", [3, 4])
def test_bf16_varlen_small(seed):
    """Packed sequences with ragged chunk tails and late-skewed anchors."""
    w = wl.scaled(wl.WORKLOADS["varlen8_fwdbwd"], len_median=1500, len_min=300, len_max=5000,
                  blocks_per_seq=6, n_seq=5)
    w, g, t = wl.make(w, seed)
    allc = np.arange(len(g.chunk_pos))
    announce("bf16 varlen", seed)
    O, L, _ = gpu_fwd(w, g, t, allc, True, n_wg=48)
    Oo, Lo = oracle_partial(w, g, t, allc, True)
    compare(O, L, Oo, Lo, "bf16", "varlen")


def test_bf16_cp_shards_partials_and_merge():
    """8 LPT shards of a 16K context (non-contiguous chunks per shard):
    every shard's partial, then the GPU 8-way merge vs unsplit attention."""
    w = wl.scaled(wl.WORKLOADS["cp64_rank0_ctx512k"], ctx=16384, anchor_lo=4096,
                  anchor_hi=16384, blocks_per_seq=12, chunk=512, n_shards=8)
    w, g, t = wl.make(w, 5)
    ids, _, _, _ = shards.lpt_shards(w, g, w.n_shards)
    Os, Ls = [], []
    for r in range(w.n_shards):
        announce("bf16 cp shard", r)
        O, L, _ = gpu_fwd(w, g, t, ids[r], r == 0, n_wg=40)
        Oo, Lo = oracle_partial(w, g, t, ids[r], r == 0)
        compare(O, L, Oo, Lo, "bf16", f"shard {r}")
        Os.append(O)
        Ls.append(L)
    for out_dt in (torch.float32, torch.bfloat16):
        Om = torch.empty(Os[0].shape, dtype=out_dt, device="cuda")
        Lm = torch.empty_like(Ls[0])
        announce("bf16 cp merge", out_dt)
        skv.skv_merge_lse(torch.stack(Os), torch.stack(Ls), Om, Lm)
        torch.cuda.synchronize()
        Of, Lf = oracle.attention(t.Q, t.K, t.V, t.Kd, t.Vd, g.anchors, g.lo,
                                  wl.softmax_scale(w.d))
        compare(Om, Lm, Of, Lf, "bf16", "merged")


def test_empty_and_draft_only_shards():
    w, g, t = _small32k(9, blocks_per_seq=4)
    announce("empty shard")
    O, L, _ = gpu_fwd(w, g, t, [], False, n_wg=16)
    assert torch.all(O.float() == 0) and torch.all(torch.isneginf(L))
    announce("draft-only shard")
    O, L, _ = gpu_fwd(w, g, t, [], True, n_wg=16)
    Oo, Lo = oracle_partial(w, g, t, [], True)
    compare(O, L, Oo, Lo, "bf16", "draft only")
    # anchors at the sequence start: context invisible, only draft keys
    g0 = wl.Geometry(g.seq_start, g.seq_len, np.zeros_like(g.anchors), g.lo, g.ctx,
                     g.chunk_pos, g.chunk_len)
    allc = np.arange(len(g.chunk_pos))
    announce("zero anchors")
    O, L, _ = gpu_fwd(w, g0, t, allc, True, n_wg=16)
    Oo, Lo = oracle_partial(w, g0, t, allc, True)
    compare(O, L, Oo, Lo, "bf16", "zero anchors")


@pytest.mark.parametrize("k,rows,d,in_dt,out_dt", [
    (1, 100, 128, "f32", "f32"), (3, 1000, 64, "f32", "f32"), (5, 333, 128, "bf16", "f32"),
    (64, 2048, 128, "bf16", "bf16"), (7, 517, 64, "f32", "bf16"),
    # sixteen partials per unrolled pass: one full pass, and a pass plus a tail
    (16, 64, 64, "f32", "f32"), (20, 777, 128, "bf16", "bf16")])
def test_merge_random_partials(k, rows, d, in_dt, out_dt):
    rng = np.random.default_rng(k * 1000 + rows)
    O = rng.standard_normal((k, rows, d)).astype(np.float32)
    L = (rng.standard_normal((k, rows)) * 4).astype(np.float32)
    dead = rng.random((k, rows)) < 0.2
    L[dead] = -np.inf
    O[dead] = 0
    L[:, :3] = -np.inf  # rows with no key anywhere
    O[:, :3] = 0
    if in_dt == "bf16":
        O = wl.round_to_bf16(O)
    Od, Ld = to_dev(O, in_dt), torch.from_numpy(L).cuda()
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    Om = torch.full((rows, d), float("nan"), dtype=odt, device="cuda")
    Lm = torch.full((rows,), float("nan"), device="cuda")
    announce("merge", k, rows, d, in_dt, out_dt)
    skv.skv_merge_lse(Od, Ld, Om, Lm)
    torch.cuda.synchronize()
    Oo, Lo = oracle.merge_lse(O, L)
    Og = Om.float().cpu().numpy()
    Lg = Lm.cpu().numpy()
    assert np.array_equal(np.isneginf(Lg), np.isneginf(Lo))
    fin = np.isfinite(Lo)
    assert np.abs(Lg[fin] - Lo[fin]).max() <= 1e-5
    err = np.abs(Og - Oo).max()
    print(f"[merge] k={k} O max-abs {err:.3g}", flush=True)
    if out_dt == "f32":
        assert err <= 1e-5
    else:
        # bf16 output: one rounding of a value of size max|O|
        assert err <= 2e-2 * max(1.0, np.abs(Oo).max())
    assert np.all(Og[~fin] == 0)


# ---------------------------------------------------------------- full sizes

def _sample_blocks(g, n_extra=4, seed=0):
    nb = len(g.anchors)
    rng = np.random.default_rng(seed)
    fixed = [0, 1, nb // 2, nb - 2, nb - 1]
    return sorted(set(fixed) | set(rng.choice(nb, n_extra, replace=False).tolist()))


def _full_plan(w, g, plan, chunk_ids=None, with_draft=True):
    """None (the uniform plan on every CU) or a per-XCD plan with cost
    scales, as the benchmark times, of the whole context or of a shard."""
    if plan == "uniform":
        return None
    prob = (shards.whole_context_problem(w, g) if chunk_ids is None
            else shards.shard_problem(w, g, chunk_ids, with_draft))
    return measured_like_plan(w, prob, 12)[0]


@pytest.mark.parametrize("plan", ["uniform", "xcd"])
def test_full_ctx32k_sampled_rows(plan):
    """32K context, 2048 queries, 32q/8kv, d=128 on all CUs (the benchmark
    launch): sampled anchor blocks x all heads against the oracle."""
    w, g, t = wl.make("ctx32k_q2k", 1)
    allc = np.arange(len(g.chunk_pos))
    announce("full ctx32k", plan)
    O, L, _ = gpu_fwd(w, g, t, allc, True, shard=_full_plan(w, g, plan))
    blocks = _sample_blocks(g)
    Oo, Lo = oracle.attention(t.Q, t.K, t.V, t.Kd, t.Vd, g.anchors, g.lo,
                              wl.softmax_scale(w.d), blocks=blocks)
    rows = block_rows(blocks)
    compare(O[rows], L[rows], Oo, Lo, "bf16", "ctx32k sampled")
    assert torch.all(torch.isfinite(L))


@pytest.mark.parametrize("plan", ["uniform", "xcd"])
def test_full_cp64_rank0_sampled_rows(plan):
    """512K context split over 64 LPT ranks; rank 0's chunks against all
    4096 queries; sampled blocks against the oracle partial."""
    w, g, _ = wl.make("cp64_rank0_ctx512k", 2, tensors=False)
    ids, _, _, _ = shards.lpt_shards(w, g, w.n_shards)
    t = wl.draw_tensors(w, g, 2, chunk_ids=ids[0])
    announce("full cp64 rank0", plan)
    O, L, _ = gpu_fwd(w, g, t, ids[0], True, shard=_full_plan(w, g, plan, ids[0], True))
    blocks = _sample_blocks(g, seed=1)
    Oo, Lo = oracle_partial(w, g, t, ids[0], True, blocks=blocks)
    rows = block_rows(blocks)
    compare(O[rows], L[rows], Oo, Lo, "bf16", "cp64 rank0 sampled")


@pytest.mark.parametrize("plan", ["uniform", "xcd"])
def test_full_varlen_fwd_sampled_rows(plan):
    w, g, t = wl.make("varlen8_fwdbwd", 3)
    allc = np.arange(len(g.chunk_pos))
    announce("full varlen fwd", plan)
    O, L, _ = gpu_fwd(w, g, t, allc, True, shard=_full_plan(w, g, plan))
    blocks = _sample_blocks(g, n_extra=6, seed=2)
    Oo, Lo = oracle.attention(t.Q, t.K, t.V, t.Kd, t.Vd, g.anchors, g.lo,
                              wl.softmax_scale(w.d), blocks=blocks)
    rows = block_rows(blocks)
    compare(O[rows], L[rows], Oo, Lo, "bf16", "varlen sampled")


def test_full_ctx1m_64_shards_then_64way_merge():
    """1M context, 8192 queries, 4096 chunks of 256 over 64 LPT shards: all
    64 partials on the GPU (draft keys on shard 0), then one 64-way LSE merge;
    the two anchor blocks with the smallest anchors (their ~260K visible keys
    lie in chunks spread over all 64 shards) against fp64 attention over the
    keys they see.  Each shard's K/V are drawn in fp32 and rounded to bf16 on
    the device (round to nearest even, as the host rounding does); the oracle
    gets the host-rounded rows."""
    w, g, _ = wl.make("ctx1m_merge64", 4, tensors=False)
    w32 = wl.scaled(w, dtype="f32")
    ids, _, _, load = shards.lpt_shards(w, g, w.n_shards)
    assert load.max() / load.mean() - 1 < 0.01
    t = wl.draw_tensors(w, g, 4, chunk_ids=[])
    Q = to_dev(t.Q, "bf16")
    Kd, Vd = to_dev(t.Kd, "bf16"), to_dev(t.Vd, "bf16")
    Op = torch.empty((w.n_shards, w.nq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    Lp = torch.empty((w.n_shards, w.nq, w.hq), dtype=torch.float32, device="cuda")
    for r in range(w.n_shards):
        if r % 8 == 0:
            announce("ctx1m shard", r)
        prob = shards.shard_problem(w, g, ids[r], r == 0)
        sh = skv.Shard(prob)
        K = to_dev(wl.draw_kv_chunks(w32, g, 4, ids[r], "K"), "bf16")
        V = to_dev(wl.draw_kv_chunks(w32, g, 4, ids[r], "V"), "bf16")
        sh.fwd(Q, K, V, Kd if r == 0 else None, Vd if r == 0 else None, Op[r], Lp[r])
        torch.cuda.synchronize()
        del K, V, sh
    Om = torch.empty((w.nq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    Lm = torch.empty((w.nq, w.hq), dtype=torch.float32, device="cuda")
    announce("ctx1m: 64-way merge")
    skv.skv_merge_lse(Op, Lp, Om, Lm)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        skv.skv_merge_lse(Op, Lp, Om, Lm)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    nbytes = (Op.numel() * 2 + Lp.numel() * 4) + (Om.numel() * 2 + Lm.numel() * 4)
    print(f"[ctx1m] 64-way merge {ms:.3f} ms, {nbytes / ms / 1e6:.0f} GB/s", flush=True)
    assert torch.all(torch.isfinite(Lm))
    blocks = [0, 1]
    need = np.nonzero(g.chunk_pos < g.anchors[blocks].max())[0]
    assert len(np.unique(ids_of(ids, need))) == w.n_shards
    announce("ctx1m: oracle on blocks", blocks, "over", len(need), "chunks")
    Ko = wl.draw_kv_chunks(w, g, 4, need, "K")
    Vo = wl.draw_kv_chunks(w, g, 4, need, "V")
    pos = shards.shard_rows(g, need)
    Oo, Lo = oracle.attention_partial(t.Q, Ko, Vo, pos, g.anchors, g.lo, wl.softmax_scale(w.d),
                                      t.Kd, t.Vd, blocks=blocks)
    rows = block_rows(blocks)
    compare(Om[rows], Lm[rows], Oo, Lo, "bf16", "ctx1m merged sampled")
    del Ko, Vo, Oo, Lo

    # The last anchor block sees (nearly) the whole 1M context.  One kv head
    # (and its G query heads) keeps the fp64 oracle within host memory.
    top = [len(g.anchors) - 1]
    h = w.hkv - 1
    G = w.hq // w.hkv
    need = np.nonzero(g.chunk_pos < g.anchors[top].max())[0]
    announce("ctx1m: oracle on block", top, "kv head", h, "over", len(need), "chunks")
    Ko = np.concatenate([wl.draw_kv_chunks(w, g, 4, need[i:i + 256], "K")[:, h:h + 1]
                         for i in range(0, len(need), 256)])
    Vo = np.concatenate([wl.draw_kv_chunks(w, g, 4, need[i:i + 256], "V")[:, h:h + 1]
                         for i in range(0, len(need), 256)])
    pos = shards.shard_rows(g, need)
    heads = slice(h * G, (h + 1) * G)
    Oo, Lo = oracle.attention_partial(t.Q[:, heads], Ko, Vo, pos, g.anchors, g.lo,
                                      wl.softmax_scale(w.d), t.Kd[:, h:h + 1],
                                      t.Vd[:, h:h + 1], blocks=top)
    assert pos.size > 1_000_000 - 8192
    rows = block_rows(top)
    compare(Om[rows][:, heads], Lm[rows][:, heads], Oo, Lo, "bf16", "ctx1m merged top block")


def ids_of(ids, chunks):
    """Shard of each chunk."""
    owner = {int(c): r for r, cs in enumerate(ids) for c in cs}
    return [owner[int(c)] for c in chunks]
