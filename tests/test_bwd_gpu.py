"""GPU parity of the backward (dQ, dK, dV and the draft-key gradients)
against the fp64 oracle through the C ABI.  Bar: max-abs <= 2e-2 for the
bf16 path; every check also bounds the error relative to the largest
reference value, so small gradients cannot pass by being small."""
import functools

import numpy as np
import pytest
import torch

import oracle
from block_sparse_split_amd import splitkv as skv
from block_sparse_split_amd import shards
from block_sparse_split_amd import workloads as wl
from gpu_util import announce, block_rows, gpu_fwd, measured_like_plan, rows_of, to_dev

pytestmark = pytest.mark.gpu

ABS_TOL = 2e-2
REL_TOL = 2e-2  # of max |reference|


def check_grad(got, want, what, abs_tol=ABS_TOL):
    got = got.float().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else got
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    err = np.abs(got - want).max(initial=0.0)
    scale = np.abs(want).max(initial=0.0)
    if abs_tol is not None:
        assert err <= abs_tol, f"{what}: max-abs {err:.3g} > {abs_tol}"
    assert err <= REL_TOL * scale + 1e-7, f"{what}: max-abs {err:.3g} vs max|ref| {scale:.3g}"
    return err, scale


def gpu_bwd(w, g, t, chunk_ids, with_draft, O, LSE, n_wg=0, grad_dtype=skv.SKV_F32,
            xcd_speed=None, cost_scale=None):
    prob = shards.shard_problem(w, g, chunk_ids, with_draft)
    sh = skv.Shard(prob, n_workgroups=n_wg, xcd_speed=xcd_speed, cost_scale=cost_scale)
    r = rows_of(t, g, chunk_ids)
    dt = w.dtype
    Q, K, V = to_dev(t.Q, dt), to_dev(t.K[r], dt), to_dev(t.V[r], dt)
    Kd = to_dev(t.Kd, dt) if with_draft else None
    Vd = to_dev(t.Vd, dt) if with_draft else None
    dO = to_dev(t.dO, dt)
    gdt = torch.float32 if grad_dtype == skv.SKV_F32 else torch.bfloat16
    nl = len(r)
    dQ = torch.full((w.nq, w.hq, w.d), float("nan"), device="cuda")
    dK = torch.full((nl, w.hkv, w.d), float("nan"), dtype=gdt, device="cuda")
    dV = torch.full_like(dK, float("nan"))
    dKd = torch.full((w.nq, w.hkv, w.d), float("nan"), dtype=gdt, device="cuda") \
        if with_draft else None
    dVd = torch.full_like(dKd, float("nan")) if with_draft else None
    sh.bwd(Q, K, V, Kd, Vd, O, dO, LSE, dQ, dK, dV, dKd, dVd, grad_dtype)
    torch.cuda.synchronize()
    return dQ, dK, dV, dKd, dVd


def oracle_fwd_bwd(w, g, t, chunk_ids, with_draft, blocks=None):
    scale = wl.softmax_scale(w.d)
    O, L = oracle.attention(t.Q, t.K, t.V, t.Kd, t.Vd, g.anchors, g.lo, scale,
                            pos=shards.shard_rows(g, t.chunk_ids))
    r = rows_of(t, g, chunk_ids)
    pos = shards.shard_rows(g, chunk_ids)
    grads = oracle.attention_bwd(t.Q, t.K[r], t.V[r], pos, g.anchors, g.lo, scale, O, t.dO, L,
                                 t.Kd if with_draft else None, t.Vd if with_draft else None,
                                 blocks=blocks)
    return O, L, grads


def _small(seed, **over):
    base = dict(ctx=4096, anchor_lo=1024, anchor_hi=4096, blocks_per_seq=16)
    base.update(over)
    return wl.make(wl.scaled(wl.WORKLOADS["ctx32k_q2k"], **base), seed, with_grad=True)


@pytest.mark.parametrize("seed,n_wg,gdt", [(0, 256, skv.SKV_F32), (1, 17, skv.SKV_BF16),
                                           (2, 1, skv.SKV_F32)])
def test_bwd_small_with_oracle_stats(seed, n_wg, gdt):
    """The backward alone, fed the oracle's O (rounded to bf16) and LSE."""
    w, g, t = _small(seed)
    allc = np.arange(len(g.chunk_pos))
    O, L, (dQ, dK, dV, dKd, dVd) = oracle_fwd_bwd(w, g, t, allc, True)
    announce("bwd small oracle-stats", seed, n_wg, gdt)
    got = gpu_bwd(w, g, t, allc, True, to_dev(wl.round_to_bf16(O.astype(np.float32)), "bf16"),
                  torch.from_numpy(L.astype(np.float32)).cuda(), n_wg=n_wg, grad_dtype=gdt)
    for name, a, b in zip(("dQ", "dK", "dV", "dKd", "dVd"), got, (dQ, dK, dV, dKd, dVd)):
        check_grad(a, b, name)


@pytest.mark.parametrize("seed", [3, 4])
def test_fwd_then_bwd_chain_small(seed):
    """GPU forward output and LSE feed the GPU backward."""
    w, g, t = _small(seed)
    allc = np.arange(len(g.chunk_pos))
    announce("fwd->bwd chain", seed)
    O, L, _ = gpu_fwd(w, g, t, allc, True, n_wg=64)
    got = gpu_bwd(w, g, t, allc, True, O, L, n_wg=64)
    _, _, want = oracle_fwd_bwd(w, g, t, allc, True)
    for name, a, b in zip(("dQ", "dK", "dV", "dKd", "dVd"), got, want):
        check_grad(a, b, name)


@pytest.mark.parametrize("seed,n_wg", [(8, 1), (9, 64)])
def test_fwd_bwd_wide_logits(seed, n_wg):
    """Logits that grow along the context: key rows at position p are scaled
    by 2^min(5, p // 600) (a power of two, so the bf16 inputs stay exact).
    Each row's running maximum then rises by tens of units (log2) inside one
    work item, which drives the forward's rescale of O and its recomputation
    of P, and puts weights far below the maximum next to ones near it.

    The bar follows from the arithmetic, because the fp32 error of S grows
    with the logits: S sums d exact bf16 products in fp32, so it errs by at
    most eps_s = d 2^-24 max|q| max|k|; a weight 2^(c S - m) then errs by a
    factor of at most 2^(c eps_s) in numerator and denominator, P is rounded
    to bf16 (8 significant bits: at most 2^-8 of the value) and so is O
    (2^-8 |O|).  LSE errs by at most scale eps_s.  A missed or wrong rescale
    is off by O(1) in both.  The gradients grow with the inputs (dQ reaches
    about 1e2), so they are held to the relative bar alone."""
    w, g, t = _small(seed)
    pos = shards.shard_rows(g, t.chunk_ids)
    t.K *= (2.0 ** np.minimum(5, pos // 600)).astype(np.float32)[:, None, None]
    allc = np.arange(len(g.chunk_pos))
    announce("fwd+bwd wide logits", seed, n_wg)
    O, L, _ = gpu_fwd(w, g, t, allc, True, n_wg=n_wg)
    Oo, Lo, want = oracle_fwd_bwd(w, g, t, allc, True)
    assert np.nanmax(Lo) > 100.0   # the logits really are wide
    scale = wl.softmax_scale(w.d)
    c = scale * np.log2(np.e)
    kmax = max(np.linalg.norm(t.K, axis=-1).max(), np.linalg.norm(t.Kd, axis=-1).max())
    eps_s = w.d * 2.0 ** -24 * np.linalg.norm(t.Q, axis=-1).max() * kmax
    vmax = max(np.abs(t.V).max(), np.abs(t.Vd).max())
    o_bar = vmax * (2.0 ** -8 + 2 * np.log(2) * c * eps_s) + 2.0 ** -8 * np.abs(Oo).max()
    l_bar = scale * eps_s + 1e-5
    Og = O.float().cpu().numpy().astype(np.float64)
    Lg = L.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(Lg), np.isneginf(Lo))
    fin = np.isfinite(Lo)
    dl = np.abs(Lg[fin] - Lo[fin]).max()
    do = np.abs(Og - Oo).max()
    announce("O err", do, "bar", o_bar, "LSE err", dl, "bar", l_bar)
    assert dl <= l_bar, f"LSE max-abs {dl:.3g} > {l_bar:.3g}"
    assert do <= o_bar, f"O max-abs {do:.3g} > {o_bar:.3g}"
    got = gpu_bwd(w, g, t, allc, True, O, L, n_wg=n_wg)
    for name, a, b in zip(("dQ", "dK", "dV", "dKd", "dVd"), got, want):
        check_grad(a, b, f"wide logits {name}", abs_tol=None)


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 64), (16, 1, 128), (8, 4, 128), (16, 2, 64)])
def test_bwd_gqa_and_head_dims(hq, hkv, d):
    w, g, t = _small(5, hq=hq, hkv=hkv, d=d, ctx=2048, anchor_lo=100, anchor_hi=2048,
                     blocks_per_seq=9)
    allc = np.arange(len(g.chunk_pos))
    O, L, want = oracle_fwd_bwd(w, g, t, allc, True)
    announce("bwd gqa", hq, hkv, d)
    got = gpu_bwd(w, g, t, allc, True, to_dev(wl.round_to_bf16(O.astype(np.float32)), "bf16"),
                  torch.from_numpy(L.astype(np.float32)).cuda(), n_wg=24)
    for name, a, b in zip(("dQ", "dK", "dV", "dKd", "dVd"), got, want):
        check_grad(a, b, f"{name} G={hq // hkv} d={d}")


def test_bwd_split_over_shards():
    """Per-shard backward with the final merged O/LSE: the dQ shares sum to
    the full dQ and each shard's dK/dV are its rows of the unsplit ones."""
    w = wl.scaled(wl.WORKLOADS["cp64_rank0_ctx512k"], ctx=8192, anchor_lo=2048,
                  anchor_hi=8192, blocks_per_seq=8, chunk=512, n_shards=4)
    w, g, t = wl.make(w, 6, with_grad=True)
    ids, _, _, _ = shards.lpt_shards(w, g, w.n_shards)
    allc = np.arange(len(g.chunk_pos))
    O, L, full = oracle_fwd_bwd(w, g, t, allc, True)
    Od = to_dev(wl.round_to_bf16(O.astype(np.float32)), "bf16")
    Ld = torch.from_numpy(L.astype(np.float32)).cuda()
    shares = torch.empty((w.n_shards, w.nq, w.hq, w.d), device="cuda")
    for r in range(w.n_shards):
        announce("bwd shard", r)
        dQ, dK, dV, dKd, dVd = gpu_bwd(w, g, t, ids[r], r == 0, Od, Ld, n_wg=32)
        shares[r] = dQ
        rr = rows_of(t, g, ids[r])
        check_grad(dK, full[1][rr], f"dK shard {r}")
        check_grad(dV, full[2][rr], f"dV shard {r}")
        if r == 0:
            check_grad(dKd, full[3], "dKd")
            check_grad(dVd, full[4], "dVd")
    announce("dq_finalize of the shard shares")
    for dt in (torch.float32, torch.bfloat16):
        dq = torch.full((w.nq, w.hq, w.d), float("nan"), dtype=dt, device="cuda")
        skv.skv_dq_finalize(shares, dq)
        torch.cuda.synchronize()
        check_grad(dq, full[0], f"finalized dQ ({dt})")


@pytest.mark.parametrize("n,shape,pad,odt", [
    (1, (64, 32, 128), 0, "f32"), (3, (16, 4, 64), 0, "bf16"), (8, (37, 5, 3), 1, "f32"),
    (64, (256, 8, 64), 0, "bf16"), (5, (1, 1, 7), 3, "bf16"), (2, (2, 2, 2), 0, "f32")])
def test_dq_finalize_random_shares(n, shape, pad, odt):
    """Sum of n fp32 shares (dim 0 padded by `pad` floats per share, then
    rounded up to a multiple of 4) against the fp64 sum.  Bound from the
    arithmetic: n - 1 fp32 additions in index order err by at most
    (n - 1) 2^-24 sum_k |x_k|; a bf16 output adds one rounding to nearest
    (8 significant bits), at most 2^-8 of the value."""
    rng = np.random.default_rng(n * 100 + pad)
    elems = int(np.prod(shape))
    stride = -(-(elems + pad) // 4) * 4
    buf = torch.full((n, stride), float("nan"), device="cuda")
    x = rng.standard_normal((n,) + shape).astype(np.float32)
    buf[:, :elems] = torch.from_numpy(x.reshape(n, elems)).cuda()
    parts = buf[:, :elems].view((n,) + shape)
    dt = torch.bfloat16 if odt == "bf16" else torch.float32
    out = torch.full(shape, float("nan"), dtype=dt, device="cuda")
    announce("dq_finalize", n, shape, pad, odt)
    skv.skv_dq_finalize(parts, out)
    torch.cuda.synchronize()
    want = oracle.dq_finalize(x)
    got = out.float().cpu().numpy().astype(np.float64)
    bound = (n - 1) * 2.0 ** -24 * np.abs(x.astype(np.float64)).sum(0)
    if odt == "bf16":
        bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(want)
    assert np.all(np.abs(got - want) <= bound + 1e-30)
    if odt == "f32" and n <= 8:
        assert np.abs(got - want).max() <= 1e-5
    if odt == "f32":
        # in place: the output may be share 0 itself
        skv.skv_dq_finalize(parts, parts[0])
        torch.cuda.synchronize()
        assert torch.equal(parts[0], out)


def test_bwd_varlen_small():
    w = wl.scaled(wl.WORKLOADS["varlen8_fwdbwd"], len_median=1500, len_min=300, len_max=5000,
                  blocks_per_seq=6, n_seq=5)
    w, g, t = wl.make(w, 7, with_grad=True)
    allc = np.arange(len(g.chunk_pos))
    announce("bwd varlen small")
    O, L, _ = gpu_fwd(w, g, t, allc, True, n_wg=40)
    got = gpu_bwd(w, g, t, allc, True, O, L, n_wg=40)
    _, _, want = oracle_fwd_bwd(w, g, t, allc, True)
    for name, a, b in zip(("dQ", "dK", "dV", "dKd", "dVd"), got, want):
        check_grad(a, b, f"varlen {name}")


def full_fwd_bwd(w, g, t, plan):
    """Forward then backward over the whole context on every CU: with the
    uniform plan and fp32 gradients, or as the benchmark runs it (a per-XCD
    plan with cost scales, bf16 gradients)."""
    allc = np.arange(len(g.chunk_pos))
    if plan == "uniform":
        O, L, _ = gpu_fwd(w, g, t, allc, True)
        return gpu_bwd(w, g, t, allc, True, O, L)
    sh, speed, scale = measured_like_plan(w, shards.whole_context_problem(w, g), 11)
    O, L, _ = gpu_fwd(w, g, t, allc, True, shard=sh)
    return gpu_bwd(w, g, t, allc, True, O, L, grad_dtype=skv.SKV_BF16, xcd_speed=speed,
                   cost_scale=scale)


@functools.lru_cache(maxsize=1)
def expected_ctx32k():
    """The 32K workload and the oracle's gradients on sampled anchor blocks
    (dQ and the draft-key gradients) and sampled key ranges (dK, dV); the
    oracle recomputes the full forward for the normaliser."""
    w, g, t = wl.make("ctx32k_q2k", 1, with_grad=True)
    scale = wl.softmax_scale(w.d)
    Oo, Lo = oracle.attention(t.Q, t.K, t.V, t.Kd, t.Vd, g.anchors, g.lo, scale)
    blocks = [0, 5, 63, 64, 126, 127]
    gq = oracle.attention_bwd(t.Q, t.K, t.V, np.arange(g.ctx), g.anchors, g.lo, scale, Oo,
                              t.dO, Lo, t.Kd, t.Vd, blocks=blocks)
    keys = np.concatenate([np.arange(0, 64), np.arange(20000, 20100), np.arange(32700, 32768)])
    gk = oracle.attention_bwd(t.Q, t.K[keys], t.V[keys], keys, g.anchors, g.lo, scale, Oo, t.dO,
                              Lo)
    return (w, g, t), block_rows(blocks), keys, gq, gk


@pytest.mark.parametrize("plan", ["uniform", "xcd_bf16_grads"])
def test_bwd_full_ctx32k_sampled(plan):
    """The 32K-context shapes on all CUs: dQ on sampled anchor blocks and
    dK/dV on sampled key ranges, against the oracle."""
    (w, g, t), rows, keys, gq, gk = expected_ctx32k()
    announce("bwd full ctx32k", plan)
    dQ, dK, dV, dKd, dVd = full_fwd_bwd(w, g, t, plan)
    check_grad(dQ[rows], gq[0][rows], "dQ sampled rows")
    check_grad(dKd[rows], gq[3][rows], "dKd sampled rows")
    check_grad(dVd[rows], gq[4][rows], "dVd sampled rows")
    check_grad(dK[keys], gk[1], "dK sampled keys")
    check_grad(dV[keys], gk[2], "dV sampled keys")


@functools.lru_cache(maxsize=1)
def expected_varlen():
    """Varlen batch (8 packed sequences, lognormal lengths, late-skewed
    anchors) and the oracle's gradients on sampled key ranges (a sequence
    start, a late range and a sequence end) and on exactly the anchor
    blocks that see those keys, plus three more blocks for dQ."""
    w, g, t = wl.make("varlen8_fwdbwd", 5, with_grad=True)
    scale = wl.softmax_scale(w.d)
    s0 = int(g.seq_start[1])
    s1, l1 = int(g.seq_start[3]), int(g.seq_len[3])
    keys = np.concatenate([np.arange(s0, s0 + 32),
                           np.arange(s1 + int(0.92 * l1), s1 + int(0.92 * l1) + 48),
                           np.arange(s1 + l1 - 32, s1 + l1)])
    sees = (g.lo[:, None] <= keys[None, :]) & (keys[None, :] < g.anchors[:, None])
    nb = len(g.anchors)
    blocks = sorted(set(np.nonzero(sees.any(1))[0].tolist()) | {0, nb // 2, nb - 1})
    announce("bwd full varlen: oracle on", len(blocks), "blocks")
    Ob, Lb = oracle.attention(t.Q, t.K, t.V, t.Kd, t.Vd, g.anchors, g.lo, scale, blocks=blocks)
    rows = block_rows(blocks)
    Of = np.zeros((w.nq, w.hq, w.d))
    Lf = np.full((w.nq, w.hq), -np.inf)
    Of[rows], Lf[rows] = Ob, Lb
    gq = oracle.attention_bwd(t.Q, t.K, t.V, np.arange(g.ctx), g.anchors, g.lo, scale, Of,
                              t.dO, Lf, t.Kd, t.Vd, blocks=blocks)
    # rows outside `blocks` see none of the sampled keys
    gk = oracle.attention_bwd(t.Q, t.K[keys], t.V[keys], keys, g.anchors, g.lo, scale, Of, t.dO,
                              Lf)
    return (w, g, t), rows, keys, gq, gk


@pytest.mark.parametrize("plan", ["uniform", "xcd_bf16_grads"])
def test_bwd_full_varlen_sampled(plan):
    """The varlen batch on all CUs: dQ and the draft-key gradients on
    sampled anchor blocks, dK/dV on sampled key ranges, against the
    oracle."""
    (w, g, t), rows, keys, gq, gk = expected_varlen()
    announce("bwd full varlen", plan)
    dQ, dK, dV, dKd, dVd = full_fwd_bwd(w, g, t, plan)
    check_grad(dQ[rows], gq[0][rows], "varlen dQ sampled rows")
    check_grad(dKd[rows], gq[3][rows], "varlen dKd sampled rows")
    check_grad(dVd[rows], gq[4][rows], "varlen dVd sampled rows")
    check_grad(dK[keys], gk[1], "varlen dK sampled keys")
    check_grad(dV[keys], gk[2], "varlen dV sampled keys")


def test_hip_graph_replays_match_eager():
    """One forward + backward captured in a HIP graph and replayed: the entry
    points allocate nothing and clear nothing with memset, so every replay
    must give the eager step's bits.  Between replays the program runs eager
    work of its own, and the last replay reads new query values written into
    the captured buffer in place."""
    w, g, t = _small(6, ctx=8192, anchor_lo=2048, anchor_hi=8192, blocks_per_seq=32)
    prob = shards.whole_context_problem(w, g)
    sh = skv.Shard(prob)
    dt = w.dtype
    Q, K, V = to_dev(t.Q, dt), to_dev(t.K, dt), to_dev(t.V, dt)
    Kd, Vd, dO = to_dev(t.Kd, dt), to_dev(t.Vd, dt), to_dev(t.dO, dt)
    O = torch.empty((w.nq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    LSE = torch.empty((w.nq, w.hq), device="cuda")
    dQ = torch.empty((w.nq, w.hq, w.d), device="cuda")
    dK, dV = torch.empty_like(K), torch.empty_like(V)
    dKd, dVd = torch.empty_like(Kd), torch.empty_like(Vd)
    outs = (O, LSE, dQ, dK, dV, dKd, dVd)

    def step():
        sh.fwd(Q, K, V, Kd, Vd, O, LSE)
        sh.bwd(Q, K, V, Kd, Vd, O, dO, LSE, dQ, dK, dV, dKd, dVd, skv.SKV_BF16)

    def eager():
        step()
        torch.cuda.synchronize()
        return [x.clone() for x in outs]

    announce("hip graph replay vs eager", w.nq, g.ctx)
    ref = eager()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in outs:
            x.fill_(float("nan"))
        # eager work of the program's own between replays
        (K.float() * 1.5).sum().item()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("O", "LSE", "dQ", "dK", "dV", "dKd", "dVd"), outs, ref):
            assert torch.equal(x, r), f"replay {rep}: {name} differs from the eager step"
    # new inputs, written in place: the replay must follow them
    Q.copy_(torch.flip(Q, dims=(0,)))
    new = eager()
    assert not torch.equal(new[0], ref[0])
    for x in outs:
        x.fill_(float("nan"))
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    for name, x, r in zip(("O", "LSE", "dQ", "dK", "dV", "dKd", "dVd"), outs, new):
        assert torch.equal(x, r), f"replay on new Q: {name} differs from the eager step"


def test_bwd_empty_and_draft_only_shards():
    """Shards with no context keys: an empty shard adds exactly nothing to
    dQ; a draft-only shard adds the draft keys' share and their gradients.
    With every anchor at the sequence start no row sees a context key, so
    dK and dV are exactly zero."""
    w, g, t = _small(9, blocks_per_seq=4)
    allc = np.arange(len(g.chunk_pos))
    O, L, _ = oracle_fwd_bwd(w, g, t, allc, True)
    Od = to_dev(wl.round_to_bf16(O.astype(np.float32)), "bf16")
    Ld = torch.from_numpy(L.astype(np.float32)).cuda()
    announce("bwd empty shard")
    dQ, dK, dV, _, _ = gpu_bwd(w, g, t, [], False, Od, Ld, n_wg=16)
    assert dK.shape[0] == 0 and dV.shape[0] == 0
    assert torch.all(dQ == 0), "an empty shard must add nothing to dQ"
    announce("bwd draft-only shard")
    dQ, _, _, dKd, dVd = gpu_bwd(w, g, t, [], True, Od, Ld, n_wg=16)
    _, _, (wq, _, _, wkd, wvd) = oracle_fwd_bwd(w, g, t, [], True)
    check_grad(dQ, wq, "draft-only dQ share")
    check_grad(dKd, wkd, "draft-only dKd")
    check_grad(dVd, wvd, "draft-only dVd")
    g0 = wl.Geometry(g.seq_start, g.seq_len, np.zeros_like(g.anchors), g.lo, g.ctx,
                     g.chunk_pos, g.chunk_len)
    O0, L0, (zq, zk, zv, zkd, zvd) = oracle_fwd_bwd(w, g0, t, allc, True)
    announce("bwd zero anchors")
    dQ, dK, dV, dKd, dVd = gpu_bwd(w, g0, t, allc, True,
                                   to_dev(wl.round_to_bf16(O0.astype(np.float32)), "bf16"),
                                   torch.from_numpy(L0.astype(np.float32)).cuda(), n_wg=16)
    assert torch.all(dK.float() == 0) and torch.all(dV.float() == 0)
    assert not np.any(zk) and not np.any(zv)
    check_grad(dQ, zq, "zero anchors dQ")
    check_grad(dKd, zkd, "zero anchors dKd")
    check_grad(dVd, zvd, "zero anchors dVd")


def test_workgroup_clock_stamps():
    """With a per-workgroup clock buffer set, the forward, dQ and dK/dV
    kernels stamp every workgroup (start <= end, plus the hardware ids of
    where it ran) and compute the same bits;
    a buffer too small for the schedule is refused before any launch."""
    w, g, t = _small(8, blocks_per_seq=16)
    prob = shards.whole_context_problem(w, g)
    sh = skv.Shard(prob, n_workgroups=40)
    dt = w.dtype
    Q, K, V = to_dev(t.Q, dt), to_dev(t.K, dt), to_dev(t.V, dt)
    Kd, Vd, dO = to_dev(t.Kd, dt), to_dev(t.Vd, dt), to_dev(t.dO, dt)

    def step():
        O = torch.empty((w.nq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
        LSE = torch.empty((w.nq, w.hq), device="cuda")
        dQ = torch.empty((w.nq, w.hq, w.d), device="cuda")
        dK, dV = torch.empty_like(K), torch.empty_like(V)
        dKd, dVd = torch.empty_like(Kd), torch.empty_like(Vd)
        sh.fwd(Q, K, V, Kd, Vd, O, LSE)
        sh.bwd(Q, K, V, Kd, Vd, O, dO, LSE, dQ, dK, dV, dKd, dVd, skv.SKV_BF16)
        torch.cuda.synchronize()
        return O, LSE, dQ, dK, dV, dKd, dVd

    announce("workgroup clock stamps, 40 workgroups")
    ref = step()
    clk = torch.zeros(3 * 40 * 4, dtype=torch.int64, device="cuda")
    skv.skv_timing_wg_clock(clk)
    try:
        got = step()
        small = torch.zeros(3 * 39 * 4, dtype=torch.int64, device="cuda")
        skv.skv_timing_wg_clock(small)
        with pytest.raises(skv.SplitKVError):
            step()
    finally:
        skv.skv_timing_wg_clock(None)
    for x, r in zip(got, ref):
        assert torch.equal(x, r)
    st = clk.view(3, 40, 4).cpu().numpy()
    assert np.all(st[:, :, 0] > 0) and np.all(st[:, :, 1] >= st[:, :, 0])
    # hardware ids: an XCD in 0..7 and 32-bit register values
    assert np.all((st[:, :, 2] & 15) < 8) and np.all(st[:, :, 2:] < 2 ** 32)
    print("[stamps] workgroups on XCD w mod 8:",
          float(np.mean((st[:, :, 2] & 15) == np.arange(40) % 8)), flush=True)
    # the three kernels run one after another on the stream
    assert st[0, :, 1].max() <= st[1, :, 0].min() + 1
    assert st[1, :, 1].max() <= st[2, :, 0].min() + 1
