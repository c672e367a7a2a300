"""Pins for the fp64 attention oracle (CPU only).

Each check ties the oracle to something other than itself: a dense
brute-force masked softmax through torch's own attention routine, closed
forms (Q = 0, constant V, key shift), GQA against repeated-KV MHA, merging
random K-way key partitions, central finite differences and torch autograd.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention_fp64 as oatt
from block_sparse_split_amd import workloads as wl

BLOCK = 16


def tiny_problem(seed, nb=3, ctx=80, hq=4, hkv=2, d=8, nseq=1, draft=True):
    """Small random problem; anchors anywhere in [lo, ctx] incl. 0 keys."""
    rng = np.random.default_rng(seed)
    if nseq == 1:
        lo = np.zeros(nb, np.int32)
        anchors = np.sort(rng.integers(0, ctx + 1, size=nb)).astype(np.int32)
    else:
        cuts = np.sort(rng.choice(np.arange(1, ctx), nseq - 1, replace=False))
        starts = np.concatenate([[0], cuts])
        ends = np.concatenate([cuts, [ctx]])
        seq = rng.integers(0, nseq, size=nb)
        seq.sort()
        lo = starts[seq].astype(np.int32)
        anchors = np.array([rng.integers(starts[s], ends[s] + 1) for s in seq],
                           np.int32)
    nq = nb * BLOCK
    Q = rng.standard_normal((nq, hq, d))
    K = rng.standard_normal((ctx, hkv, d))
    V = rng.standard_normal((ctx, hkv, d))
    Kd = rng.standard_normal((nq, hkv, d)) if draft else None
    Vd = rng.standard_normal((nq, hkv, d)) if draft else None
    return dict(Q=Q, K=K, V=V, Kd=Kd, Vd=Vd, anchors=anchors, lo=lo,
                scale=1.0 / math.sqrt(d))


def dense_mask(anchors, lo, ctx, nq, with_draft=True):
    """[nq, ctx + nq] boolean mask built key by key (no interval tricks)."""
    m = np.zeros((nq, ctx + (nq if with_draft else 0)), bool)
    for r in range(nq):
        i = r // BLOCK
        for j in range(ctx):
            m[r, j] = lo[i] <= j < anchors[i]
        if with_draft:
            for rp in range(nq):
                m[r, ctx + rp] = (rp // BLOCK) == i
    return m


def torch_dense(p, requires_grad=False):
    """O, LSE via torch's scaled_dot_product_attention (fp64, CPU)."""
    Q, K, V, Kd, Vd = (torch.tensor(p[k]) for k in ("Q", "K", "V", "Kd", "Vd"))
    if requires_grad:
        for t in (Q, K, V, Kd, Vd):
            t.requires_grad_(True)
    nq, hq, d = Q.shape
    ctx, hkv, _ = K.shape
    G = hq // hkv
    mask = torch.tensor(dense_mask(p["anchors"], p["lo"], ctx, nq))
    Kall = torch.cat([K, Kd], 0).repeat_interleave(G, dim=1)  # [n, hq, d]
    Vall = torch.cat([V, Vd], 0).repeat_interleave(G, dim=1)
    q = Q.permute(1, 0, 2)
    k = Kall.permute(1, 0, 2)
    v = Vall.permute(1, 0, 2)
    O = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, scale=p["scale"]).permute(1, 0, 2)
    z = p["scale"] * (q @ k.transpose(1, 2))
    lse = torch.logsumexp(z.masked_fill(~mask, -math.inf), dim=-1).T
    return O, lse, (Q, K, V, Kd, Vd)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("nseq", [1, 3])
def test_matches_torch_dense_attention(seed, nseq):
    p = tiny_problem(seed, nseq=nseq)
    O, L = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                            p["anchors"], p["lo"], p["scale"])
    Ot, Lt, _ = torch_dense(p)
    np.testing.assert_allclose(O, Ot.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(L, Lt.numpy(), atol=1e-12, rtol=0)


def test_q_zero_closed_form():
    """Q = 0: every visible key gets equal weight, so LSE = ln(#visible) with
    #visible = a_i - lo_i + 16 and O = mean of the visible values."""
    p = tiny_problem(5, nb=4, ctx=100, nseq=2)
    p["Q"][:] = 0
    O, L = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                            p["anchors"], p["lo"], p["scale"])
    G = p["Q"].shape[1] // p["K"].shape[1]
    for r in range(p["Q"].shape[0]):
        i = r // BLOCK
        a, l = int(p["anchors"][i]), int(p["lo"][i])
        assert np.all(L[r] == pytest.approx(math.log(a - l + BLOCK), abs=1e-13))
        for h in range(p["Q"].shape[1]):
            g = h // G
            vals = np.concatenate([p["V"][l:a, g],
                                   p["Vd"][BLOCK * i:BLOCK * (i + 1), g]])
            np.testing.assert_allclose(O[r, h], vals.mean(axis=0), atol=1e-13)


def test_constant_v_gives_v():
    p = tiny_problem(7, nseq=2)
    c = np.random.default_rng(1).standard_normal((p["K"].shape[1], p["K"].shape[2]))
    p["V"][:] = c[None]
    p["Vd"][:] = c[None]
    O, _ = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                            p["anchors"], p["lo"], p["scale"])
    G = p["Q"].shape[1] // p["K"].shape[1]
    np.testing.assert_allclose(O, np.repeat(c, G, axis=0)[None].repeat(O.shape[0], 0),
                               atol=1e-13)


def test_key_shift_moves_lse_only():
    p = tiny_problem(8)
    O0, L0 = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                              p["anchors"], p["lo"], p["scale"])
    c = np.random.default_rng(2).standard_normal((p["K"].shape[1], p["K"].shape[2]))
    O1, L1 = oracle.attention(p["Q"], p["K"] + c[None], p["V"], p["Kd"] + c[None],
                              p["Vd"], p["anchors"], p["lo"], p["scale"])
    G = p["Q"].shape[1] // p["K"].shape[1]
    shift = p["scale"] * np.einsum("rhd,hd->rh", p["Q"], np.repeat(c, G, axis=0))
    np.testing.assert_allclose(O1, O0, atol=1e-12)
    np.testing.assert_allclose(L1, L0 + shift, atol=1e-12)


def test_gqa_equals_repeated_kv_mha():
    p = tiny_problem(9, hq=6, hkv=2)
    O, L = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                            p["anchors"], p["lo"], p["scale"])
    rep = lambda x: np.repeat(x, 3, axis=1)
    Om, Lm = oracle.attention(p["Q"], rep(p["K"]), rep(p["V"]), rep(p["Kd"]),
                              rep(p["Vd"]), p["anchors"], p["lo"], p["scale"])
    np.testing.assert_allclose(O, Om, atol=1e-14)
    np.testing.assert_allclose(L, Lm, atol=1e-14)


def test_weights_sum_to_one_and_block_subset():
    p = tiny_problem(10, nb=4)
    O, L = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                            p["anchors"], p["lo"], p["scale"])
    Os, Ls = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                              p["anchors"], p["lo"], p["scale"], blocks=[3, 1])
    np.testing.assert_array_equal(Os[:16], O[48:64])
    np.testing.assert_array_equal(Ls[16:], L[16:32])
    # weights with V = identity rows sum to one: O of all-ones V is 1
    p["V"][:] = 1.0
    p["Vd"][:] = 1.0
    O1, _ = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                             p["anchors"], p["lo"], p["scale"])
    np.testing.assert_allclose(O1, 1.0, atol=1e-14)


def _random_partition(rng, n, k):
    lab = rng.integers(0, k, size=n)
    lab[rng.random(n) < 0.1] = k - 1  # make the last part larger
    return [np.nonzero(lab == j)[0] for j in range(k)]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_merge_of_any_partition_is_exact(seed):
    rng = np.random.default_rng(100 + seed)
    p = tiny_problem(seed, nb=4, ctx=120, nseq=2)
    O, L = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                            p["anchors"], p["lo"], p["scale"])
    k = int(rng.integers(2, 7))
    parts = _random_partition(rng, p["K"].shape[0], k)
    # a shard holding only keys 0..3 leaves most rows fully masked
    parts = [idx[idx >= 4] for idx in parts] + [np.arange(0, 4)]
    parts.append(np.array([], np.int64))          # an empty shard
    Op, Lp = [], []
    draft_at = int(rng.integers(0, len(parts)))
    for j, idx in enumerate(parts):
        with_d = j == draft_at
        o, l = oracle.attention_partial(
            p["Q"], p["K"][idx], p["V"][idx], idx, p["anchors"], p["lo"],
            p["scale"], p["Kd"] if with_d else None, p["Vd"] if with_d else None)
        # the empty shard must give O = 0 and LSE = -inf everywhere
        if idx.size == 0 and not with_d:
            assert np.all(np.isneginf(l)) and np.all(o == 0)
        Op.append(o)
        Lp.append(l)
    Om, Lm = oracle.merge_lse(np.stack(Op), np.stack(Lp))
    np.testing.assert_allclose(Om, O, atol=1e-12)
    np.testing.assert_allclose(Lm, L, atol=1e-12)


def test_merge_associative_and_all_neg_inf():
    rng = np.random.default_rng(3)
    O = rng.standard_normal((3, 5, 2, 4))
    L = rng.standard_normal((3, 5, 2)) * 3
    L[1, 2, 0] = -np.inf
    O[1, 2, 0] = 0
    Oab, Lab = oracle.merge_lse(O[:2], L[:2])
    O1, L1 = oracle.merge_lse(np.stack([Oab, O[2]]), np.stack([Lab, L[2]]))
    O2, L2 = oracle.merge_lse(O, L)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    np.testing.assert_allclose(L1, L2, atol=1e-13)
    # all partials empty for a row -> that row stays (0, -inf)
    L[:, 4, 1] = -np.inf
    O[:, 4, 1] = 0
    O3, L3 = oracle.merge_lse(O, L)
    assert np.isneginf(L3[4, 1]) and np.all(O3[4, 1] == 0)
    # a single partial merges to itself
    O4, L4 = oracle.merge_lse(O[:1], L[:1])
    np.testing.assert_array_equal(L4, L[0])
    np.testing.assert_allclose(O4, O[0], atol=0)


def _loss(p, dO, **over):
    q = dict(p, **over)
    O, _ = oracle.attention(q["Q"], q["K"], q["V"], q["Kd"], q["Vd"],
                            q["anchors"], q["lo"], q["scale"])
    return float((O * dO).sum())


def _oracle_grads(p, dO):
    O, L = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                            p["anchors"], p["lo"], p["scale"])
    pos = np.arange(p["K"].shape[0])
    return oracle.attention_bwd(p["Q"], p["K"], p["V"], pos, p["anchors"],
                                p["lo"], p["scale"], O, dO, L, p["Kd"], p["Vd"])


def test_bwd_central_finite_differences():
    p = tiny_problem(11, nb=2, ctx=48, hq=4, hkv=2, d=8, nseq=2)
    rng = np.random.default_rng(4)
    dO = rng.standard_normal(p["Q"].shape)
    grads = dict(zip(("Q", "K", "V", "Kd", "Vd"), _oracle_grads(p, dO)))
    h = 1e-6
    for name, g in grads.items():
        x = p[name]
        flat = rng.choice(x.size, size=12, replace=False)
        for f in flat:
            idx = np.unravel_index(f, x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            num = (_loss(p, dO, **{name: xp}) - _loss(p, dO, **{name: xm})) / (2 * h)
            assert g[idx] == pytest.approx(num, abs=2e-8, rel=1e-6), (name, idx)


@pytest.mark.parametrize("seed", [12, 13])
def test_bwd_matches_torch_autograd_dense(seed):
    p = tiny_problem(seed, nb=3, ctx=64, nseq=2)
    dO = np.random.default_rng(seed).standard_normal(p["Q"].shape)
    mine = _oracle_grads(p, dO)
    Ot, _, leaves = torch_dense(p, requires_grad=True)
    (Ot * torch.tensor(dO)).sum().backward()
    for a, t in zip(mine, leaves):
        np.testing.assert_allclose(a, t.grad.numpy(), atol=1e-12)


def test_bwd_constant_v_and_dv_sum():
    p = tiny_problem(14, nseq=2)
    dO = np.random.default_rng(5).standard_normal(p["Q"].shape)
    dQ, dK, dV, dKd, dVd = _oracle_grads(p, dO)
    # sum over keys of dV equals the sum of dO over the q-heads of each kv head
    G = p["Q"].shape[1] // p["K"].shape[1]
    for g in range(p["K"].shape[1]):
        want = dO[:, g * G:(g + 1) * G].sum(axis=(0, 1))
        np.testing.assert_allclose(dV[:, g].sum(0) + dVd[:, g].sum(0), want,
                                   atol=1e-12)
    c = np.random.default_rng(6).standard_normal((p["K"].shape[1], p["K"].shape[2]))
    p["V"][:] = c[None]
    p["Vd"][:] = c[None]
    dQ, dK, dV, dKd, dVd = _oracle_grads(p, dO)
    assert np.abs(dQ).max() < 1e-13 and np.abs(dK).max() < 1e-13
    assert np.abs(dKd).max() < 1e-13


def test_bwd_split_over_shards():
    """Shard dQ shares sum to dQ; each shard's dK/dV are its rows of the
    unsplit gradients.  Using a shard's own partial O/LSE instead of the
    merged ones gives a different (wrong) dQ."""
    p = tiny_problem(15, nb=4, ctx=100, nseq=2)
    dO = np.random.default_rng(7).standard_normal(p["Q"].shape)
    O, L = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                            p["anchors"], p["lo"], p["scale"])
    full = _oracle_grads(p, dO)
    parts = _random_partition(np.random.default_rng(8), p["K"].shape[0], 3)
    shares = []
    for j, idx in enumerate(parts):
        wd = j == 0
        dq, dk, dv, dkd, dvd = oracle.attention_bwd(
            p["Q"], p["K"][idx], p["V"][idx], idx, p["anchors"], p["lo"],
            p["scale"], O, dO, L, p["Kd"] if wd else None, p["Vd"] if wd else None)
        shares.append(dq)
        np.testing.assert_allclose(dk, full[1][idx], atol=1e-12)
        np.testing.assert_allclose(dv, full[2][idx], atol=1e-12)
        if wd:
            np.testing.assert_allclose(dkd, full[3], atol=1e-12)
            np.testing.assert_allclose(dvd, full[4], atol=1e-12)
    # the finalized dQ of the shares is the unsplit dQ (and no share alone is)
    np.testing.assert_allclose(oracle.dq_finalize(np.stack(shares)), full[0], atol=1e-12)
    assert all(np.abs(sh - full[0]).max() > 1e-3 for sh in shares)
    # negative: the shard's partial statistics are not the ones to use
    idx = parts[1]
    o1, l1 = oracle.attention_partial(p["Q"], p["K"][idx], p["V"][idx], idx,
                                      p["anchors"], p["lo"], p["scale"])
    l1 = np.where(np.isfinite(l1), l1, 0.0)
    dq_wrong = oracle.attention_bwd(p["Q"], p["K"][idx], p["V"][idx], idx,
                                    p["anchors"], p["lo"], p["scale"], o1, dO,
                                    l1)[0]
    dq_right = oracle.attention_bwd(p["Q"], p["K"][idx], p["V"][idx], idx,
                                    p["anchors"], p["lo"], p["scale"], O, dO,
                                    L)[0]
    assert np.abs(dq_wrong - dq_right).max() > 1e-3


def test_mutation_non_strict_mask_is_caught(monkeypatch):
    """Planting '<=' in the mask must break the Q = 0 closed form."""
    def bad(anchors, lo, pos):
        a = np.asarray(anchors, np.int64)[:, None]
        l = np.asarray(lo, np.int64)[:, None]
        q = np.asarray(pos, np.int64)[None, :]
        return (q >= l) & (q <= a)
    p = tiny_problem(16, nb=3, ctx=60)
    p["anchors"] = np.minimum(p["anchors"], 50).astype(np.int32)
    p["Q"][:] = 0
    monkeypatch.setattr(oatt, "visible_context", bad)
    _, L = oatt.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                          p["anchors"], p["lo"], p["scale"])
    want = np.log(p["anchors"].astype(float) - p["lo"] + BLOCK)
    assert not np.allclose(L[::BLOCK, 0], want)


def test_mutation_dropped_draft_keys_is_caught():
    p = tiny_problem(17)
    Ot, Lt, _ = torch_dense(p)
    O, L = oracle.attention(p["Q"], p["K"], p["V"], None, None,
                            p["anchors"], p["lo"], p["scale"])
    assert np.abs(L - Lt.numpy()).max() > 1e-3


def test_generator_bf16_rounding_and_shapes():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.0e-3, 65504.0], np.float32)
    r = wl.round_to_bf16(x)
    t = torch.tensor(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(r, t)
    w, g, t = wl.make("tiny_f32_ctx1k", 0)
    assert t.Q.shape == (64, 2, 64) and t.K.shape == (1024, 2, 64)
    assert np.all(np.diff(g.anchors) > 0) and g.anchors.min() >= 256
    assert g.chunk_pos.tolist() == list(range(0, 1024, 128))
    w3 = wl.scaled(wl.WORKLOADS["varlen8_fwdbwd"], len_median=512, len_min=128,
                   len_max=2048, blocks_per_seq=4)
    _, g3, t3 = wl.make(w3, 3)
    assert np.all((g3.anchors >= g3.lo))
    for s in range(8):
        sl = slice(4 * s, 4 * s + 4)
        assert np.all(g3.anchors[sl] < g3.seq_start[s] + g3.seq_len[s])


def test_bwd_block_subset_gives_exact_dq_rows():
    p = tiny_problem(18, nb=4, ctx=90, nseq=2)
    dO = np.random.default_rng(9).standard_normal(p["Q"].shape)
    O, L = oracle.attention(p["Q"], p["K"], p["V"], p["Kd"], p["Vd"],
                            p["anchors"], p["lo"], p["scale"])
    pos = np.arange(p["K"].shape[0])
    full = oracle.attention_bwd(p["Q"], p["K"], p["V"], pos, p["anchors"], p["lo"],
                                p["scale"], O, dO, L, p["Kd"], p["Vd"])
    parts = [oracle.attention_bwd(p["Q"], p["K"], p["V"], pos, p["anchors"], p["lo"],
                                  p["scale"], O, dO, L, p["Kd"], p["Vd"], blocks=b)
             for b in ([0, 2], [1, 3])]
    np.testing.assert_array_equal(parts[0][0][:16], full[0][:16])
    np.testing.assert_array_equal(parts[1][0][16:32], full[0][16:32])
    for k in range(1, 5):
        np.testing.assert_allclose(parts[0][k] + parts[1][k], full[k], atol=1e-13)
