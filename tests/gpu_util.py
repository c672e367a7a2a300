"""Helpers for the GPU parity tests (imported by test modules only)."""
import numpy as np
import torch

import oracle
from block_sparse_split_amd import splitkv as skv
from block_sparse_split_amd import shards
from block_sparse_split_amd import workloads as wl

TOL = {"f32": dict(o=1e-5, lse=1e-5, grad=1e-5), "bf16": dict(o=2e-2, lse=1e-3, grad=2e-2)}


def announce(*what):
    print("[case]", *what, flush=True)


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def rows_of(t: wl.Tensors, g: wl.Geometry, chunk_ids):
    """Local rows (into t.K/t.V) of the given chunks, in the given order."""
    start = {}
    off = 0
    for c in t.chunk_ids:
        start[int(c)] = off
        off += int(g.chunk_len[c])
    idx = [np.arange(start[int(c)], start[int(c)] + int(g.chunk_len[c])) for c in chunk_ids]
    return np.concatenate(idx).astype(np.int64) if idx else np.zeros(0, np.int64)


def gpu_fwd(w, g, t, chunk_ids, with_draft, n_wg=0, o_dtype=None, shard=None):
    """Run skv_attn_fwd_partial for one shard; returns (O, LSE) on host."""
    prob = shards.shard_problem(w, g, chunk_ids, with_draft)
    sh = shard or skv.Shard(prob, n_workgroups=n_wg)
    r = rows_of(t, g, chunk_ids)
    Q = to_dev(t.Q, w.dtype)
    K = to_dev(t.K[r], w.dtype)
    V = to_dev(t.V[r], w.dtype)
    Kd = to_dev(t.Kd, w.dtype) if with_draft else None
    Vd = to_dev(t.Vd, w.dtype) if with_draft else None
    odt = o_dtype or (torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    O = torch.full((w.nq, w.hq, w.d), float("nan"), dtype=odt, device="cuda")
    LSE = torch.full((w.nq, w.hq), float("nan"), dtype=torch.float32, device="cuda")
    sh.fwd(Q, K, V, Kd, Vd, O, LSE)
    torch.cuda.synchronize()
    return O, LSE, sh


def measured_like_plan(w, prob, seed):
    """Per-XCD speeds and per-(kv head, query tile) cost scales spread as
    measured ones are (a few per cent): the kind of plan the benchmark
    times, built for every CU."""
    rng = np.random.default_rng(seed)
    speed = (1.0 + 0.04 * rng.uniform(-1, 1, (3, 8))).astype(np.float32)
    scale = rng.uniform(0.97, 1.03, (2, w.hkv, prob.qt_per_head))
    sh = skv.Shard(prob, xcd_speed=speed, cost_scale=scale)
    assert sh.info.xcd_mode == 1
    return sh, speed, scale


def oracle_partial(w, g, t, chunk_ids, with_draft, blocks=None):
    r = rows_of(t, g, chunk_ids)
    pos = shards.shard_rows(g, chunk_ids)
    return oracle.attention_partial(t.Q, t.K[r], t.V[r], pos, g.anchors, g.lo,
                                    wl.softmax_scale(w.d), t.Kd if with_draft else None,
                                    t.Vd if with_draft else None, blocks=blocks)


def block_rows(blocks):
    return np.concatenate([np.arange(16 * b, 16 * b + 16) for b in blocks])


def compare(O, LSE, Oo, Lo, dtype, what=""):
    """Element-wise check of a GPU (O, LSE) against the oracle's."""
    O = O.float().cpu().numpy().astype(np.float64) if torch.is_tensor(O) else O
    L = LSE.float().cpu().numpy().astype(np.float64) if torch.is_tensor(LSE) else LSE
    tol = TOL[dtype]
    assert np.array_equal(np.isneginf(L), np.isneginf(Lo)), f"{what}: -inf rows differ"
    assert np.all(np.isfinite(O)), f"{what}: non-finite O"
    fin = np.isfinite(Lo)
    dl = np.abs(L[fin] - Lo[fin]).max(initial=0.0)
    do = np.abs(O - Oo).max(initial=0.0)
    assert np.all(O[~fin] == 0), f"{what}: rows with no key must be 0"
    assert dl <= tol["lse"], f"{what}: LSE max-abs {dl:.3g} > {tol['lse']}"
    assert do <= tol["o"], f"{what}: O max-abs {do:.3g} > {tol['o']}"
    return do, dl
