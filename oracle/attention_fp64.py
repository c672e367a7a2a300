"""fp64 definition of the draft cross-attention, its split/merge and gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages state it:

* Draft queries come in anchor blocks of 16 tokens.  Block ``i`` sees the
  context keys at absolute positions ``lo_i <= j < a_i`` (its sequence start
  up to, not including, its anchor) plus the 16 draft keys of its own block,
  in both directions.  The pages say only that the short draft-query set
  attends to a much longer context through a block-sparse mask built from
  anchor positions sampled in the responses (arXiv abstract; rit.work blog,
  section "A short query sufficed for a long context").  The exact rule
  (strict ``j < a_i``, the draft block's own keys) is the reading recorded in
  the design notes.
* Partial attention over a local key shard, with the per-row log-sum-exp as
  the normaliser, and an exact merge of the partials: the blog, section
  "Split-KV moves queries, not keys and values", says each participant
  computes its local parts of attention for the full query set, the
  normalisation is then reconciled across participants, and the split
  reproduces single-device attention exactly (no approximation).  The
  normaliser is read as the natural-log LSE.
* Backward: query gradients are the only ones that cross participants (same
  blog section); K/V gradients stay with the shard that holds the keys.  The
  formulas are the standard softmax-attention gradients written out from the
  chain rule, using the final (merged) LSE and output.

All inputs are upcast to fp64; outputs are fp64.  Rows with no visible key in
a partial get ``O = 0`` and ``LSE = -inf``.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def visible_context(anchors, lo, pos):
    """Boolean [nb, n]: block i sees the context key at position pos[j] iff
    lo[i] <= pos[j] < anchors[i]."""
    a = np.asarray(anchors, np.int64)[:, None]
    l = np.asarray(lo, np.int64)[:, None]
    p = np.asarray(pos, np.int64)[None, :]
    return (p >= l) & (p < a)


def _block_keys(K, V, Kd, Vd, vis_row, i, g):
    """Keys/values visible to block i for kv head g (context, then draft)."""
    idx = np.nonzero(vis_row)[0]
    keys = K[idx, g]
    vals = V[idx, g]
    if Kd is not None:
        rows = slice(BLOCK * i, BLOCK * (i + 1))
        keys = np.concatenate([keys, Kd[rows, g]], axis=0)
        vals = np.concatenate([vals, Vd[rows, g]], axis=0)
    return idx, keys, vals


def attention_partial(Q, K, V, pos, anchors, lo, scale, Kd=None, Vd=None,
                      blocks=None):
    """Attention of the draft queries over one key subset.

    Q [Nq, Hq, d]; K, V [n, Hkv, d] with absolute positions pos[n]; Kd, Vd
    [Nq, Hkv, d] (the draft-block keys) or None when this subset does not
    hold them.  ``blocks`` restricts the computation to some anchor blocks
    (rows are independent, so a subset is exact).  Query head h reads kv
    head h // (Hq // Hkv).

    Returns O [len(blocks)*16, Hq, d] and LSE [len(blocks)*16, Hq] in fp64.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    Kd = None if Kd is None else _f64(Kd)
    Vd = None if Vd is None else _f64(Vd)
    nq, hq, d = Q.shape
    hkv = K.shape[1]
    G = hq // hkv
    nb = nq // BLOCK
    blocks = list(range(nb)) if blocks is None else list(blocks)
    vis = visible_context(anchors, lo, pos)
    O = np.zeros((len(blocks) * BLOCK, hq, d))
    LSE = np.full((len(blocks) * BLOCK, hq), -np.inf)
    for bi, i in enumerate(blocks):
        rows = slice(BLOCK * i, BLOCK * (i + 1))
        out = slice(BLOCK * bi, BLOCK * (bi + 1))
        for g in range(hkv):
            _, keys, vals = _block_keys(K, V, Kd, Vd, vis[i], i, g)
            if keys.shape[0] == 0:
                continue
            q = Q[rows, g * G:(g + 1) * G].reshape(BLOCK * G, d)
            z = scale * (q @ keys.T)
            m = z.max(axis=1, keepdims=True)
            lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
            p = np.exp(z - lse[:, None])
            O[out, g * G:(g + 1) * G] = (p @ vals).reshape(BLOCK, G, d)
            LSE[out, g * G:(g + 1) * G] = lse.reshape(BLOCK, G)
    return O, LSE


def attention(Q, K, V, Kd, Vd, anchors, lo, scale, pos=None, blocks=None):
    """Single-device attention: every context key plus the draft keys."""
    if pos is None:
        pos = np.arange(np.asarray(K).shape[0])
    return attention_partial(Q, K, V, pos, anchors, lo, scale, Kd, Vd, blocks)


def merge_lse(O_parts, LSE_parts):
    """Exact merge of K partials: O_parts [K, ..., d], LSE_parts [K, ...].

    LSE = M + ln sum_k exp(LSE_k - M) with M the largest finite LSE_k, and
    O = sum_k exp(LSE_k - LSE) O_k.  A partial with LSE_k = -inf has weight
    zero; a row whose partials are all -inf stays O = 0, LSE = -inf.
    """
    O_parts, L = _f64(O_parts), _f64(LSE_parts)
    M = L.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.exp(L - Ms[None])
    lse = np.where(finite, Ms + np.log(np.where(finite, w.sum(axis=0), 1.0)),
                   -np.inf)
    lse_s = np.where(finite, lse, 0.0)
    coef = np.where(finite[None], np.exp(L - lse_s[None]), 0.0)
    O = (coef[..., None] * O_parts).sum(axis=0)
    return O, lse


def dq_finalize(dQ_parts):
    """The query gradient from the shards' shares dQ_parts [S, ...]: their
    sum.  Each shard's share covers the keys it holds, and the query
    gradients are the ones returned to the query owner (rit.work blog,
    section "Split-KV moves queries, not keys and values"), who adds them.
    """
    return _f64(dQ_parts).sum(axis=0)


def attention_bwd(Q, K, V, pos, anchors, lo, scale, O, dO, LSE, Kd=None,
                  Vd=None, blocks=None):
    """Gradients of sum(O * dO) for the keys of one subset.

    O and LSE must be the FINAL (merged, single-device) output and
    log-sum-exp; with them, P = exp(scale * q k^T - LSE) are the true
    attention weights restricted to this subset's keys.  With
    D = rowsum(dO * O) and dP = dO V^T:
        dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
    Query heads sharing a kv head sum into its dK/dV.

    ``blocks`` restricts the sum to some anchor blocks: their dQ rows are
    then exact, while dK/dV only hold those blocks' contributions.

    Returns dQ [Nq, Hq, d] (this subset's share; shares sum to the full dQ),
    dK, dV [n, Hkv, d] and dKd, dVd [Nq, Hkv, d] (None without draft keys).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    O, dO, LSE = _f64(O), _f64(dO), _f64(LSE)
    Kd = None if Kd is None else _f64(Kd)
    Vd = None if Vd is None else _f64(Vd)
    nq, hq, d = Q.shape
    n, hkv, _ = K.shape
    G = hq // hkv
    nb = nq // BLOCK
    vis = visible_context(anchors, lo, pos)
    D = (dO * O).sum(axis=-1)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    dKd = None if Kd is None else np.zeros_like(Kd)
    dVd = None if Vd is None else np.zeros_like(Vd)
    for i in (range(nb) if blocks is None else blocks):
        rows = slice(BLOCK * i, BLOCK * (i + 1))
        for g in range(hkv):
            idx, keys, vals = _block_keys(K, V, Kd, Vd, vis[i], i, g)
            if keys.shape[0] == 0:
                continue
            hs = slice(g * G, (g + 1) * G)
            q = Q[rows, hs].reshape(BLOCK * G, d)
            do = dO[rows, hs].reshape(BLOCK * G, d)
            lse = LSE[rows, hs].reshape(BLOCK * G)
            Dv = D[rows, hs].reshape(BLOCK * G)
            p = np.exp(scale * (q @ keys.T) - lse[:, None])
            dvals = p.T @ do
            dp = do @ vals.T
            ds = p * (dp - Dv[:, None])
            dq = scale * (ds @ keys)
            dkeys = scale * (ds.T @ q)
            dQ[rows, hs] += dq.reshape(BLOCK, G, d)
            nc = idx.shape[0]
            dK[idx, g] += dkeys[:nc]
            dV[idx, g] += dvals[:nc]
            if Kd is not None:
                dKd[rows, g] += dkeys[nc:]
                dVd[rows, g] += dvals[nc:]
    return dQ, dK, dV, dKd, dVd

