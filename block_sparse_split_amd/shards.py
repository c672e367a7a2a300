"""Shard descriptions for simulated context-parallel participants.

A shard is a subset of the context chunks; its keys/values are those chunks'
rows stacked in chunk order.  This module only gathers rows and writes chunk
tables; the placement itself comes from the LPT planner in libsplitkv.
"""
from __future__ import annotations

import numpy as np

from . import splitkv as skv
from .workloads import Geometry, Workload, softmax_scale


def shard_rows(g: Geometry, chunk_ids) -> np.ndarray:
    """Absolute key positions of a shard's local rows, in chunk order."""
    chunk_ids = np.asarray(chunk_ids, np.int64)
    if chunk_ids.size == 0:
        return np.zeros(0, np.int64)
    return np.concatenate([np.arange(g.chunk_pos[c], g.chunk_pos[c] + g.chunk_len[c])
                           for c in chunk_ids]).astype(np.int64)


def shard_problem(w: Workload, g: Geometry, chunk_ids, with_draft: bool,
                  dtype=None) -> skv.Problem:
    chunk_ids = np.asarray(chunk_ids, np.int64)
    lens = g.chunk_len[chunk_ids] if chunk_ids.size else np.zeros(0, np.int32)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pos = g.chunk_pos[chunk_ids] if chunk_ids.size else np.zeros(0, np.int32)
    if dtype is None:
        dtype = skv.SKV_BF16 if w.dtype == "bf16" else skv.SKV_F32
    return skv.Problem(nb=w.nb, hq=w.hq, hkv=w.hkv, d=w.d, scale=softmax_scale(w.d),
                       dtype=dtype, anchors=g.anchors, lo=g.lo, chunk_pos=pos,
                       chunk_off=off, with_draft=with_draft)


def whole_context_problem(w: Workload, g: Geometry, dtype=None) -> skv.Problem:
    """Single participant holding every chunk (and the draft keys)."""
    return shard_problem(w, g, np.arange(len(g.chunk_pos)), True, dtype)


def lpt_shards(w: Workload, g: Geometry, n_shards: int, tile_k: int = None):
    """Chunk ids of each simulated participant under the LPT plan."""
    bins, cost, load = skv.skv_plan_lpt(g.anchors, g.lo, g.chunk_pos, g.chunk_len,
                                        tile_k or w.tile_k, n_shards)
    return [np.nonzero(bins == r)[0] for r in range(n_shards)], bins, cost, load
