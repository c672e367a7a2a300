"""Cost model and longest-processing-time-first (LPT) placement, plain Python.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages (arXiv abstract of "Split-KV: Efficient Context Parallelism for
Training Diffusion Drafters"; rit.work blog, section "Split-KV moves queries,
not keys and values") say: anchor sampling loads parts of the context
unevenly; because every participant sees all queries, the realised attention
cost of each context key/value chunk can be computed before the step; LPT
orders the chunks from most to least expensive and gives each, in turn, to
the least-loaded participant.  The imbalance the pages report (below 1%) is
read here as max(load) / mean(load) - 1 over all bins.

Readings where the pages are silent (listed in the design notes):
* cost unit: a chunk is cut into key tiles of ``tile_k`` keys laid out from
  the chunk's first key (the last tile may be short); a (query block, key
  tile) pair counts once when at least one key of the tile is visible to the
  block, i.e. the tile meets [lo_i, a_i);
* ties: equal costs are taken in increasing chunk index; equal loads go to
  the lowest bin index.  With these rules the plan is unique.
"""
from __future__ import annotations

import numpy as np


def tile_pairs_visible(anchors, lo, t0, t1):
    """Number of anchor blocks i whose visible interval [lo_i, a_i) meets the
    key interval [t0, t1)."""
    a = np.asarray(anchors, np.int64)
    l = np.asarray(lo, np.int64)
    return int(np.count_nonzero(np.maximum(l, t0) < np.minimum(a, t1)))


def chunk_costs(anchors, lo, chunk_pos, chunk_len, tile_k):
    """Realised cost of each chunk: visible (query block, key tile) pairs."""
    costs = np.zeros(len(chunk_pos), np.int64)
    for c, (p, n) in enumerate(zip(chunk_pos, chunk_len)):
        p, n = int(p), int(n)
        total = 0
        for t0 in range(p, p + n, tile_k):
            total += tile_pairs_visible(anchors, lo, t0, min(t0 + tile_k, p + n))
        costs[c] = total
    return costs


def plan_lpt(costs, m):
    """LPT placement of n jobs with integer costs on m bins.

    Jobs are taken by decreasing cost (ties: lower index first); each goes to
    the bin with the smallest current load (ties: lowest bin).  This is an
    O(n*m) scan, not a heap.  Returns (bin[n] int32, load[m] int64)."""
    costs = [int(c) for c in costs]
    order = sorted(range(len(costs)), key=lambda c: (-costs[c], c))
    load = np.zeros(m, np.int64)
    bins = np.zeros(len(costs), np.int32)
    for c in order:
        b = int(np.argmin(load))       # first minimum = lowest bin index
        bins[c] = b
        load[b] += costs[c]
    return bins, load


def plan_contiguous(n, m):
    """Equal-count contiguous split: job c goes to bin floor(c*m/n)."""
    return (np.arange(n, dtype=np.int64) * m // n).astype(np.int32)


def loads_of(costs, bins, m):
    load = np.zeros(m, np.int64)
    np.add.at(load, np.asarray(bins, np.int64), np.asarray(costs, np.int64))
    return load


def makespan(costs, bins, m):
    return int(loads_of(costs, bins, m).max())


def imbalance(load):
    """max(load)/mean(load) - 1, the mean over all bins (empty ones too)."""
    load = np.asarray(load, np.float64)
    mean = load.mean()
    return float(load.max() / mean - 1.0) if mean > 0 else 0.0
