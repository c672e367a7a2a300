"""fp64 CPU oracle for Split-KV draft cross-attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The product path (``block_sparse_split_amd``) never imports this package and
this package never imports the product: the two share no kernels, headers,
helpers, tables or pre/post-processing.  Only the seeded input generator
(``block_sparse_split_amd.workloads``, which holds none of the method's
arithmetic) feeds both.

Sources: the arXiv abstract of "Split-KV: Efficient Context Parallelism for
Training Diffusion Drafters" (pages aiqbench.com and feed.astralor.com) and
the rit.work blog post on Split-KV, sections "A short query sufficed for a
long context" and "Split-KV moves queries, not keys and values".

Every function here is pinned by the ``-m "not gpu"`` tests against
something other than itself (brute force, closed forms, invariants, library
routines, hand-worked fixtures under ``tests/golden/``).  No function is
"parity unpinned".
"""
from .attention_fp64 import (BLOCK, visible_context, attention_partial,
                             attention, merge_lse, attention_bwd, dq_finalize)
from .planner import (chunk_costs, tile_pairs_visible, plan_lpt,
                      plan_contiguous, imbalance, makespan)

__all__ = [
    "BLOCK", "visible_context", "attention_partial", "attention", "merge_lse",
    "attention_bwd", "dq_finalize", "chunk_costs", "tile_pairs_visible",
    "plan_lpt", "plan_contiguous", "imbalance", "makespan",
]
