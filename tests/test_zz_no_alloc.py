"""GPU check of the allocation-free forward (skv_attn_fwd_partial_noalloc):
it must give the same O and LSE as skv_attn_fwd_partial with a caller
workspace, on two calls in a row, the second with a smaller problem (the
static scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from block_sparse_split_amd import shards, splitkv as skv, workloads as wl
from gpu_util import announce

pytestmark = pytest.mark.gpu


def _problem(seed, ctx, nb_per_seq, lo, hi):
    w = wl.scaled(wl.WORKLOADS["ctx32k_q2k"], ctx=ctx, anchor_lo=lo, anchor_hi=hi,
                  blocks_per_seq=nb_per_seq)
    return wl.make(w, seed)


@pytest.mark.parametrize("n_wg", [256, 7])
def test_noalloc_forward_equals_workspace_forward(n_wg):
    dev = "cuda"
    used = 0
    for case, (ctx, nbs, lo, hi) in enumerate([(8192, 48, 2048, 8192), (2048, 8, 512, 2048)]):
        w, g, t = _problem(11 + case, ctx, nbs, lo, hi)
        announce("noalloc fwd", n_wg, case, ctx)
        prob = shards.whole_context_problem(w, g)
        sh = skv.Shard(prob, device=dev, n_workgroups=n_wg)
        used += sh.info.n_split_qtiles > 0
        to = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
        Q, K, V, Kd, Vd = (to(x) for x in (t.Q, t.K, t.V, t.Kd, t.Vd))
        outs = {}
        for kind in ("workspace", "noalloc"):
            O = torch.full((w.nq, w.hq, w.d), float("nan"), dtype=torch.bfloat16, device=dev)
            L = torch.full((w.nq, w.hq), float("nan"), dtype=torch.float32, device=dev)
            if kind == "workspace":
                sh.fwd(Q, K, V, Kd, Vd, O, L)
            else:
                sh.fwd_noalloc(Q, K, V, Kd, Vd, O, L)
            torch.cuda.synchronize()
            outs[kind] = (O, L)
        (O1, L1), (O2, L2) = outs["workspace"], outs["noalloc"]
        assert torch.isfinite(O2).all() and not torch.isnan(L2).any()
        assert torch.equal(O1, O2), f"case {case}: O differs"
        assert torch.equal(L1, L2), f"case {case}: LSE differs"
    # the scratch (partial slots of split query tiles) was really used
    assert used > 0
