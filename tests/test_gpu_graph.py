"""The step's launches captured in a HIP graph: every replay gives the bits
of the same launches run eagerly.  The library allocates nothing and sets no
memory on its own, so its kernels can be captured as they are; replays run
the captured arguments again (the step number t, so the bias correction, is
the one captured), and the host-side counters count the capture once."""
import pytest
import torch

import workloads as wl
import zero_sharded_mixed_reduce_amd as z
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


def _bits(share):
    return [share.master.view(torch.int32).clone(), share.m.view(torch.int32).clone(),
            share.v.view(torch.int32).clone(), share.wc.view(torch.int16).clone()]


@pytest.mark.parametrize("rank,world,defer", [(3, 32, 3), (0, 8, 3), (5, 64, 0)])
def test_graph_replays_match_eager_steps(rank, world, defer):
    S = 1_000_003
    w = wl.Workload("graphshare", "one_rank_share_graph", world * S, world, 2, "bf16", 1e-3, 1e-4, 3)
    say(f"[graph] rank={rank} world={world} defer={defer}")
    z.zsmr_set_launch_shape(0, 0, defer, 24)
    try:
        eager = wl.RankShare(w, rank=rank)
        eager.gen_grads(1)
        graphed = wl.RankShare(w, rank=rank)
        graphed.gen_grads(1)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            graphed.step(1)
        # capture records the launches without running them
        torch.cuda.synchronize()
        other = torch.empty(1 << 20, device="cuda")
        for replay in range(4):
            eager.step(1)
            torch.cuda.synchronize()
            want = _bits(eager)
            other.fill_(replay)             # eager work on the same device between replays
            g.replay()
            torch.cuda.synchronize()
            got = _bits(graphed)
            for a, b in zip(got, want):
                assert torch.equal(a, b), f"replay {replay}"
        c = z.zero_counters(graphed.ctx, rank)
        assert c["ag_elems"] == (world - 1) * S      # the capture counted one step
    finally:
        z.zsmr_set_launch_shape(0, 0, 3, 24)
