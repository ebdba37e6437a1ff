"""Checkpoint and resume: a rank's whole optimizer state is the fp32 master,
m and v of its shard, its 16-bit working copy and the step number t, all in
caller-owned buffers (the library keeps no numeric state of its own).  So T
steps run straight must give the same bits as k steps, a save of those
buffers to host memory, a restore into freshly allocated buffers of a new
context, and T-k more steps that start from t = k+1."""
import pytest
import torch

import workloads as wl
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

T, K = 5, 2


def _state(obj):
    wc = obj.wc if hasattr(obj, "wc") else obj.p16
    return [obj.master, obj.m, obj.v, wc]


def _save(obj):
    torch.cuda.synchronize()
    return [x.cpu() for x in _state(obj)]          # synchronous copies to host


def _restore(obj, saved):
    for dst, src in zip(_state(obj), saved):
        dst.copy_(src)
    torch.cuda.synchronize()


def _bits(obj):
    torch.cuda.synchronize()
    return [x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16)
            for x in (y.cpu() for y in _state(obj))]


def _steps(obj, first, last):
    for t in range(first, last + 1):
        if not isinstance(obj, wl.Stage3World):    # stage 3 makes each unit's gradients itself
            obj.gen_grads(t)
        obj.step(t)


def _check(make, what):
    say(f"[resume] {what}")
    straight = make()
    _steps(straight, 1, T)
    want = _bits(straight)
    del straight
    first = make()
    _steps(first, 1, K)
    saved = _save(first)
    del first
    torch.cuda.empty_cache()
    resumed = make()                                # a new context and new buffers
    _restore(resumed, saved)
    _steps(resumed, K + 1, T)
    got = _bits(resumed)
    for name, a, b in zip(("master", "m", "v", "16-bit copy"), got, want):
        assert torch.equal(a, b), f"{what}: {name} differs after resume"


@pytest.mark.parametrize("world,rank", [(64, 17), (8, 0)])
def test_rank_share_resumes_bit_exact(world, rank):
    # 64 rows take the deferred-write kernel, 8 rows the direct one
    S = 300_007
    w = wl.Workload("resume_share", "one_rank_share_resume", world * S, world, 2, "bf16",
                    1e-3, 1e-4, T, seed=11)
    _check(lambda: wl.RankShare(w, rank=rank), f"rank share world={world} rank={rank}")


@pytest.mark.parametrize("stage,dtype", [(1, "fp16"), (2, "bf16")])
def test_sharded_world_resumes_bit_exact(stage, dtype):
    w = wl.Workload("resume_world", "world_resume", 1_000_003, 4, stage, dtype, 1e-2, 1e-3, T,
                    pad=True, seed=12, outlier_permyriad=50)
    _check(lambda: wl.ShardedWorld(w), f"sharded world stage={stage} {dtype}")


@pytest.mark.parametrize("owner", [False, True])
def test_stage3_world_resumes_bit_exact(owner):
    units = (70_000, 33_333, 120_001)
    w = wl.Workload("resume_s3", "stage3_resume", sum(units), 4, 3, "bf16", 1e-3, 1e-4, T,
                    units=units, pad=True, seed=13)
    _check(lambda: wl.Stage3World(w, owner=owner), f"stage 3 owner={owner}")
