"""Parity at the workloads' full sizes, run exactly as bench.py runs them
(same drivers, same launch shape).  The oracle recomputes sampled elements
one by one from regenerated inputs (boundary windows of every shard and unit,
the ends of each launch's vector range, and random indices); every element is
also checked against properties that hold at any size: the 16-bit working
copy is torch's round-to-nearest-even cast of the fp32 master, received peer
slots equal what was staged, and the counters equal the accounting."""
import gc

import numpy as np
import pytest
import torch

import workloads as wl
import zero_sharded_mixed_reduce_amd as z
from oracle import accounting as acc
from oracle import sampled
from oracle.layout import make_layout
from tests.gpu_helpers import compare, host16, say

pytestmark = pytest.mark.gpu

WINDOW = 2048
N_RANDOM = 1 << 20          # random indices sampled per full-size check


def windows(starts_ends, lo, hi, n_random, seed):
    """Positions in [lo, hi): WINDOW-wide windows at each listed position and
    n_random uniform ones."""
    pos = []
    for p in starts_ends:
        a = max(lo, min(p, hi) - WINDOW // 2)
        b = min(hi, a + WINDOW)
        pos.append(np.arange(a, b, dtype=np.int64))
    rng = np.random.default_rng(seed)
    pos.append(rng.integers(lo, hi, n_random, dtype=np.int64))
    return np.unique(np.concatenate(pos))


def gather_at(t: torch.Tensor, pos: np.ndarray) -> torch.Tensor:
    return t[torch.from_numpy(pos).to(t.device)]


def cast_matches(master: torch.Tensor, p16: torch.Tensor, dtype: str, chunk=1 << 27) -> int:
    """Elements where p16 differs from torch's RNE cast of master (on the GPU)."""
    bad = 0
    for lo in range(0, master.numel(), chunk):
        ref = master[lo:lo + chunk].to(wl.TORCH16[dtype]).view(torch.int16)
        bad += int((ref != p16[lo:lo + chunk].view(torch.int16)).sum().item())
    return bad


def free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def check_sampled(w, par_idx, master, m, v, p16, what):
    want = sampled.trajectory(par_idx, w.world, w.steps, w.dtype, w.grad_sigma, w.lr, w.betas, w.eps,
                              w.seed, w.outlier_permyriad, w.theta_sigma)
    return compare({"master": master, "m": m, "v": v}, {"master": want[0], "m": want[1], "v": want[2]},
                   p16, want[3], what)


@pytest.mark.parametrize("key", ["gpt2s", "gpt2xl"])
def test_sharded_world_full_size(key):
    w = wl.WORKLOADS[key]
    say(f"[full] {key}: numel={w.numel} world={w.world} stage={w.stage} T={w.steps}")
    world = wl.ShardedWorld(w)
    world.run(w.steps)
    torch.cuda.synchronize()
    S, P = world.S, world.P
    marks = []
    for r in range(w.world):
        marks += [r * S, (r + 1) * S - 1]
    # fp32 byte offsets 2^31 and 2^32 (elements 2^29, 2^30) where they exist
    marks += [P - 1, P // 2] + [e for e in (1 << 29, 1 << 30) if e < w.numel]
    pos = windows(marks, 0, w.numel, N_RANDOM, seed=len(key))
    check_sampled(w, pos, gather_at(world.master, pos).cpu().numpy(), gather_at(world.m, pos).cpu().numpy(),
                  gather_at(world.v, pos).cpu().numpy(), host16(gather_at(world.wc, pos)), f"{key} sampled")
    assert cast_matches(world.master, world.wc, w.dtype) == 0
    if P > w.numel:
        assert not world.master[w.numel:].any() and not world.wc[w.numel:].view(torch.int16).any()
    lay = make_layout(w.numel, w.world, w.stage, pad=w.pad)
    want = acc.bytes_per_rank(lay)
    for r in range(w.world):
        c = z.zero_counters(world.ctx, r)
        assert (c["rs_elems"], c["ag_elems"]) == (w.steps * want.rs_elems, w.steps * want.ag_elems)
    del world
    free()


@pytest.mark.parametrize("rank", [0, 63])
def test_rank_share_full_size(rank):
    """One rank of the 7.5e9 / 64 world: S = 117,187,500 is 4 modulo 8, so an
    odd rank's slot in the working copy is only 8-byte aligned."""
    w = wl.WORKLOADS["share64"]
    say(f"[full] share64 rank={rank}")
    share = wl.RankShare(w, rank=rank)
    share.run(w.steps)
    torch.cuda.synchronize()
    S, off, P = share.S, share.off, share.P
    pos = windows([0, S - 1, S // 2, (S // 512) * 512, S - 600], 0, S, N_RANDOM, seed=rank)
    check_sampled(w, off + pos, gather_at(share.master, pos).cpu().numpy(),
                  gather_at(share.m, pos).cpu().numpy(), gather_at(share.v, pos).cpu().numpy(),
                  host16(gather_at(share.wc, off + pos)), f"share64 rank {rank} sampled")
    own = share.wc[off:off + S]
    assert cast_matches(share.master, own, w.dtype) == 0
    # every peer slot of the 7.5e9-element working copy was received intact
    # (positions past 2^31 and 2^32 included)
    for lo, hi in ((0, off), (off + S, P)):
        for c in range(lo, hi, 1 << 28):
            e = min(hi, c + (1 << 28))
            assert torch.equal(share.wc[c:e].view(torch.int16), share.staged[c:e].view(torch.int16))
    lay = make_layout(w.numel, w.world, w.stage)
    want = acc.bytes_per_rank(lay)
    c = z.zero_counters(share.ctx, rank)
    assert (c["rs_elems"], c["ag_elems"]) == (w.steps * want.rs_elems, w.steps * want.ag_elems)
    del share, own
    free()


# The corners of the space bench.py's window tuner searches (cycle, write,
# margin, lead in ns): cycles 62-82 us, write windows 9-11 us, leads 2-4 us.
TUNER_CORNERS = [(62000, 9000, 1000, 2000), (62000, 11000, 1000, 4000),
                 (82000, 9000, 1000, 4000), (82000, 11000, 1000, 2000)]


def test_share64_tuner_windows_give_the_default_bits():
    """The full share64 fused step (117,187,500 elements, 64 rows, about 38
    write windows) at the corners of the tuner's search space stores the
    same bits as at the library's default window, which the full-vector
    test checks against the oracle on every element: the window the bench
    picks on a device changes only when results are stored."""
    w = wl.WORKLOADS["share64"]
    say("[full] share64 fused step at the tuner's corner windows")
    share = wl.RankShare(w, rank=5)
    start = [x.clone() for x in (share.master, share.m, share.v)]
    own = share.wc[share.off:share.off + share.S]
    share.gen_grads(1)

    def run(window):
        for x, x0 in zip((share.master, share.m, share.v), start):
            x.copy_(x0)
        own.zero_()
        z.zsmr_set_write_window(*window)
        try:
            plan = z.zsmr_fused_step_plan(share.ctx, share.rank, 0, share.grads, share.row_stride, 0,
                                          share.master, share.m, share.v, own)
            assert plan["kernel"] == "deferred" and plan["windowed"], plan
            share.fused(1)
            torch.cuda.synchronize()
        finally:
            z.zsmr_set_write_window()
        return [x.clone() for x in (share.master, share.m, share.v, own)]

    ref = run(z.WRITE_WINDOW_DEFAULT)
    for window in TUNER_CORNERS:
        got = run(window)
        for name, a, b in zip(("master", "m", "v", "p16"), ref, got):
            ai = a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16)
            bi = b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)
            assert torch.equal(ai, bi), f"window {window}: {name} differs"
        say(f"[full] window {window}: same bits as the default")
        del got
    del share, start, ref, own
    free()


@pytest.mark.parametrize("rank", [0, 63])
def test_bucketed_step_full_size(rank):
    """The share64 step as ``bench.py --buckets 8`` runs it (each bucket's
    gradients filled on a second stream, its fused launch, then the receive
    of the 63 peers' pieces of the bucket as blocks S apart): the same bits
    as the unbucketed step, in every element of master, m, v and the 7.5e9-
    element working copy, and the same counters."""
    w = wl.WORKLOADS["share64"]
    say(f"[full] share64 bucketed rank={rank}")
    ref = wl.RankShare(w, rank=rank)
    ref.gen_grads(1)
    ref.step(1)
    bk = wl.RankShare(w, rank=rank)
    side = torch.cuda.Stream()
    bk.step_bucketed(1, 8, side)
    torch.cuda.synchronize()
    for a, b in ((ref.master, bk.master), (ref.m, bk.m), (ref.v, bk.v)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    for c in range(0, ref.P, 1 << 28):
        e = min(ref.P, c + (1 << 28))
        assert torch.equal(ref.wc[c:e].view(torch.int16), bk.wc[c:e].view(torch.int16))
    assert z.zero_counters(ref.ctx, rank) == z.zero_counters(bk.ctx, rank)
    del ref, bk
    free()


def test_stage3_llama8b_full_size():
    w = wl.WORKLOADS["llama8b"]
    say(f"[full] llama8b: units={len(w.units)} numel={w.numel}")
    s3 = wl.Stage3World(w, check_gathers=True)
    s3.run(w.steps)
    torch.cuda.synchronize()
    assert s3.gather_mismatch == 0
    lay = make_layout(w.numel, w.world, 3, list(w.units))
    marks = []
    for u in range(lay.n_units):
        for r in range(w.world):
            off, n = lay.owned(r, u)
            marks += [off, off + n - 1]
    marks += [(1 << 31), (1 << 32), lay.padded_numel - 1]
    pos = windows(marks, 0, lay.padded_numel, N_RANDOM, seed=8)
    par, ok = lay.padded_to_param(pos)
    assert ok.all()                                   # every unit divides by 8: no pad
    check_sampled(w, par, gather_at(s3.master, pos).cpu().numpy(), gather_at(s3.m, pos).cpu().numpy(),
                  gather_at(s3.v, pos).cpu().numpy(), host16(gather_at(s3.p16, pos)), "llama8b sampled")
    assert cast_matches(s3.master, s3.p16, w.dtype) == 0
    want = acc.bytes_per_rank(lay)
    for r in range(w.world):
        c = z.zero_counters(s3.ctx, r)
        assert (c["rs_elems"], c["ag_elems"]) == (w.steps * want.rs_elems, w.steps * want.ag_elems)
    c = z.zero_counters(s3.ctx, 0)
    assert c["stage3_gathers"] == 2 * lay.n_units * w.steps == c["stage3_releases"]
    assert c["peak_live_bytes"] == want.gathered and c["live_units"] == 0
    del s3
    free()


@pytest.mark.parametrize("defer", [0, 5])
def test_piece_larger_than_one_launch(defer):
    """A piece of 2^30 + 1,029 elements: the host cuts it into a launch of
    2^30 elements and one of the rest (a partial wave tile plus a ragged
    tail); 9 rows on 128-byte lines, so that defer=0 runs the direct kernel
    and defer=5 the deferred-write kernel across the cut (the library's plan
    says so); checked around the cut and at the ends."""
    import synth
    import synth.gpu as sgpu
    z.zsmr_set_launch_shape(0, 0, defer, 1)
    try:
        n, world, T, lr = (1 << 30) + 1029, 9, 2, 1e-3
        stride = (n + 63) // 64 * 64
        say(f"[full] piece over 2^30: n={n} stride={stride} defer={defer}")
        ctx = z.zero_init_shards(n * world, world, 2, "bf16")
        grads = torch.empty(world * stride, dtype=torch.bfloat16, device="cuda")
        theta = torch.empty(n, dtype=torch.float32, device="cuda")
        sgpu.fill32(theta, n, 0, n, 0, synth.TAG_THETA, 0, 0, 0.02)
        master, m, v = torch.empty_like(theta), torch.empty_like(theta), torch.empty_like(theta)
        p16 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        plan = z.zsmr_fused_step_plan(ctx, 0, 0, grads, stride, 0, master, m, v, p16)
        assert plan["kernel"] == ("deferred" if defer else "direct") and plan["launches"] == 2, plan
        z.zero_init_state(ctx, 0, 0, theta, master, m, v, p16)
        del theta
        for t in range(1, T + 1):
            sgpu.fill16(grads, world, stride, n, 0, n, 0, synth.TAG_GRAD, 0, t, 1e-3, "bf16")
            z.zero_fused_step(ctx, 0, 0, grads, stride, 0, master, m, v, p16, t, lr)
        torch.cuda.synchronize()
        pos = windows([0, 1 << 30, n - 1, (1 << 30) - 512, n - 1029], 0, n, 1 << 14, seed=30)
        want = sampled.trajectory(pos, world, T, "bf16", 1e-3, lr)
        compare({"master": gather_at(master, pos).cpu().numpy(), "m": gather_at(m, pos).cpu().numpy(),
                 "v": gather_at(v, pos).cpu().numpy()},
                {"master": want[0], "m": want[1], "v": want[2]}, host16(gather_at(p16, pos)), want[3],
                f"piece over 2^30 defer={defer}")
        assert cast_matches(master, p16, "bf16") == 0
        del grads, master, m, v, p16
    finally:
        z.zsmr_set_launch_shape()
        free()


def test_stage3_gather_more_ranks_than_one_launch():
    """A ZeRO-3 gather over 100 ranks takes two launches (64 shard pointers
    each at most); padded units; every gathered unit equals its shards."""
    world, units = 100, [100 * 37, 100 * 5 + 3, 7]
    numel = sum(units)
    ctx = z.zero_init_shards(numel, world, 3, "fp16", pad=True, units=units)
    info = ctx.info()
    shards = torch.arange(info["padded_numel"], dtype=torch.int32, device="cuda").to(torch.int16)
    buf = torch.full((info["max_unit_numel"] + 8,), -1, dtype=torch.int16, device="cuda")
    for u in range(len(units)):
        q0, su, _ = z.zero_layout(ctx, 0, u)
        ptrs = [shards[z.zero_layout(ctx, r, u)[0]:] for r in range(world)]
        z.zero_stage3_unit_gather(ctx, u, ptrs, buf)
        torch.cuda.synchronize()
        assert torch.equal(buf[:world * su], shards[q0:q0 + world * su]), f"unit {u}"
        if u == 0:                       # the widest unit: nothing written past it
            assert bool((buf[world * su:] == -1).all())
        z.zero_stage3_unit_release(ctx, u)
    c = z.zero_counters(ctx, 17)
    lay = make_layout(numel, world, 3, units, pad=True)
    assert c["ag_elems"] == (world - 1) * lay.shard_numel


def _small_stage3():
    units = (3 * 1 << 20, 1 << 20, 5 * 1 << 19, 1 << 20)
    return wl.Workload("s3small", "stage3_small_4_units_n8_bf16", sum(units), 8, 3, "bf16", 1e-3, 1e-4,
                       2, units=units)


def test_stage3_prefetch_matches_plain_schedule():
    """Gathering the next unit on a second stream while the current one is in
    use (two units live) gives the same bits as the plain schedule; only the
    peak changes, to the largest pair of adjacent units."""
    w = _small_stage3()
    plain = wl.Stage3World(w, check_gathers=True)
    plain.run(w.steps)
    pre = wl.Stage3World(w, check_gathers=True, prefetch=True)
    pre.run(w.steps)
    torch.cuda.synchronize()
    assert plain.gather_mismatch == 0 and pre.gather_mismatch == 0
    for a, b in ((plain.master, pre.master), (plain.m, pre.m), (plain.v, pre.v)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(plain.p16.view(torch.int16), pre.p16.view(torch.int16))
    lay = make_layout(w.numel, w.world, 3, list(w.units))
    c_plain, c_pre = z.zero_counters(plain.ctx, 0), z.zero_counters(pre.ctx, 0)
    assert c_pre["stage3_gathers"] == c_plain["stage3_gathers"] == 2 * lay.n_units * w.steps
    assert c_pre["ag_elems"] == c_plain["ag_elems"]
    assert c_plain["peak_live_bytes"] == acc.bytes_per_rank(lay, max_live=1).gathered
    assert c_pre["peak_live_bytes"] == acc.bytes_per_rank(lay, max_live=2).gathered
    del plain, pre
    free()


@pytest.mark.parametrize("n_buckets", [1, 3, 16])
def test_bucketed_step_matches_one_launch(n_buckets):
    """Gradients arriving in buckets (last parameters first, filled on a
    second stream) and consumed bucket by bucket give the same bits as one
    fused launch over the shard."""
    S = 2_000_003
    w = wl.Workload("share64small", "one_rank_share_small_n64_zero2_bf16", 64 * S, 64, 2, "bf16",
                    1e-3, 1e-4, 2)
    ref = wl.RankShare(w, rank=5)
    ref.run(w.steps)
    bk = wl.RankShare(w, rank=5)
    side = torch.cuda.Stream()
    for t in range(1, w.steps + 1):
        bk.step_bucketed(t, n_buckets, side)
    torch.cuda.synchronize()
    for a, b in ((ref.master, bk.master), (ref.m, bk.m), (ref.v, bk.v)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(ref.wc.view(torch.int16), bk.wc.view(torch.int16))
    assert z.zero_counters(ref.ctx, 5) == z.zero_counters(bk.ctx, 5)
    del ref, bk
    free()


def test_fused_ranges_with_ragged_unaligned_cuts():
    """Sub-ranges whose ends fall anywhere (odd offsets, so the 16-byte
    vector path and the one-element path both run) give the bits of one
    zero_fused_step over the shard, and count the same traffic."""
    w = wl.Workload("cuts", "one_rank_share_ragged_cuts_n64_zero2_bf16", 64 * 300_007, 64, 2,
                    "bf16", 1e-3, 1e-4, 2)
    ref, cut = wl.RankShare(w, rank=63), wl.RankShare(w, rank=63)
    S = ref.S
    edges = [0, 1, 513, 777, 4096, 150_001, S - 3, S]
    for t in (1, 2):
        ref.gen_grads(t)
        cut.gen_grads(t)
        ref.fused(t)
        for b0, b1 in zip(edges[:-1], edges[1:]):
            z.zero_fused_step_range(cut.ctx, 63, 0, b0, b1 - b0, cut.grads, cut.row_stride, 0,
                                    cut.master, cut.m, cut.v, cut.wc[cut.off:], t, w.lr, w.betas,
                                    w.eps)
    torch.cuda.synchronize()
    for a, b in ((ref.master, cut.master), (ref.m, cut.m), (ref.v, cut.v)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(ref.wc.view(torch.int16), cut.wc.view(torch.int16))
    assert z.zero_counters(ref.ctx, 63) == z.zero_counters(cut.ctx, 63)
    del ref, cut
    free()


# ------------------------------------------------- owner-broadcast ZeRO-3 --
_OWNER_UNITS = (300_001, 1 << 17, 250_003, (1 << 17) - 1, 64, 200_000)
OWNER_CASES = {
    # uneven units, an odd world, owners chosen out of order (rank 2 owns
    # nothing, rank 3 two units that are not neighbours): pieces start at any
    # alignment
    "explicit": (_OWNER_UNITS, 5, (3, 0, 3, 1, 4, 0)),
    # the pages' partition: U = k*N equal units, k consecutive ones per rank
    "pages": ((40_000,) * 15, 5, None),
}


@pytest.mark.parametrize("prefetch", [False, True])
@pytest.mark.parametrize("case", list(OWNER_CASES))
def test_owner_broadcast_matches_oracle(case, prefetch):
    """Whole units owned by single ranks, owners given explicitly (the same
    map to the library and to the oracle): every element against the
    oracle's owner-broadcast scheme, every rank's counters against the
    per-rank accounting, and gathered units against the owners' copies."""
    import synth
    from oracle import schemes as sc
    from oracle.layout import pages_owners
    units, world, owners = OWNER_CASES[case]
    if owners is None:
        owners = pages_owners(len(units), world)
    w = wl.Workload("owner_small", f"stage3_owner_small_{case}", sum(units), world, 3, "bf16", 1e-2,
                    1e-3, 2, units=units)
    say(f"[owner] {case} prefetch={prefetch} owners={owners}")
    s3 = wl.Stage3World(w, check_gathers=True, owner=True, prefetch=prefetch, owners=owners)
    s3.run(w.steps)
    torch.cuda.synchronize()
    assert s3.gather_mismatch == 0
    p = np.arange(w.numel)
    theta = synth.theta0(w.seed, p, w.theta_sigma)
    g = lambda t: [synth.grad16(w.seed, r, t, p, w.grad_sigma, w.dtype) for r in range(w.world)]
    ref = sc.run(3, w.numel, w.world, theta, g, w.steps, w.dtype, w.lr, units=list(w.units),
                 owner_broadcast=True, owners=owners)
    compare({"master": s3.master.cpu().numpy(), "m": s3.m.cpu().numpy(), "v": s3.v.cpu().numpy()},
            {"master": ref.full_master(), "m": ref.full_m(), "v": ref.full_v()},
            host16(s3.p16), ref.working_copy(), f"owner broadcast {case}")
    assert np.array_equal(s3.master.cpu().numpy().view(np.uint32), ref.full_master().view(np.uint32))
    assert np.array_equal(host16(s3.p16), ref.working_copy())
    lay = make_layout(w.numel, w.world, 3, list(w.units), owner_broadcast=True, owners=owners)
    assert [z.zero_unit_owner(s3.ctx, u) for u in range(lay.n_units)] == list(owners)
    ml = 2 if prefetch else 1
    for r in range(w.world):
        c = z.zero_counters(s3.ctx, r)
        want = acc.bytes_per_rank(lay, max_live=ml, rank=r)
        assert (c["rs_elems"], c["ag_elems"]) == (w.steps * want.rs_elems, w.steps * want.ag_elems)
        assert (c["rs_elems"], c["ag_elems"]) == (ref.rs_elems[r], ref.ag_elems[r])
        assert c["peak_live_bytes"] == want.gathered, r
        assert c["live_units"] == 0
    c0 = z.zero_counters(s3.ctx, 0)
    assert c0["stage3_gathers"] == 2 * lay.n_units * w.steps == c0["stage3_releases"]
    del s3
    free()


def test_owner_broadcast_llama8b_full_size():
    """The Llama-3-8B shape with whole units owned by ranks (the explicit
    map: embeddings and head alone on rank 0, the layers in contiguous runs
    on ranks 1-7): sampled elements against the oracle, the whole 16-bit copy
    against the cast of the master, and the counters of every rank."""
    base = wl.WORKLOADS["llama8b"]
    w = wl.Workload("llama8b_owner", "llama3_8b_shape_33_units_n8_zero3_owner_bf16", base.numel,
                    base.world, 3, base.dtype, base.grad_sigma, base.lr, base.steps, units=base.units)
    say(f"[full] llama8b owner broadcast: units={len(w.units)}")
    s3 = wl.Stage3World(w, check_gathers=True, owner=True, owners=wl.LLAMA8B_OWNERS)
    s3.run(w.steps)
    torch.cuda.synchronize()
    assert s3.gather_mismatch == 0
    lay = make_layout(w.numel, w.world, 3, list(w.units), owner_broadcast=True,
                      owners=wl.LLAMA8B_OWNERS)
    marks = []
    for u in range(lay.n_units):
        marks += [lay.unit_start[u], lay.unit_start[u] + lay.units[u] - 1]
    marks += [(1 << 31), (1 << 32), w.numel - 1]
    pos = windows(marks, 0, w.numel, N_RANDOM, seed=9)
    check_sampled(w, pos, gather_at(s3.master, pos).cpu().numpy(), gather_at(s3.m, pos).cpu().numpy(),
                  gather_at(s3.v, pos).cpu().numpy(), host16(gather_at(s3.p16, pos)),
                  "llama8b owner sampled")
    assert cast_matches(s3.master, s3.p16, w.dtype) == 0
    for r in range(w.world):
        c = z.zero_counters(s3.ctx, r)
        want = acc.bytes_per_rank(lay, rank=r)
        assert (c["rs_elems"], c["ag_elems"]) == (w.steps * want.rs_elems, w.steps * want.ag_elems)
        assert c["peak_live_bytes"] == want.gathered
    del s3
    free()
