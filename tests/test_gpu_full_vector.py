"""Whole-vector parity against the oracle: every element of master, m, v and
the 16-bit working copy, compared after every step.

* Every workload at its full size, as "ZeRO and FSDP"'s zero_check.py
  compares every parameter of the sharded run with the unsharded one:
  GPT-2 small (124,439,808 parameters, 8 ranks, ZeRO-2, 10 steps) and GPT-2
  1.5B (1,558,000,000, 16 ranks, ZeRO-1, outliers, 3 steps) after every
  step; one rank's share of the 7.5e9 / 64-rank world (117,187,500 owned
  elements, 64 rows; ranks 0 and 63) after every step; the Llama-3-8B
  shape (8,030,261,248 parameters in 33 units, ZeRO-3) after its 2 steps,
  unit by unit.
* The bucketed share step (gradients arriving bucket by bucket during a
  simulated backward, each bucket updated and received as it lands; 1, 3 and
  16 buckets, and sub-ranges cut at ragged, unaligned places) on a
  2,000,003-element share of a 64-rank world.
* The ZeRO-3 split layout with the next unit prefetched on a second stream.

The oracle's initial parameters come from the generator's CPU definition
(at 10^9 elements and more from the device fill, checked against the CPU
definition on a sample).  Its gradients are the device fill's, read back
after each step: at these sizes the CPU generator would take minutes per
step.  The largest vectors are read back and checked range by range.  The device fill is the
generator itself (``tests/test_gpu_synth.py`` pins it to the CPU definition
bit for bit), and each step's read-back is checked against the CPU
definition again on a random sample of every row.  The oracle runs on
contiguous chunks of the vector in a thread pool; every element's result
depends on that element's inputs alone, so chunking changes nothing.
"""
import concurrent.futures as cf
import gc
import os

import numpy as np
import pytest
import torch

import synth
import workloads as wl
import zero_sharded_mixed_reduce_amd as z
from oracle import accounting as acc
from oracle import numerics as nm
from oracle.layout import make_layout
from tests.gpu_helpers import compare, host16, say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 22
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
SAMPLE = 1 << 15             # read-back gradient positions checked per row and step


def free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _chunks(n):
    return [(lo, min(n, lo + CHUNK)) for lo in range(0, n, CHUNK)]


def theta_host(seed, p0, n, sigma=0.02):
    """theta0 at parameters [p0, p0 + n) from the generator's CPU definition."""
    out = np.empty(n, np.float32)

    def fill(span):
        lo, hi = span
        out[lo:hi] = synth.theta0(seed, np.arange(p0 + lo, p0 + hi, dtype=np.int64), sigma)
    with cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(fill, _chunks(n)))
    return out


class OracleState:
    """The oracle's master, m and v of n parameters, advanced one step at a
    time over contiguous chunks in a thread pool."""

    def __init__(self, theta, dtype, lr, betas=(0.9, 0.999), eps=1e-8):
        self.master = theta.copy()
        self.m = np.zeros_like(theta)
        self.v = np.zeros_like(theta)
        self.dtype, self.lr, self.betas, self.eps = dtype, lr, betas, eps

    def step(self, t, rows16):
        """rows16: N x n 16-bit gradient patterns (one row per rank)."""
        k = nm.adam_consts(self.lr, self.betas[0], self.betas[1], self.eps, t)

        def run(span):
            lo, hi = span
            g = nm.reduce_rank_order([nm.widen16(r[lo:hi], self.dtype) for r in rows16])
            self.master[lo:hi], self.m[lo:hi], self.v[lo:hi] = nm.adam_update(
                self.master[lo:hi], self.m[lo:hi], self.v[lo:hi], g, k)
        with cf.ThreadPoolExecutor(THREADS) as ex:
            list(ex.map(run, _chunks(self.master.size)))

    def step_range(self, t, lo, rows16):
        """One step on parameters [lo, lo + rows16.shape[1]) only."""
        k = nm.adam_consts(self.lr, self.betas[0], self.betas[1], self.eps, t)
        n = rows16.shape[1]

        def run(span):
            a, b = span
            g = nm.reduce_rank_order([nm.widen16(r[a:b], self.dtype) for r in rows16])
            sl = slice(lo + a, lo + b)
            self.master[sl], self.m[sl], self.v[sl] = nm.adam_update(
                self.master[sl], self.m[sl], self.v[sl], g, k)
        with cf.ThreadPoolExecutor(THREADS) as ex:
            list(ex.map(run, _chunks(n)))

    def cast(self):
        out = np.empty(self.master.size, np.uint16)

        def run(span):
            lo, hi = span
            out[lo:hi] = nm.cast16(self.master[lo:hi], self.dtype)
        with cf.ThreadPoolExecutor(THREADS) as ex:
            list(ex.map(run, _chunks(self.master.size)))
        return out


def rows_back(grads: torch.Tensor, rows: int, stride: int, n: int) -> np.ndarray:
    """rows x n 16-bit patterns read back from a device buffer of rows x stride."""
    h = grads.view(torch.int16)[:rows * stride].cpu().numpy().view(np.uint16)
    return h.reshape(rows, stride)[:, :n]


def check_generator_sample(rows16, seed, step, p0, sigma, dtype, outlier=0, rng_seed=0):
    """The read-back gradients equal the generator's CPU definition on a
    random sample of every row."""
    n = rows16.shape[1]
    rng = np.random.default_rng(rng_seed + step)
    k = np.unique(np.concatenate([rng.integers(0, n, SAMPLE), [0, n - 1]]))
    for r in range(rows16.shape[0]):
        want = synth.grad16(seed, r, step, p0 + k, sigma, dtype, outlier)
        assert np.array_equal(rows16[r, k], want), f"device fill differs from the generator: row {r}"


def rows_range(grads: torch.Tensor, rows: int, stride: int, lo: int, hi: int) -> np.ndarray:
    """rows x (hi - lo) 16-bit patterns, columns [lo, hi) of a device buffer
    of rows x stride."""
    v = grads.view(torch.int16)[:rows * stride].view(rows, stride)[:, lo:hi]
    return v.contiguous().cpu().numpy().view(np.uint16)


def theta_device_checked(n, p0, seed, sigma=0.02):
    """theta0 of parameters [p0, p0 + n) from the device fill, checked against
    the generator's CPU definition on a sample."""
    import synth.gpu as sgpu
    th = torch.empty(n, dtype=torch.float32, device="cuda")
    sgpu.fill32(th, n, p0, n, seed, synth.TAG_THETA, 0, 0, sigma)
    host = th.cpu().numpy()
    del th
    rng = np.random.default_rng(p0 % 1000)
    k = np.unique(np.concatenate([rng.integers(0, n, SAMPLE), [0, n - 1]]))
    assert np.array_equal(host[k].view(np.uint32), synth.theta0(seed, p0 + k, sigma).view(np.uint32))
    return host


class RangeCounts:
    """Differing-element counts accumulated over ranges of a vector, with the
    acceptance bar checked on every range."""

    def __init__(self, what):
        self.what = what
        self.counts = {"master": 0, "m": 0, "v": 0, "p16": 0}
        self.n = 0

    def add(self, got, want, got16, want16):
        diff = {k: np.flatnonzero(got[k].view(np.uint32) != want[k].view(np.uint32)) for k in want}
        d16 = np.flatnonzero(got16 != want16)
        idx = np.unique(np.concatenate([*diff.values(), d16, [0]]))
        compare({k: got[k][idx] for k in want}, {k: want[k][idx] for k in want}, got16[idx],
                want16[idx], self.what + " (differing elements of a range)")
        for k, v in diff.items():
            self.counts[k] += int(v.size)
        self.counts["p16"] += int(d16.size)
        self.n += got16.size

    def report(self):
        say(f"[full vector] {self.what}: {self.n} elements, differing " +
            ", ".join(f"{k}={v}" for k, v in self.counts.items()))
        return self.counts


def compare_all(got, want, got16, want16, what):
    """Bit-exact counts over every element, then the acceptance bar on all
    of them (elements with equal bits have zero error, so only differing
    ones need the tolerance computation)."""
    diff = {}
    for k in want:
        d = got[k].view(np.uint32) != want[k].view(np.uint32)
        diff[k] = np.flatnonzero(d)
    d16 = np.flatnonzero(got16 != want16)
    idx = np.unique(np.concatenate([*diff.values(), d16, [0]]))
    compare({k: got[k][idx] for k in want}, {k: want[k][idx] for k in want}, got16[idx],
            want16[idx], what + " (differing elements)")
    counts = {k: int(v.size) for k, v in diff.items()}
    counts["p16"] = int(d16.size)
    say(f"[full vector] {what}: {got16.size} elements, differing " +
        ", ".join(f"{k}={v}" for k, v in counts.items()))
    return counts


# --------------------------------------------------------- GPT-2 small ---
@pytest.mark.timeout(1200)
def test_gpt2s_every_element_every_step():
    w = wl.WORKLOADS["gpt2s"]
    say(f"[full vector] gpt2s: numel={w.numel} world={w.world} T={w.steps}")
    world = wl.ShardedWorld(w)
    n, P = w.numel, world.P
    assert P == n                                   # 8 divides the count: no pad
    oracle = OracleState(theta_host(w.seed, 0, n, w.theta_sigma), w.dtype, w.lr, w.betas, w.eps)
    totals = []
    for t in range(1, w.steps + 1):
        world.gen_grads(t)
        rows16 = rows_back(world.grads, w.world, P, n)
        check_generator_sample(rows16, w.seed, t, 0, w.grad_sigma, w.dtype, w.outlier_permyriad)
        world.step(t)
        oracle.step(t, rows16)
        del rows16
        torch.cuda.synchronize()
        got = {"master": world.master.cpu().numpy(), "m": world.m.cpu().numpy(),
               "v": world.v.cpu().numpy()}
        counts = compare_all(got, {"master": oracle.master, "m": oracle.m, "v": oracle.v},
                             host16(world.wc), oracle.cast(), f"gpt2s step {t}")
        totals.append(counts)
        del got
    lay = make_layout(w.numel, w.world, w.stage)
    want = acc.bytes_per_rank(lay)
    for r in range(w.world):
        c = z.zero_counters(world.ctx, r)
        assert (c["rs_elems"], c["ag_elems"]) == (w.steps * want.rs_elems, w.steps * want.ag_elems)
    say(f"[full vector] gpt2s: differing elements over all steps: "
        f"{sum(sum(c.values()) for c in totals)}")
    del world, oracle
    free()


# ------------------------------------------------ bucketed share step ---
SHARE_S = 2_000_003


def _share_workload():
    return wl.Workload("share64small", "one_rank_share_small_n64_zero2_bf16", 64 * SHARE_S, 64, 2,
                       "bf16", 1e-3, 1e-4, 2)


def _check_share(share, oracle, rows16_by_step, what):
    """master, m, v and the own slot against the oracle; every peer slot
    against the staged values (the receive is a copy), which are checked
    against the generator's CPU definition on a sample."""
    S, off, P = share.S, share.off, share.P
    got = {"master": share.master.cpu().numpy(), "m": share.m.cpu().numpy(),
           "v": share.v.cpu().numpy()}
    wc = host16(share.wc)
    compare_all(got, {"master": oracle.master, "m": oracle.m, "v": oracle.v}, wc[off:off + S],
                oracle.cast(), what)
    staged = host16(share.staged)
    rng = np.random.default_rng(1)
    k = rng.integers(0, P, SAMPLE)
    assert np.array_equal(staged[k], synth.peer16(share.w.seed, k, share.w.dtype, share.w.theta_sigma))
    assert np.array_equal(wc[:off], staged[:off]) and np.array_equal(wc[off + S:], staged[off + S:])


@pytest.mark.parametrize("n_buckets", [1, 3, 16])
def test_bucketed_share_step_against_oracle(n_buckets):
    """Gradients that arrive bucket by bucket (last parameters first, filled
    on a second stream), each bucket updated and its peers' pieces received
    at once: every element against the oracle after every step."""
    w = _share_workload()
    rank = 5
    say(f"[full vector] bucketed share: S={SHARE_S} buckets={n_buckets}")
    share = wl.RankShare(w, rank=rank)
    plan = z.zsmr_fused_step_plan(share.ctx, rank, 0, share.grads, share.row_stride, 0, share.master,
                                  share.m, share.v, share.wc[share.off:])
    assert plan["kernel"] == "deferred", plan      # 64 rows: the production kernel
    oracle = OracleState(theta_host(w.seed, share.off, share.S), w.dtype, w.lr, w.betas, w.eps)
    side = torch.cuda.Stream()
    for t in range(1, w.steps + 1):
        share.step_bucketed(t, n_buckets, side)
        torch.cuda.synchronize()
        rows16 = rows_back(share.grads, w.world, share.row_stride, share.S)
        check_generator_sample(rows16, w.seed, t, share.off, w.grad_sigma, w.dtype)
        oracle.step(t, rows16)
        _check_share(share, oracle, None, f"bucketed x{n_buckets} step {t}")
    lay = make_layout(w.numel, w.world, w.stage)
    want = acc.bytes_per_rank(lay)
    c = z.zero_counters(share.ctx, rank)
    assert (c["rs_elems"], c["ag_elems"]) == (w.steps * want.rs_elems, w.steps * want.ag_elems)
    del share, oracle
    free()


def test_ragged_fused_ranges_against_oracle():
    """Sub-ranges of the shard cut at ragged, unaligned places (the vector and
    the one-element paths both run), each followed by the receive of the
    peers' pieces of the same range: every element against the oracle."""
    w = _share_workload()
    rank = 63
    share = wl.RankShare(w, rank=rank)
    S = share.S
    edges = [0, 1, 513, 777, 4096, 150_001, 1_000_003, S - 3, S]
    oracle = OracleState(theta_host(w.seed, share.off, S), w.dtype, w.lr, w.betas, w.eps)
    for t in range(1, w.steps + 1):
        share.gen_grads(t)
        for b0, b1 in zip(edges[:-1], edges[1:]):
            z.zero_fused_step_range(share.ctx, rank, 0, b0, b1 - b0, share.grads, share.row_stride, 0,
                                    share.master, share.m, share.v, share.wc[share.off:], t, w.lr,
                                    w.betas, w.eps)
            share.receive_range(b0, b1)
        torch.cuda.synchronize()
        rows16 = rows_back(share.grads, w.world, share.row_stride, S)
        check_generator_sample(rows16, w.seed, t, share.off, w.grad_sigma, w.dtype)
        oracle.step(t, rows16)
        _check_share(share, oracle, None, f"ragged ranges step {t}")
    del share, oracle
    free()


# --------------------------------------------- ZeRO-3 split, prefetched ---
@pytest.mark.parametrize("prefetch", [False, True])
def test_stage3_split_layout_against_oracle(prefetch):
    """ZeRO-3 with each unit split N ways (four units of unequal size, 8
    ranks), with and without the next unit gathered on a second stream:
    every element against the oracle after the run, counters and peak
    against the accounting."""
    units = (3 << 20, 1 << 20, 5 << 19, 1 << 20)
    w = wl.Workload("s3small", "stage3_small_4_units_n8_bf16", sum(units), 8, 3, "bf16", 1e-3, 1e-4,
                    2, units=units)
    say(f"[full vector] stage 3 split prefetch={prefetch}")
    s3 = wl.Stage3World(w, check_gathers=True, prefetch=prefetch)
    n = w.numel
    lay = make_layout(n, w.world, 3, list(units))
    assert lay.padded_numel == n                    # every unit divides by 8: padded order = natural
    oracle = OracleState(theta_host(w.seed, 0, n), w.dtype, w.lr, w.betas, w.eps)
    g = torch.empty(w.world * n, dtype=torch.int16, device="cuda")
    import synth.gpu as sgpu
    for t in range(1, w.steps + 1):
        s3.step(t)
        # the same gradients the run drew unit by unit, drawn for the whole vector
        sgpu.fill16(g, w.world, n, n, 0, n, w.seed, synth.TAG_GRAD, 0, t, w.grad_sigma, w.dtype)
        torch.cuda.synchronize()
        rows16 = rows_back(g, w.world, n, n)
        check_generator_sample(rows16, w.seed, t, 0, w.grad_sigma, w.dtype)
        oracle.step(t, rows16)
    assert s3.gather_mismatch == 0
    got = {"master": s3.master.cpu().numpy(), "m": s3.m.cpu().numpy(), "v": s3.v.cpu().numpy()}
    compare_all(got, {"master": oracle.master, "m": oracle.m, "v": oracle.v}, host16(s3.p16),
                oracle.cast(), f"stage 3 split prefetch={prefetch}")
    ml = 2 if prefetch else 1
    want = acc.bytes_per_rank(lay, max_live=ml)
    for r in range(w.world):
        c = z.zero_counters(s3.ctx, r)
        assert (c["rs_elems"], c["ag_elems"]) == (w.steps * want.rs_elems, w.steps * want.ag_elems)
        assert c["peak_live_bytes"] == want.gathered
    c = z.zero_counters(s3.ctx, 0)
    assert c["stage3_gathers"] == 2 * lay.n_units * w.steps == c["stage3_releases"]
    del s3, g, oracle
    free()


# ------------------------------------------------------------ GPT-2 1.5B ---
RANGE = 1 << 27                 # parameters read back and checked at once


@pytest.mark.timeout(1800)
def test_gpt2xl_every_element_every_step():
    """GPT-2 1.5B: 1,558,000,000 parameters, 16 ranks, ZeRO-1, bf16 with one
    entry in a hundred scaled by 100, 3 steps: every element after every
    step, range by range."""
    w = wl.WORKLOADS["gpt2xl"]
    say(f"[full vector] gpt2xl: numel={w.numel} world={w.world} T={w.steps}")
    world = wl.ShardedWorld(w)
    n, P = w.numel, world.P
    assert P == n
    oracle = OracleState(theta_device_checked(n, 0, w.seed, w.theta_sigma), w.dtype, w.lr, w.betas,
                         w.eps)
    total = 0
    for t in range(1, w.steps + 1):
        world.gen_grads(t)
        for lo in range(0, n, RANGE):
            hi = min(n, lo + RANGE)
            rows16 = rows_range(world.grads, w.world, P, lo, hi)
            if lo == 0:
                check_generator_sample(rows16, w.seed, t, 0, w.grad_sigma, w.dtype,
                                       w.outlier_permyriad)
            oracle.step_range(t, lo, rows16)
            del rows16
        say(f"[full vector] gpt2xl step {t}: oracle stepped")
        world.step(t)
        torch.cuda.synchronize()
        rc = RangeCounts(f"gpt2xl step {t}")
        for lo in range(0, n, RANGE):
            hi = min(n, lo + RANGE)
            got = {"master": world.master[lo:hi].cpu().numpy(), "m": world.m[lo:hi].cpu().numpy(),
                   "v": world.v[lo:hi].cpu().numpy()}
            want = {"master": oracle.master[lo:hi], "m": oracle.m[lo:hi], "v": oracle.v[lo:hi]}
            rc.add(got, want, host16(world.wc[lo:hi]), nm.cast16(oracle.master[lo:hi], w.dtype))
        total += sum(rc.report().values())
    say(f"[full vector] gpt2xl: differing elements over all steps: {total}")
    del world, oracle
    free()


# ------------------------------------------ one rank's share, 64 ranks ---
@pytest.mark.timeout(1800)
@pytest.mark.parametrize("rank", [0, 63])
def test_share64_every_owned_element_every_step(rank):
    """One rank of the 7.5e9-parameter, 64-rank world: every one of its
    117,187,500 owned elements after each of the 3 steps (64 bf16
    contributions each); the 63 peer slots equal the staged values."""
    w = wl.WORKLOADS["share64"]
    say(f"[full vector] share64 rank={rank}")
    share = wl.RankShare(w, rank=rank)
    S, off = share.S, share.off
    oracle = OracleState(theta_host(w.seed, off, S), w.dtype, w.lr, w.betas, w.eps)
    total = 0
    for t in range(1, w.steps + 1):
        share.gen_grads(t)
        for lo in range(0, S, RANGE // 4):
            hi = min(S, lo + RANGE // 4)
            rows16 = rows_range(share.grads, w.world, share.row_stride, lo, hi)
            if lo == 0:
                check_generator_sample(rows16, w.seed, t, off, w.grad_sigma, w.dtype)
            oracle.step_range(t, lo, rows16)
            del rows16
        say(f"[full vector] share64 rank {rank} step {t}: oracle stepped")
        share.step(t)
        torch.cuda.synchronize()
        rc = RangeCounts(f"share64 rank {rank} step {t}")
        got = {"master": share.master.cpu().numpy(), "m": share.m.cpu().numpy(), "v": share.v.cpu().numpy()}
        rc.add(got, {"master": oracle.master, "m": oracle.m, "v": oracle.v},
               host16(share.wc[off:off + S]), oracle.cast())
        total += sum(rc.report().values())
    for lo, hi in ((0, off), (off + S, share.P)):
        for c in range(lo, hi, 1 << 28):
            e = min(hi, c + (1 << 28))
            assert torch.equal(share.wc[c:e].view(torch.int16), share.staged[c:e].view(torch.int16))
    say(f"[full vector] share64 rank {rank}: differing elements over all steps: {total}")
    del share, oracle
    free()


# --------------------------------------------------- Llama-3-8B shape ---
@pytest.mark.timeout(1800)
@pytest.mark.parametrize("part", [0, 1, 2])
def test_llama8b_every_element_after_the_run(part):
    """The Llama-3-8B shape (33 units, 8 ranks, ZeRO-3 per-unit split, 2
    steps): after the run, every element of the units u with u % 3 == part
    against the oracle, unit by unit (each unit's trajectory depends on its
    own inputs alone; the three parts together cover all 33 units)."""
    import synth.gpu as sgpu
    w = wl.WORKLOADS["llama8b"]
    say(f"[full vector] llama8b: units={len(w.units)} numel={w.numel} part={part}")
    s3 = wl.Stage3World(w, check_gathers=True)
    s3.run(w.steps)
    torch.cuda.synchronize()
    assert s3.gather_mismatch == 0
    rc = RangeCounts(f"llama8b after 2 steps, units {part}, {part + 3}, ...")
    for u in range(part, s3.U, 3):
        p0, size, width, q0 = s3.P_start[u], s3.P_size[u], s3.width[u], s3.Q_u[u]
        assert width == size                        # every unit divides by 8: no pad
        oracle = OracleState(theta_device_checked(size, p0, w.seed, w.theta_sigma), w.dtype, w.lr,
                             w.betas, w.eps)
        for t in range(1, w.steps + 1):
            # the unit's gradients of step t, drawn again exactly as the run drew them
            sgpu.fill16(s3.grads, w.world, width, width, p0, size, w.seed, synth.TAG_GRAD, 0, t,
                        w.grad_sigma, w.dtype, w.outlier_permyriad)
            torch.cuda.synchronize()
            for lo in range(0, size, RANGE):
                hi = min(size, lo + RANGE)
                rows16 = rows_range(s3.grads, w.world, width, lo, hi)
                if lo == 0 and u in (0, 1, 2, s3.U - 1):
                    check_generator_sample(rows16, w.seed, t, p0, w.grad_sigma, w.dtype)
                oracle.step_range(t, lo, rows16)
                del rows16
        for lo in range(0, size, RANGE):
            hi = min(size, lo + RANGE)
            a, b = q0 + lo, q0 + hi
            got = {"master": s3.master[a:b].cpu().numpy(), "m": s3.m[a:b].cpu().numpy(),
                   "v": s3.v[a:b].cpu().numpy()}
            want = {"master": oracle.master[lo:hi], "m": oracle.m[lo:hi], "v": oracle.v[lo:hi]}
            rc.add(got, want, host16(s3.p16[a:b]), nm.cast16(oracle.master[lo:hi], w.dtype))
        del oracle
    rc.report()
    del s3
    free()
