"""The five synthetic workloads of the ZeRO shard step and their GPU drivers.

Used by ``bench.py`` and the GPU tests.  Device memory comes from torch; the
inputs are filled by the seeded GPU generator (``synth.gpu``, outside any
timed region); every step of the method runs through the C ABI of
``libzsmr.so`` (``zero_sharded_mixed_reduce_amd``).  Nothing here computes
part of the method itself.

Workloads (theta0 ~ N(0, 0.02) fp32, betas (0.9, 0.999), eps 1e-8, seed 0):
  psi65k    Psi = 65,536, N = 4, fp16 grads ~ N(0, 1e-2), lr 1e-2, T = 5, all
            four schemes; ZeRO-3 in 4 units of 16,384.
  gpt2s     Psi = 124,439,808 (GPT-2 small), N = 8, ZeRO-2, bf16 ~ N(0, 1e-3),
            lr 1e-4, T = 10.
  gpt2xl    Psi = 1,558,000,000 (GPT-2 1.5B), N = 16, ZeRO-1, bf16 ~ N(0, 1e-3)
            with one entry in a hundred scaled by 100, lr 1e-4, T = 3.
  share64   one rank's share of Psi = 7.5e9 on N = 64 (the ZeRO paper's
            Figure-1 model): owned shard S = 117,187,500, 64 bf16 gradient
            contributions for it ~ N(0, 1e-3), the whole 7.5e9-element bf16
            working copy written (own slot by the cast, 63 peer slots received
            from a staged buffer), ZeRO-2, lr 1e-4, T = 3.
  llama8b   Llama-3-8B-shaped vector, 33 units (embeddings + head + final norm
            1,050,677,248; 32 layers of 218,112,000), N = 8, ZeRO-3 per-unit
            bf16 gather -> release -> re-gather, bf16 grads ~ N(0, 1e-3),
            lr 1e-4, T = 2.
"""
from __future__ import annotations

import time
from dataclasses import dataclass, field
from typing import List, Optional

import torch

import synth
import synth.gpu as sgpu
import zero_sharded_mixed_reduce_amd as z

TORCH16 = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    key: str
    name: str
    numel: int
    world: int
    stage: int
    dtype: str
    grad_sigma: float
    lr: float
    steps: int
    units: Optional[tuple] = None
    outlier_permyriad: int = 0
    pad: bool = False
    seed: int = 0
    theta_sigma: float = 0.02
    betas: tuple = (0.9, 0.999)
    eps: float = 1e-8


LLAMA8B_UNITS = (1_050_677_248,) + (218_112_000,) * 32
# Owner broadcast on the Llama-3-8B shape: the pages fix owners only for equal
# partitions, so the owners are chosen here: embeddings + head + final norm
# alone on rank 0, the 32 layers in contiguous runs of 5, 5, 5, 5, 4, 4, 4 on
# ranks 1-7 (0.87e9-1.09e9 parameters per rank).
LLAMA8B_OWNERS = (0,) + (1,) * 5 + (2,) * 5 + (3,) * 5 + (4,) * 5 + (5,) * 4 + (6,) * 4 + (7,) * 4

WORKLOADS = {
    "psi65k": Workload("psi65k", "psi65536_n4_fp16_all_schemes", 65536, 4, 2, "fp16", 1e-2, 1e-2, 5,
                       units=(16384,) * 4),
    "gpt2s": Workload("gpt2s", "gpt2_small_psi124439808_n8_zero2_bf16", 124_439_808, 8, 2, "bf16",
                      1e-3, 1e-4, 10),
    "gpt2xl": Workload("gpt2xl", "gpt2_1.5b_psi1558000000_n16_zero1_bf16_outliers", 1_558_000_000,
                       16, 1, "bf16", 1e-3, 1e-4, 3, outlier_permyriad=100),
    "share64": Workload("share64", "one_rank_share_psi7.5e9_n64_zero2_bf16", 7_500_000_000, 64, 2,
                        "bf16", 1e-3, 1e-4, 3),
    "llama8b": Workload("llama8b", "llama3_8b_shape_33_units_n8_zero3_bf16", sum(LLAMA8B_UNITS), 8,
                        3, "bf16", 1e-3, 1e-4, 2, units=LLAMA8B_UNITS),
}


def empty16(n: int, dtype: str, device="cuda") -> torch.Tensor:
    return torch.empty(n, dtype=TORCH16[dtype], device=device)


def aligned_view(n: int, dtype: str, like_ptr: int, device="cuda") -> torch.Tensor:
    """16-bit buffer of n elements whose address equals ``like_ptr`` modulo 16."""
    raw = torch.empty(n + 8, dtype=TORCH16[dtype], device=device)
    shift = ((like_ptr - raw.data_ptr()) % 16) // 2
    return raw[shift:shift + n]


class Timer:
    """Sums HIP event intervals recorded on one stream (only the method's
    kernels sit inside an interval; input generation sits outside)."""

    def __init__(self, stream):
        self.stream = stream
        self.pairs = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append([e, None])

    def stop(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs[-1][1] = e

    def ms(self) -> float:
        self.stream.synchronize()
        return sum(a.elapsed_time(b) for a, b in self.pairs)

    def reset(self):
        self.pairs = []


# --------------------------------------------------------- stages 1 and 2 --
class ShardedWorld:
    """Stages 1-2 with all N ranks simulated: N full gradient rows, the fp32
    master/m/v of every rank (rank r's shard at r*S of one padded buffer) and
    one canonical 16-bit working copy (slot r at r*S)."""

    def __init__(self, w: Workload, device="cuda"):
        self.w = w
        self.ctx = z.zero_init_shards(w.numel, w.world, w.stage, w.dtype, pad=w.pad)
        info = self.ctx.info()
        self.P, self.S = info["padded_numel"], info["shard_numel"]
        P = self.P
        self.master = torch.empty(P, dtype=torch.float32, device=device)
        self.m = torch.empty_like(self.master)
        self.v = torch.empty_like(self.master)
        self.wc = empty16(P, w.dtype, device)
        self.grads = empty16(w.world * P, w.dtype, device)
        self.stream = torch.cuda.current_stream()
        theta = torch.empty(P, dtype=torch.float32, device=device)
        sgpu.fill32(theta, P, 0, w.numel, w.seed, synth.TAG_THETA, 0, 0, w.theta_sigma)
        for r in range(w.world):
            off, n, _ = z.zero_layout(self.ctx, r, 0)
            z.zero_init_state(self.ctx, r, 0, theta[off:], self.master[off:], self.m[off:],
                              self.v[off:], self.wc[off:])
        del theta
        self.t = 0

    def gen_grads(self, step: int):
        w = self.w
        sgpu.fill16(self.grads, w.world, self.P, self.P, 0, w.numel, w.seed, synth.TAG_GRAD, 0,
                    step, w.grad_sigma, w.dtype, w.outlier_permyriad)

    def step(self, t: int, timer: Optional[Timer] = None, fused: bool = True, g_tmp=None):
        w = self.w
        if timer:
            timer.start()
        for r in range(w.world):
            off = r * self.S
            if fused:
                z.zero_fused_step(self.ctx, r, 0, self.grads, self.P, off, self.master[off:],
                                  self.m[off:], self.v[off:], self.wc[off:], t, w.lr, w.betas, w.eps)
            else:
                z.zero_reduce_shard(self.ctx, r, 0, self.grads, self.P, off, True, g_tmp)
                z.zero_adam_step(self.master[off:], self.m[off:], self.v[off:], g_tmp, self.S, t,
                                 w.lr, w.betas, w.eps)
                z.zero_gather_cast(self.ctx, r, 0, self.master[off:], self.wc[off:])
        if timer:
            timer.stop()

    def run(self, steps: int, timer: Optional[Timer] = None, fused: bool = True):
        g_tmp = None if fused else torch.empty(self.S, dtype=torch.float32, device=self.master.device)
        for t in range(1, steps + 1):
            self.gen_grads(t)
            self.step(t, timer, fused, g_tmp)
        self.t = steps


# ------------------------------------------------ one rank's share (N=64) --
class RankShare:
    """One rank s of a large world: its S-element fp32 shard, the N gradient
    contributions to it (row stride S rounded up to 64 elements, so that every
    row starts on a 128-byte line: with S = 117,187,500 a stride rounded only
    to 16 bytes leaves every other row 32 bytes into a 64-byte HBM granule,
    and the reads then fetch about 6% more than they use), and the full
    16-bit working copy of N*S elements, whose peer slots are received from a
    staged buffer laid out like the working copy."""

    def __init__(self, w: Workload, rank: int = 0, device="cuda"):
        self.w, self.rank = w, rank
        self.ctx = z.zero_init_shards(w.numel, w.world, w.stage, w.dtype, pad=w.pad)
        off, S, _ = z.zero_layout(self.ctx, rank, 0)
        self.off, self.S = off, S
        self.row_stride = (S + 63) // 64 * 64
        self.P = S * w.world
        self.master = torch.empty(S, dtype=torch.float32, device=device)
        self.m = torch.empty_like(self.master)
        self.v = torch.empty_like(self.master)
        self.grads = empty16(w.world * self.row_stride, w.dtype, device)
        self.wc = empty16(self.P, w.dtype, device)
        self.staged = aligned_view(self.P, w.dtype, self.wc.data_ptr(), device)
        theta = torch.empty(S, dtype=torch.float32, device=device)
        sgpu.fill32(theta, S, off, S, w.seed, synth.TAG_THETA, 0, 0, w.theta_sigma)
        z.zero_init_state(self.ctx, rank, 0, theta, self.master, self.m, self.v, self.wc[off:])
        del theta
        # what the other ranks' all-gather delivers (the own slot is never read)
        sgpu.fill16(self.staged, 1, self.P, self.P, 0, self.P, w.seed, synth.TAG_PEER, 0, 0,
                    w.theta_sigma, w.dtype)
        self.wc[:off].zero_()
        self.wc[off + S:].zero_()

    def gen_grads(self, step: int):
        w = self.w
        sgpu.fill16(self.grads, w.world, self.row_stride, self.row_stride, self.off, self.S, w.seed,
                    synth.TAG_GRAD, 0, step, w.grad_sigma, w.dtype, w.outlier_permyriad)

    def fused(self, t: int):
        w = self.w
        z.zero_fused_step(self.ctx, self.rank, 0, self.grads, self.row_stride, 0, self.master,
                          self.m, self.v, self.wc[self.off:], t, w.lr, w.betas, w.eps)

    def receive(self):
        off, S = self.off, self.S
        if off:
            z.zero_gather_copy(self.ctx, self.rank, self.staged, self.wc, off)
        rest = self.P - off - S
        if rest:
            z.zero_gather_copy(self.ctx, self.rank, self.staged[off + S:], self.wc[off + S:], rest)

    def receive_range(self, b0: int, b1: int):
        """The receive of bucket [b0, b1) alone: every peer q's piece of it
        sits at q*S + b0 of the working copy (and of the staged buffer), so
        the peers below and above this rank are two runs of blocks."""
        r, S, N, n = self.rank, self.S, self.w.world, b1 - b0
        if r > 0:
            z.zero_gather_copy_blocks(self.ctx, r, self.staged[b0:], self.wc[b0:], n, r, S)
        if r + 1 < N:
            o = (r + 1) * S + b0
            z.zero_gather_copy_blocks(self.ctx, r, self.staged[o:], self.wc[o:], n, N - r - 1, S)

    def step(self, t: int, timer: Optional[Timer] = None):
        if timer:
            timer.start()
        self.fused(t)
        self.receive()
        if timer:
            timer.stop()

    def run(self, steps: int, timer: Optional[Timer] = None):
        for t in range(1, steps + 1):
            self.gen_grads(t)
            self.step(t, timer)

    def bucket_bounds(self, n_buckets: int):
        """[begin, end) of each bucket of the owned shard, in the order a
        backward pass produces them (last parameters first); boundaries are
        multiples of 512 elements (one wave tile)."""
        size = -(-self.S // n_buckets + 511) // 512 * 512
        edges = list(range(0, self.S, size)) + [self.S]
        return [(edges[i], edges[i + 1]) for i in reversed(range(len(edges) - 1))]

    def step_bucketed(self, t: int, n_buckets: int, backward_stream, generate: bool = True):
        """One step whose gradients arrive in buckets: the simulated backward
        (the input generator, on ``backward_stream``) fills one bucket of all
        N rows at a time, and the fused step consumes each bucket on the
        current stream as soon as it is ready, followed by the receive of the
        peers' pieces of the same bucket, overlapping both with the
        backward."""
        w = self.w
        compute = torch.cuda.current_stream()
        start = torch.cuda.Event()
        start.record(compute)
        backward_stream.wait_event(start)
        for b0, b1 in self.bucket_bounds(n_buckets):
            if generate:
                with torch.cuda.stream(backward_stream):
                    sgpu.fill16(self.grads[b0:], w.world, self.row_stride, b1 - b0, self.off + b0,
                                b1 - b0, w.seed, synth.TAG_GRAD, 0, t, w.grad_sigma, w.dtype,
                                w.outlier_permyriad, stream=backward_stream)
            ready = torch.cuda.Event()
            ready.record(backward_stream)
            compute.wait_event(ready)
            z.zero_fused_step_range(self.ctx, self.rank, 0, b0, b1 - b0, self.grads, self.row_stride,
                                    0, self.master, self.m, self.v, self.wc[self.off:], t, w.lr,
                                    w.betas, w.eps)
            self.receive_range(b0, b1)


# ---------------------------------------------------------------- stage 3 --
class Stage3World:
    """ZeRO-3 with all N ranks simulated.  fp32 master/m/v and the 16-bit
    shards are kept in the padded order (unit-major, rank-minor), so shard
    (r, u) sits at Q_u + r*S_u; one unit buffer holds the gathered unit; the
    gradients of one unit (N rows of N*S_u) are generated when the backward
    pass reaches it.

    owner=True: the owner-broadcast layout instead (whole units owned by
    single ranks, natural order, no pad): unit u sits at its start Q_u, its
    owner alone initialises and updates it, a gather copies the owner's
    16-bit copy into the unit buffer, and a unit's gradients are N rows of
    P_u.  ``owners`` gives each unit's owner (None: the library's default)."""

    def __init__(self, w: Workload, device="cuda", check_gathers: bool = False,
                 prefetch: bool = False, fixed_grads: bool = False, owner: bool = False,
                 owners=None):
        """prefetch: gather the next unit on a second stream while the current
        one is in use (two unit buffers, at most two units live).
        fixed_grads: generate each unit size's gradients once and reuse them
        in every step (timing runs; the values then differ from the per-step
        recipe, so parity runs leave it off)."""
        self.w = w
        self.prefetch = prefetch
        self.fixed_grads = fixed_grads
        self.owner = owner
        stage = z.ZSMR_ZERO3_OWNER if owner else 3
        self.ctx = z.zero_init_shards(w.numel, w.world, stage, w.dtype, pad=w.pad,
                                      units=list(w.units) if w.units else None)
        if owner and owners is not None:
            z.zero_set_unit_owners(self.ctx, list(owners))
        if prefetch:
            z.zero_stage3_set_max_live(self.ctx, 2)
        info = self.ctx.info()
        self.P = info["padded_numel"]
        self.U = info["n_units"]
        self.maxw = info["max_unit_numel"]
        self.P_size = list(w.units or (w.numel,))
        starts, acc = [], 0
        for n in self.P_size:
            starts.append(acc)
            acc += n
        self.P_start = starts
        if owner:
            self.owner_of = [z.zero_unit_owner(self.ctx, u) for u in range(self.U)]
            self.Q_u = list(starts)
            self.width = list(self.P_size)              # a unit's gradient row
        else:
            self.S_u = [z.zero_layout(self.ctx, 0, u)[1] for u in range(self.U)]
            self.Q_u = [z.zero_layout(self.ctx, 0, u)[0] for u in range(self.U)]
            self.width = [w.world * s for s in self.S_u]
        self.master = torch.empty(self.P, dtype=torch.float32, device=device)
        self.m = torch.empty_like(self.master)
        self.v = torch.empty_like(self.master)
        self.p16 = empty16(self.P, w.dtype, device)
        self.unit_bufs = [empty16(self.maxw, w.dtype, device) for _ in range(2 if prefetch else 1)]
        self.unit_buf = self.unit_bufs[0]
        self.check_gathers = check_gathers
        self.gather_mismatch = 0
        self.gather_stream = torch.cuda.Stream() if prefetch else None
        if fixed_grads:
            # one gradient set per distinct unit width, made once (step 1)
            self.grads_by_width = {}
            for u in range(self.U):
                width = self.width[u]
                if width not in self.grads_by_width:
                    g = empty16(w.world * width, w.dtype, device)
                    sgpu.fill16(g, w.world, width, width, self.P_start[u], self.P_size[u], w.seed,
                                synth.TAG_GRAD, 0, 1, w.grad_sigma, w.dtype, w.outlier_permyriad)
                    self.grads_by_width[width] = g
        else:
            self.grads = empty16(w.world * self.maxw, w.dtype, device)
        theta = torch.empty(self.maxw, dtype=torch.float32, device=device)
        for u in range(self.U):
            sgpu.fill32(theta, self.width[u], self.P_start[u], self.P_size[u], w.seed, synth.TAG_THETA,
                        0, 0, w.theta_sigma)
            for r, o, n in self._pieces(u):
                z.zero_init_state(self.ctx, r, u, theta[o - self.Q_u[u]:], self.master[o:],
                                  self.m[o:], self.v[o:], self.p16[o:])
        del theta

    def _pieces(self, u: int):
        """(rank, padded offset, length) of every non-empty piece of unit u."""
        if self.owner:
            return [(self.owner_of[u], self.Q_u[u], self.P_size[u])]
        return [(r, self.Q_u[u] + r * self.S_u[u], self.S_u[u]) for r in range(self.w.world)]

    def _gather(self, u: int, buf=None):
        buf = self.unit_buf if buf is None else buf
        if self.owner:
            shards = [self.p16[self.Q_u[u]:]]
        else:
            shards = [self.p16[self.Q_u[u] + r * self.S_u[u]:] for r in range(self.w.world)]
        z.zero_stage3_unit_gather(self.ctx, u, shards, buf)
        if self.check_gathers:
            width = self.width[u]
            same = torch.equal(buf[:width].view(torch.int16),
                               self.p16[self.Q_u[u]:self.Q_u[u] + width].view(torch.int16))
            self.gather_mismatch += 0 if same else 1

    def gen_grads(self, u: int, step: int):
        w = self.w
        width = self.width[u]
        sgpu.fill16(self.grads, w.world, width, width, self.P_start[u], self.P_size[u], w.seed,
                    synth.TAG_GRAD, 0, step, w.grad_sigma, w.dtype, w.outlier_permyriad)

    def _grads_for(self, u: int, t: int):
        if self.fixed_grads:
            return self.grads_by_width[self.width[u]]
        self.gen_grads(u, t)                          # the unit's gradients appear
        return self.grads

    def _update(self, u: int, t: int, grads):
        w = self.w
        for r, o, n in self._pieces(u):
            z.zero_fused_step(self.ctx, r, u, grads, self.width[u], o - self.Q_u[u], self.master[o:],
                              self.m[o:], self.v[o:], self.p16[o:], t, w.lr, w.betas, w.eps)

    def step(self, t: int, timer: Optional[Timer] = None):
        if self.prefetch:
            return self._step_prefetch(t)
        timed = timer is not None and not self.fixed_grads
        if timer and self.fixed_grads:
            timer.start()
        for u in range(self.U):                        # forward: gather -> use -> release
            if timed:
                timer.start()
            self._gather(u)
            z.zero_stage3_unit_release(self.ctx, u)
            if timed:
                timer.stop()
        for u in reversed(range(self.U)):              # backward: re-gather -> reduce+Adam+cast
            if timed:
                timer.start()
            self._gather(u)
            if timed:
                timer.stop()
            grads = self._grads_for(u, t)              # untimed when generated here
            if timed:
                timer.start()
            self._update(u, t, grads)
            z.zero_stage3_unit_release(self.ctx, u)
            if timed:
                timer.stop()
        if timer and self.fixed_grads:
            timer.stop()

    def _step_prefetch(self, t: int):
        """Forward and backward with the next unit gathered on the gather
        stream while the current one is in use; a unit buffer is refilled
        only after the unit it held was released and its consumers ran."""
        compute, gs = torch.cuda.current_stream(), self.gather_stream
        order = list(range(self.U)) + list(reversed(range(self.U)))
        done = [torch.cuda.Event() for _ in range(2)]     # buffer free again
        for d in done:
            d.record(compute)
        gathered = [None] * len(order)

        def issue(k):
            u, slot = order[k], k % 2
            gs.wait_event(done[slot])
            with torch.cuda.stream(gs):
                self._gather(u, self.unit_bufs[slot])
            ev = torch.cuda.Event()
            ev.record(gs)
            gathered[k] = ev

        issue(0)
        for k, u in enumerate(order):
            more = k + 1 < len(order)
            # prefetch: two units live -- except at the turn from forward to
            # backward, where the next unit is this one, gathered again once
            # it has been released
            early = more and order[k + 1] != u
            if early:
                issue(k + 1)
            compute.wait_event(gathered[k])
            if k >= self.U:                            # backward half: update the unit
                self._update(u, t, self._grads_for(u, t))
            z.zero_stage3_unit_release(self.ctx, u)
            done[k % 2].record(compute)
            if more and not early:
                issue(k + 1)
        compute.wait_stream(gs)

    def run(self, steps: int, timer: Optional[Timer] = None):
        for t in range(1, steps + 1):
            self.step(t, timer)
