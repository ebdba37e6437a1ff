"""The four schemes (plain data parallelism, ZeRO-1, ZeRO-2, ZeRO-3) run for
N ranks simulated on the CPU.

Test infrastructure only (see the package header).

Each scheme keeps per-rank lists of bands, as the pages' prototype does ("The
four schemes", ``Base`` and its subclasses), and differs from the others only
in what it shards and which collectives it runs (the three-flag table of the
same page).  Gradients are inputs: one 16-bit vector of Psi elements per rank
per step, in place of the prototype's model (whose code is not on the pages).
Collectives are simulated in-process, and every rank's received elements are
counted so that the totals can be checked against ``accounting``.

Readings where the pages leave a step open:
* The reduce is a mean, summed in fp32 in rank order (``numerics``).
* The all-gather moves the 16-bit cast of each owned shard.  The prototype
  gathers fp32 masters and casts afterwards; the cast is elementwise, so the
  working copy is bit-identical either way (pinned by a test).
* ZeRO-3 cuts the vector into units, each split N ways ("ZeRO and FSDP",
  "ZeRO-3 and FSDP"); a unit is gathered for the forward pass, released,
  gathered again for the backward pass, and after its gradients are reduced
  and its shards updated it is released ("The four schemes", where the third
  P comes from and the mistake to avoid).  Adam runs per unit as its
  gradients arrive; elementwise, this equals running it after the whole
  backward pass.
* ``t`` advances once per step, not per unit.
* Owner broadcast (``ZeRO3Owner``; "One Poem Suffices: ZeRO" section 4.1.4,
  "ZeRO, annotated" section 7): whole units belong to one rank each.  A
  unit's owner sends its 16-bit copy to the others for the forward pass and
  again for the backward pass; its gradients are summed onto the owner (the
  same rank-order fp32 mean), which alone updates the unit.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence

import numpy as np

from . import numerics as nm
from .layout import Layout, make_layout


class ScheduleError(RuntimeError):
    """A ZeRO-3 gather/release issued in an order the schedule forbids."""


class Stage3Schedule:
    """Gather/release state machine of ZeRO-3 with exact counters.

    ``max_live`` units may be gathered at once (1 = no prefetch).  Gathering a
    live unit, releasing a unit that is not live, or exceeding ``max_live``
    raises ``ScheduleError``.
    """

    def __init__(self, lay: Layout, gather_bytes: int = 2, max_live: int = 1):
        self.lay = lay
        self.gather_bytes = gather_bytes
        self.max_live = max_live
        self.live: List[int] = []
        self.gathers = [0] * lay.n_units
        self.releases = [0] * lay.n_units
        self.ag_elems = 0            # received per rank
        self.live_bytes = 0
        self.peak_live_bytes = 0

    def gather(self, unit: int) -> None:
        if unit in self.live:
            raise ScheduleError(f"unit {unit} is already gathered")
        if len(self.live) >= self.max_live:
            raise ScheduleError(f"{len(self.live)} unit(s) live, limit {self.max_live}")
        s = self.lay.shard_u[unit]
        self.live.append(unit)
        self.gathers[unit] += 1
        self.ag_elems += (self.lay.world - 1) * s
        self.live_bytes += self.gather_bytes * self.lay.world * s
        self.peak_live_bytes = max(self.peak_live_bytes, self.live_bytes)

    def release(self, unit: int) -> None:
        if unit not in self.live:
            raise ScheduleError(f"unit {unit} is not gathered")
        self.live.remove(unit)
        self.releases[unit] += 1
        self.live_bytes -= self.gather_bytes * self.lay.world * self.lay.shard_u[unit]


class OwnerSchedule:
    """Gather/release state machine of ZeRO-3 with owner broadcast, with
    per-rank counters: a gather of unit u delivers it to every rank but its
    owner, which needs no buffer for it."""

    def __init__(self, lay: Layout, gather_bytes: int = 2, max_live: int = 1):
        self.lay = lay
        self.gather_bytes = gather_bytes
        self.max_live = max_live
        self.live: List[int] = []
        self.gathers = [0] * lay.n_units
        self.releases = [0] * lay.n_units
        self.ag_elems = [0] * lay.world              # received per rank
        self.live_bytes = [0] * lay.world
        self.peak_live_bytes = [0] * lay.world

    def gather(self, unit: int) -> None:
        if unit in self.live:
            raise ScheduleError(f"unit {unit} is already gathered")
        if len(self.live) >= self.max_live:
            raise ScheduleError(f"{len(self.live)} unit(s) live, limit {self.max_live}")
        self.live.append(unit)
        self.gathers[unit] += 1
        size = self.lay.units[unit]
        for r in range(self.lay.world):
            if r != self.lay.owners[unit]:
                self.ag_elems[r] += size
                self.live_bytes[r] += self.gather_bytes * size
                self.peak_live_bytes[r] = max(self.peak_live_bytes[r], self.live_bytes[r])

    def release(self, unit: int) -> None:
        if unit not in self.live:
            raise ScheduleError(f"unit {unit} is not gathered")
        self.live.remove(unit)
        self.releases[unit] += 1
        for r in range(self.lay.world):
            if r != self.lay.owners[unit]:
                self.live_bytes[r] -= self.gather_bytes * self.lay.units[unit]


class _Scheme:
    stage = -1

    def __init__(self, lay: Layout, theta0: np.ndarray, dtype16: str,
                 lr: float = 1e-2, betas=(0.9, 0.999), eps: float = 1e-8):
        if lay.stage != self.stage:
            raise ValueError("layout stage does not match the scheme")
        theta0 = np.asarray(theta0, dtype=np.float32)
        if theta0.shape != (lay.numel,):
            raise ValueError("theta0 must hold Psi fp32 values")
        self.lay, self.dtype = lay, dtype16
        self.hyper = (float(lr), float(betas[0]), float(betas[1]), float(eps))   # lr, beta1, beta2, eps
        self.t = 0
        self.rs_elems = [0] * lay.world     # received per rank
        self.ag_elems = [0] * lay.world
        self.ar_elems = [0] * lay.world
        self._init(self._pad(theta0))

    # padded flat view of a true-parameter-order vector (zeros in the pad)
    def _pad(self, x: np.ndarray) -> np.ndarray:
        lay = self.lay
        out = np.zeros(lay.padded_numel, dtype=x.dtype)
        if lay.stage == 3:
            for u in range(lay.n_units):
                p, q, size = lay.unit_start[u], lay.unit_pstart[u], lay.units[u]
                out[q:q + size] = x[p:p + size]
        else:
            out[:lay.numel] = x
        return out

    def _unpad(self, x: np.ndarray) -> np.ndarray:
        lay = self.lay
        if lay.stage != 3:
            return x[:lay.numel].copy()
        return np.concatenate([x[lay.unit_pstart[u]:lay.unit_pstart[u] + lay.units[u]]
                               for u in range(lay.n_units)])

    def _consts(self) -> nm.AdamConsts:
        return nm.adam_consts(*self.hyper, self.t)

    def _rows(self, grads16: Sequence[np.ndarray]) -> List[np.ndarray]:
        if len(grads16) != self.lay.world:
            raise ValueError("need one gradient vector per rank")
        return [nm.widen16(self._pad(np.asarray(g, dtype=np.uint16)), self.dtype) for g in grads16]

    # results, in true parameter order
    def full_master(self) -> np.ndarray:
        raise NotImplementedError

    def full_m(self) -> np.ndarray:
        raise NotImplementedError

    def full_v(self) -> np.ndarray:
        raise NotImplementedError

    def working_copy(self, rank: int = 0) -> np.ndarray:
        raise NotImplementedError


class DP(_Scheme):
    """Every rank keeps all bands; one all-reduce (mean) per step."""
    stage = 0

    def _init(self, theta: np.ndarray) -> None:
        w = self.lay.world
        self.master = [theta.copy() for _ in range(w)]
        self.m = [np.zeros_like(theta) for _ in range(w)]
        self.v = [np.zeros_like(theta) for _ in range(w)]
        self.p16 = [nm.cast16(theta, self.dtype) for _ in range(w)]

    def step(self, grads16) -> None:
        self.t += 1
        rows = self._rows(grads16)
        avg = nm.reduce_rank_order(rows)               # the all-reduce, mean
        k = self._consts()
        w = self.lay.world
        for r in range(w):
            self.ar_elems[r] += 2 * (w - 1) * (-(-self.lay.numel // w))
            self.master[r], self.m[r], self.v[r] = nm.adam_update(
                self.master[r], self.m[r], self.v[r], avg, k)
            self.p16[r] = nm.cast16(self.master[r], self.dtype)

    def full_master(self):
        return self.master[0].copy()

    def full_m(self):
        return self.m[0].copy()

    def full_v(self):
        return self.v[0].copy()

    def working_copy(self, rank: int = 0):
        return self.p16[rank].copy()


class ZeRO1(_Scheme):
    """Optimizer state sharded; reduce-scatter, Adam on the shard, all-gather."""
    stage = 1

    def _init(self, theta: np.ndarray) -> None:
        lay = self.lay
        self.master, self.m, self.v = [], [], []
        for r in range(lay.world):
            off, n = lay.owned(r)
            self.master.append(theta[off:off + n].copy())
            self.m.append(np.zeros(n, np.float32))
            self.v.append(np.zeros(n, np.float32))
        full16 = nm.cast16(theta, self.dtype)
        self.p16 = [full16.copy() for _ in range(lay.world)]

    def step(self, grads16) -> None:
        self.t += 1
        lay, w = self.lay, self.lay.world
        rows = self._rows(grads16)
        parts = []
        for r in range(w):                              # reduce-scatter, mean
            off, n = lay.owned(r)
            parts.append(nm.reduce_rank_order([row[off:off + n] for row in rows]))
            self.rs_elems[r] += (w - 1) * n
        k = self._consts()
        for r in range(w):
            self.master[r], self.m[r], self.v[r] = nm.adam_update(
                self.master[r], self.m[r], self.v[r], parts[r], k)
        shards16 = [nm.cast16(self.master[r], self.dtype) for r in range(w)]
        gathered = np.concatenate(shards16)             # all-gather of 16-bit shards
        for r in range(w):
            self.ag_elems[r] += (w - 1) * lay.owned(r)[1]
            self.p16[r] = gathered.copy()

    def full_master(self):
        return self._unpad(np.concatenate(self.master))

    def full_m(self):
        return self._unpad(np.concatenate(self.m))

    def full_v(self):
        return self._unpad(np.concatenate(self.v))

    def working_copy(self, rank: int = 0):
        return self._unpad(self.p16[rank])


class ZeRO2(ZeRO1):
    """ZeRO-1 with gradients sharded too: the same arithmetic, different bytes."""
    stage = 2


class ZeRO3(_Scheme):
    """Everything sharded per unit; gather -> use -> release -> re-gather."""
    stage = 3

    def __init__(self, lay: Layout, theta0, dtype16, lr=1e-2, betas=(0.9, 0.999), eps=1e-8,
                 max_live: int = 1, use: Optional[Callable[[str, int, np.ndarray], None]] = None):
        self.schedule = Stage3Schedule(lay, gather_bytes=2, max_live=max_live)
        self.use = use
        super().__init__(lay, theta0, dtype16, lr, betas, eps)

    def _init(self, theta: np.ndarray) -> None:
        lay = self.lay
        # [rank][unit] bands
        self.master = [[None] * lay.n_units for _ in range(lay.world)]
        self.m = [[None] * lay.n_units for _ in range(lay.world)]
        self.v = [[None] * lay.n_units for _ in range(lay.world)]
        self.p16 = [[None] * lay.n_units for _ in range(lay.world)]
        for r in range(lay.world):
            for u in range(lay.n_units):
                off, n = lay.owned(r, u)
                self.master[r][u] = theta[off:off + n].copy()
                self.m[r][u] = np.zeros(n, np.float32)
                self.v[r][u] = np.zeros(n, np.float32)
                self.p16[r][u] = nm.cast16(self.master[r][u], self.dtype)

    def gather(self, unit: int) -> np.ndarray:
        """All-gather of one unit's 16-bit shards into a full unit buffer."""
        self.schedule.gather(unit)
        return np.concatenate([self.p16[r][unit] for r in range(self.lay.world)])

    def release(self, unit: int) -> None:
        self.schedule.release(unit)

    def _use(self, phase: str, unit: int, buf: np.ndarray) -> None:
        if self.use is not None:
            self.use(phase, unit, buf)

    def step(self, grads16) -> None:
        self.t += 1
        lay, w = self.lay, self.lay.world
        rows = self._rows(grads16)
        k = self._consts()
        for u in range(lay.n_units):                         # forward
            buf = self.gather(u)
            self._use("forward", u, buf)
            self.release(u)
        for u in reversed(range(lay.n_units)):               # backward
            buf = self.gather(u)
            self._use("backward", u, buf)
            for r in range(w):
                off, n = lay.owned(r, u)
                g = nm.reduce_rank_order([row[off:off + n] for row in rows])
                self.rs_elems[r] += (w - 1) * n
                self.master[r][u], self.m[r][u], self.v[r][u] = nm.adam_update(
                    self.master[r][u], self.m[r][u], self.v[r][u], g, k)
                self.p16[r][u] = nm.cast16(self.master[r][u], self.dtype)
            self.release(u)
        for r in range(w):
            self.ag_elems[r] = self.schedule.ag_elems

    def _padded(self, band) -> np.ndarray:
        lay = self.lay
        return np.concatenate([band[r][u] for u in range(lay.n_units) for r in range(lay.world)])

    def full_master(self):
        return self._unpad(self._padded(self.master))

    def full_m(self):
        return self._unpad(self._padded(self.m))

    def full_v(self):
        return self._unpad(self._padded(self.v))

    def working_copy(self, rank: int = 0):
        return self._unpad(self._padded(self.p16))


class ZeRO3Owner(_Scheme):
    """ZeRO-3 with whole units owned by single ranks: the owner broadcasts a
    unit when it is needed; gradients are reduced onto the owner."""
    stage = 3

    def __init__(self, lay: Layout, theta0, dtype16, lr=1e-2, betas=(0.9, 0.999), eps=1e-8,
                 max_live: int = 1, use: Optional[Callable[[str, int, np.ndarray], None]] = None):
        if not lay.owner_broadcast:
            raise ValueError("ZeRO3Owner needs an owner-broadcast layout")
        self.schedule = OwnerSchedule(lay, gather_bytes=2, max_live=max_live)
        self.use = use
        super().__init__(lay, theta0, dtype16, lr, betas, eps)

    def _init(self, theta: np.ndarray) -> None:
        lay = self.lay
        # unit u's bands live on its owner only
        self.master, self.m, self.v, self.p16 = {}, {}, {}, {}
        for u in range(lay.n_units):
            p, n = lay.unit_start[u], lay.units[u]
            self.master[u] = theta[p:p + n].copy()
            self.m[u] = np.zeros(n, np.float32)
            self.v[u] = np.zeros(n, np.float32)
            self.p16[u] = nm.cast16(self.master[u], self.dtype)

    def gather(self, unit: int) -> np.ndarray:
        """The owner's 16-bit copy of the unit, as every other rank receives it."""
        self.schedule.gather(unit)
        return self.p16[unit].copy()

    def release(self, unit: int) -> None:
        self.schedule.release(unit)

    def _use(self, phase: str, unit: int, buf: np.ndarray) -> None:
        if self.use is not None:
            self.use(phase, unit, buf)

    def step(self, grads16) -> None:
        self.t += 1
        lay, w = self.lay, self.lay.world
        rows = self._rows(grads16)
        k = self._consts()
        for u in range(lay.n_units):                         # forward
            buf = self.gather(u)
            self._use("forward", u, buf)
            self.release(u)
        for u in reversed(range(lay.n_units)):               # backward
            buf = self.gather(u)
            self._use("backward", u, buf)
            p, n, owner = lay.unit_start[u], lay.units[u], lay.owners[u]
            g = nm.reduce_rank_order([row[p:p + n] for row in rows])
            for r in range(w):
                if r != owner:
                    self.rs_elems[r] += n                    # r's contribution to the owner
            self.master[u], self.m[u], self.v[u] = nm.adam_update(
                self.master[u], self.m[u], self.v[u], g, k)
            self.p16[u] = nm.cast16(self.master[u], self.dtype)
            self.release(u)
        self.ag_elems = list(self.schedule.ag_elems)

    def _cat(self, band) -> np.ndarray:
        return np.concatenate([band[u] for u in range(self.lay.n_units)])

    def full_master(self):
        return self._cat(self.master)

    def full_m(self):
        return self._cat(self.m)

    def full_v(self):
        return self._cat(self.v)

    def working_copy(self, rank: int = 0):
        return self._cat(self.p16)


SCHEMES = {0: DP, 1: ZeRO1, 2: ZeRO2, 3: ZeRO3}


def run(stage: int, numel: int, world: int, theta0: np.ndarray,
        grads_per_step: Callable[[int], Sequence[np.ndarray]], steps: int, dtype16: str,
        lr: float, betas=(0.9, 0.999), eps: float = 1e-8, units=None, pad: bool = False,
        owner_broadcast: bool = False, owners=None, **kw):
    """Build a scheme and run ``steps`` steps; ``grads_per_step(t)`` returns the
    N per-rank 16-bit gradient vectors of step t (t = 1..steps).  Stage 3 with
    ``owner_broadcast`` runs ``ZeRO3Owner``, its units owned as ``owners``
    says (None: the layout's default reading)."""
    lay = make_layout(numel, world, stage, units, pad, owner_broadcast, owners)
    cls = ZeRO3Owner if owner_broadcast else SCHEMES[stage]
    sch = cls(lay, theta0, dtype16, lr, betas, eps, **kw)
    for t in range(1, steps + 1):
        sch.step(grads_per_step(t))
    return sch
