"""Exact per-rank memory and traffic accounting for DP and ZeRO-1/2/3.

Test infrastructure only (see the package header).  Python integers throughout.

Bands and their bytes per element: 16-bit working parameters 2, 16-bit
gradients 2, fp32 master, m and v 4 each, 16 in all ("One Poem Suffices: ZeRO"
section 3.1, the model-states equation; "ZeRO, annotated" section 3.1; "The
four schemes", the per-band byte constants).  Which bands a stage shards
follows the three flags of "The four schemes" (optimizer state from stage 1,
gradients from stage 2, parameters at stage 3), which give the per-rank
totals 16*Psi, 4*Psi + 12*Psi/N, 2*Psi + 14*Psi/N and 16*Psi/N ("ZeRO and
FSDP", the three-stage table; "One Poem Suffices: ZeRO" sections 4.1.1-4.1.3).

Readings where the pages leave a step open:
* A sharded band counts the padded shard S = ceil(Psi/N) (per unit at stage 3,
  ceil(P_u/N)); an unsharded band counts the true Psi.  This is what makes
  ``ZeroAdam``'s printed 57,636 bytes ("ZeRO and FSDP", zero_check output).
* Peak ("The four schemes", the resident-vs-peak table): equal to resident for
  stages 0-2; at stage 3 resident plus the gathered unit(s) that are live at
  once, at ``gather_bytes`` per element (16-bit by default; the prototype
  gathers fp32, which is ``gather_bytes=4``).  The unit's full gradient is
  reported on its own, not in the peak, as the prototype does.
* Traffic ("ZeRO, annotated" section 7; "One Poem Suffices: ZeRO" section
  4.1.4 and Appendix B; "Sharding the States."): elements each rank sends per
  step, exactly (N-1) shards per ring collective.  Data parallel runs one
  all-reduce (a reduce-scatter plus an all-gather, 2(N-1) chunks of
  ceil(Psi/N)); stages 1-2 a reduce-scatter plus an all-gather; stage 3 two
  all-gathers plus a reduce-scatter.  Bytes are elements times 2 (16-bit
  gradients and parameters on the wire).
* Stage 3 with owner broadcast ("One Poem Suffices: ZeRO" section 4.1.4;
  "ZeRO, annotated" section 7, "Stage 3, step by step"): rank r keeps the
  16 bytes per element of its own units only, own(r) elements.  Each weight
  comes in twice (forward and backward) and each gradient goes once to its
  owner, so r receives 2(Psi - own(r)) and sends Psi - own(r) elements per
  step; with equal shares that is the same 3(N-1)/N Psi as the split layout.
  Its peak adds the borrowed units live at once (its own units need no
  buffer): at most ``max_live`` consecutive units of the schedule, counting
  only units r does not own.  Ranks differ when the units do not split
  evenly; ``rank=None`` reports the rank with the largest peak.
"""
from __future__ import annotations

from dataclasses import dataclass

from .layout import Layout

# Bytes one element occupies in each band: the 16-bit working parameters and
# gradients, and the fp32 master copy and Adam's two moments (16 in all).
BAND_BYTES = {"p16": 2, "grad": 2, "master": 4, "m": 4, "v": 4}
BANDS = tuple(BAND_BYTES)

# Bytes per element on the wire: the collectives move 16-bit values.
WIRE_BYTES = 2

# The bands each stage splits N ways (the others every rank holds whole):
# stage 1 the optimizer state, stage 2 also the gradients, stage 3 also the
# working parameters.
SHARDED_BANDS = {0: frozenset(),
                 1: frozenset({"master", "m", "v"}),
                 2: frozenset({"master", "m", "v", "grad"}),
                 3: frozenset(BANDS)}


@dataclass(frozen=True)
class Bytes:
    res_p16: int
    res_grad: int
    res_master: int
    res_m: int
    res_v: int
    resident: int
    gathered: int          # bytes of gathered units live at the worst moment
    peak: int
    unit_grad: int         # full 16-bit gradient of the largest unit (stage 3)
    rs_elems: int
    ag_elems: int
    ar_elems: int
    traffic_elems: int
    traffic_bytes: int


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _owner_bytes(lay: Layout, rank: int, gather_bytes: int, max_live: int) -> Bytes:
    own = lay.own_numel(rank)
    res = {band: BAND_BYTES[band] * own for band in BANDS}
    resident = sum(res.values())
    borrowed = [0 if o == rank else size for size, o in zip(lay.units, lay.owners)]
    k = max(1, min(max_live, len(borrowed)))
    gathered = gather_bytes * max(sum(borrowed[i:i + k]) for i in range(len(borrowed) - k + 1))
    unit_grad = BAND_BYTES["grad"] * max(lay.units)
    rs = lay.numel - own
    ag = 2 * (lay.numel - own)
    elems = rs + ag
    return Bytes(*(res[band] for band in BANDS), resident, gathered, resident + gathered, unit_grad,
                 rs, ag, 0, elems, elems * WIRE_BYTES)


def bytes_per_rank(lay: Layout, gather_bytes: int = 2, max_live: int = 1,
                   rank=None) -> Bytes:
    if lay.owner_broadcast:
        if rank is not None:
            return _owner_bytes(lay, rank, gather_bytes, max_live)
        per = [_owner_bytes(lay, r, gather_bytes, max_live) for r in range(lay.world)]
        return max(per, key=lambda b: b.peak)        # max() keeps the first (lowest) rank on ties
    n, w = lay.numel, lay.world
    sharded = SHARDED_BANDS[lay.stage]
    s_tot = lay.shard_numel if lay.stage else n
    res = {band: BAND_BYTES[band] * (s_tot if band in sharded else n) for band in BANDS}
    resident = sum(res.values())

    gathered = 0
    unit_grad = 0
    if lay.stage == 3:
        widths = [w * s for s in lay.shard_u]
        k = max(1, min(max_live, len(widths)))
        gathered = gather_bytes * max(sum(widths[i:i + k]) for i in range(len(widths) - k + 1))
        unit_grad = BAND_BYTES["grad"] * max(widths)
    peak = resident + gathered

    rs = ag = ar = 0
    if lay.stage == 0:
        ar = 2 * (w - 1) * _ceil_div(n, w)
    elif lay.stage in (1, 2):
        rs = (w - 1) * s_tot
        ag = (w - 1) * s_tot
    else:
        rs = (w - 1) * s_tot
        ag = 2 * (w - 1) * s_tot
    elems = rs + ag + ar
    return Bytes(*(res[band] for band in BANDS), resident, gathered, peak, unit_grad,
                 rs, ag, ar, elems, elems * WIRE_BYTES)


def bytes_per_param(lay: Layout, gather_bytes: int = 2):
    """(resident, peak) per parameter, as the prototype prints them."""
    b = bytes_per_rank(lay, gather_bytes)
    return b.resident / lay.numel, b.peak / lay.numel


def optimizer_state_bytes(lay: Layout) -> int:
    """fp32 master + m + v one rank holds (``ZeroAdam.state_bytes``)."""
    b = bytes_per_rank(lay)
    return b.res_master + b.res_m + b.res_v
