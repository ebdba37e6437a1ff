"""Partition of the flat parameter vector over N simulated ranks.

Test infrastructure only (see the package header).

* Stages 0-2 ("The four schemes", ``Base.__init__``; "ZeRO and FSDP",
  ``ZeroAdam.__init__``): the vector of Psi elements is split into N equal
  contiguous shards, rank r owning [r*S, (r+1)*S).  The prototype refuses a
  Psi that N does not divide; ``ZeroAdam`` pads with zeros to N*ceil(Psi/N).
  Both readings are offered: ``pad=False`` raises, ``pad=True`` pads.
* Stage 3 ("ZeRO and FSDP", "ZeRO-3 and FSDP"): the model is cut into units
  (a layer or a few) and each unit is split N ways on its own, with its own
  zero pad; rank r owns [Q_u + r*S_u, Q_u + (r+1)*S_u) of the padded vector,
  where Q_u is the padded start of unit u.  Data parallel keeps no shard: the
  rank's "owned" range is the whole vector.
* Stage 3, owner broadcast ("One Poem Suffices: ZeRO" section 4.1.4, the
  64-device, 192-block example; "ZeRO, annotated" sections 5.3 and 7, where
  GPU i owns shard i): every unit belongs whole to one rank, which sends it to
  the others when it is needed.  Nothing is padded; the vector keeps its
  natural order.  The pages only show equal partitions (each rank owning the
  same number of equal blocks, k consecutive ones when U = k*N).  Any other
  owner map is the caller's choice and is passed in as ``owners``; without
  one, the default is a reading: unit u goes to the rank whose equal share
  [r*Psi/N, (r+1)*Psi/N) holds the unit's midpoint, which gives exactly the
  pages' contiguous k-blocks-per-rank ownership on equal partitions and is
  parity unpinned on unequal units.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence


class IndivisibleError(ValueError):
    """Psi (or a ZeRO-3 unit) does not divide by N and padding was not asked for."""


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass(frozen=True)
class Layout:
    numel: int                  # Psi, true parameter count
    world: int                  # N
    stage: int                  # 0 = data parallel, 1, 2, 3
    units: tuple                # true element count of each unit
    pad: bool
    shard_u: tuple              # S_u per unit (stage 3); (S,) for stages 1-2; (Psi,) for DP
    unit_start: tuple           # true start P_u of each unit in [0, Psi)
    unit_pstart: tuple          # padded start Q_u of each unit
    owners: tuple = ()          # owner broadcast: the rank owning each unit; () otherwise

    @property
    def owner_broadcast(self) -> bool:
        return bool(self.owners)

    @property
    def n_units(self) -> int:
        return len(self.units)

    @property
    def padded_numel(self) -> int:
        if self.stage == 0 or self.owner_broadcast:
            return self.numel
        return sum(self.world * s for s in self.shard_u)

    def own_numel(self, rank: int) -> int:
        """Elements of optimizer state ``rank`` keeps."""
        if self.owner_broadcast:
            return sum(n for n, o in zip(self.units, self.owners) if o == rank)
        return self.shard_numel

    @property
    def shard_numel(self) -> int:
        """Elements of optimizer state each rank keeps (owner broadcast: the
        largest over the ranks)."""
        if self.owner_broadcast:
            return max(self.own_numel(r) for r in range(self.world))
        return sum(self.shard_u)

    def owned(self, rank: int, unit: int = 0):
        """(padded offset, length) of what ``rank`` owns in ``unit``."""
        if not 0 <= rank < self.world:
            raise IndexError(rank)
        if self.stage == 0:
            if unit != 0:
                raise IndexError(unit)
            return 0, self.numel
        if self.stage in (1, 2):
            if unit != 0:
                raise IndexError(unit)
            s = self.shard_u[0]
            return rank * s, s
        if self.owner_broadcast:
            return self.unit_start[unit], (self.units[unit] if self.owners[unit] == rank else 0)
        s = self.shard_u[unit]
        return self.unit_pstart[unit] + rank * s, s

    def local_offset(self, unit: int) -> int:
        """Offset of ``unit``'s piece inside a rank's concatenated shard (owner
        broadcast: inside its owner's concatenated units)."""
        if self.owner_broadcast:
            o = self.owners[unit]
            return sum(self.units[v] for v in range(unit) if self.owners[v] == o)
        return sum(self.shard_u[:unit])

    def param_index(self, padded_pos: int) -> Optional[int]:
        """True parameter index held at a padded position, or None for pad."""
        if self.stage == 0 or self.owner_broadcast:
            return padded_pos if 0 <= padded_pos < self.numel else None
        if self.stage in (1, 2):
            return padded_pos if padded_pos < self.numel else None
        for u in range(self.n_units):
            q, width = self.unit_pstart[u], self.world * self.shard_u[u]
            if q <= padded_pos < q + width:
                k = padded_pos - q
                return self.unit_start[u] + k if k < self.units[u] else None
        return None

    def padded_to_param(self, positions) -> "tuple":
        """Vectorised ``param_index``: (param indices, valid mask) for positions."""
        import numpy as np
        pos = np.asarray(positions, dtype=np.int64)
        if self.stage in (0, 1, 2) or self.owner_broadcast:
            return pos.copy(), pos < self.numel
        par = np.zeros_like(pos)
        ok = np.zeros(pos.shape, dtype=bool)
        for u in range(self.n_units):
            q, width = self.unit_pstart[u], self.world * self.shard_u[u]
            inside = (pos >= q) & (pos < q + width)
            k = pos - q
            hit = inside & (k < self.units[u])
            par = np.where(hit, self.unit_start[u] + k, par)
            ok |= hit
        return par, ok


def unit_owners(units: Sequence[int], world: int) -> tuple:
    """Owner of each unit under owner broadcast: the rank whose equal share of
    the vector holds the unit's midpoint, floor(N * (start + size/2) / Psi).
    On equal partitions this gives the pages' k consecutive units per rank
    ("One Poem Suffices: ZeRO" section 4.1.4; "ZeRO, annotated" section 7);
    on unequal units it is a reading, parity unpinned."""
    numel = sum(units)
    owners, start = [], 0
    for size in units:
        owners.append(min(world - 1, (world * (2 * start + size)) // (2 * numel)))
        start += size
    return tuple(owners)


def pages_owners(n_units: int, world: int) -> tuple:
    """The pages' owner map for U = k*N equal units: rank r owns the k
    consecutive units [r*k, (r+1)*k) ("One Poem Suffices: ZeRO" section 4.1.4,
    192 blocks on 64 devices, 3 each; "ZeRO, annotated" section 7, GPU i owns
    shard i)."""
    if n_units % world:
        raise ValueError("the pages' partition needs a multiple of N units")
    k = n_units // world
    return tuple(u // k for u in range(n_units))


def make_layout(numel: int, world: int, stage: int, units: Optional[Sequence[int]] = None,
                pad: bool = False, owner_broadcast: bool = False,
                owners: Optional[Sequence[int]] = None) -> Layout:
    """``owners`` (owner broadcast only): the rank owning each unit; None
    takes the midpoint reading of ``unit_owners``."""
    if numel < 1 or world < 1 or stage not in (0, 1, 2, 3):
        raise ValueError("bad numel/world/stage")
    if owner_broadcast and stage != 3:
        raise ValueError("owner broadcast is a stage-3 layout")
    if owners is not None and not owner_broadcast:
        raise ValueError("an owner map belongs to the owner-broadcast layout")
    unit_list: List[int] = list(units) if units else [numel]
    if any(u < 1 for u in unit_list) or sum(unit_list) != numel:
        raise ValueError("unit sizes must be positive and sum to numel")
    starts = [sum(unit_list[:i]) for i in range(len(unit_list))]
    if owner_broadcast:
        if owners is None:
            owner_map = unit_owners(unit_list, world)
        else:
            owner_map = tuple(int(o) for o in owners)
            if len(owner_map) != len(unit_list) or any(not 0 <= o < world for o in owner_map):
                raise ValueError("one owner in [0, N) per unit")
        return Layout(numel, world, 3, tuple(unit_list), pad, tuple(unit_list), tuple(starts),
                      tuple(starts), owner_map)
    if stage == 0:
        shard_u = (numel,)
    elif stage in (1, 2):
        if numel % world and not pad:
            raise IndivisibleError(f"{numel} parameters do not split into {world} equal shards (pad=True pads)")
        shard_u = (_ceil_div(numel, world),)
    else:
        for u in unit_list:
            if u % world and not pad:
                raise IndivisibleError(f"a unit of {u} parameters does not split into {world} equal shards")
        shard_u = tuple(_ceil_div(u, world) for u in unit_list)
    if stage == 3:
        pstarts = tuple(sum(world * s for s in shard_u[:i]) for i in range(len(shard_u)))
    else:
        pstarts = tuple(starts)
    return Layout(numel, world, stage, tuple(unit_list), pad, shard_u, tuple(starts), pstarts)
