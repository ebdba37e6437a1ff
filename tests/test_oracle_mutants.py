"""Planted mistakes: the oracle's pins must each be able to fail.

Every case below plants one plausible mistake in the oracle, on the CPU, by
replacing one oracle function (or constant) with a copy that differs from it
in exactly that mistake: a dropped term, a wrong constant, a swapped operand,
a wrong index, a wrong rounding.  The pins of ``test_oracle_*.py`` then run
against the mutated oracle, and at least one of them must fail; a mutant that
every pin accepts would be a mistake the pins cannot see.  The unmutated
oracle passes every pin (the control case).  Nothing here touches the GPU or
the HIP library.
"""
import dataclasses

import numpy as np
import pytest
import torch

import test_oracle_accounting as pa
import test_oracle_numerics as pn
import test_oracle_schemes as ps
from oracle import accounting as acc
from oracle import layout as lo
from oracle import numerics as nm
from oracle import sampled
from oracle import schemes as sc

# ------------------------------------------------------------ the pins ------
# each entry: (name, callable); a pin fails by raising AssertionError

NUMERIC_PINS = [
    ("cast bf16 vs torch", lambda: pn.test_cast16_matches_torch_rne("bf16", torch.bfloat16)),
    ("cast fp16 vs torch", lambda: pn.test_cast16_matches_torch_rne("fp16", torch.float16)),
    ("cast ties to even", pn.test_cast16_ties_go_to_even),
    ("widen bf16 vs torch", lambda: pn.test_widen16_all_patterns("bf16", torch.bfloat16)),
    ("widen fp16 vs torch", lambda: pn.test_widen16_all_patterns("fp16", torch.float16)),
    ("reduce brute force", pn.test_reduce_brute_force_error_bound),
    ("reduce rank order", pn.test_reduce_is_rank_order_fp32),
    ("reduce special cases", pn.test_reduce_special_cases),
    ("adam g=0", pn.test_adam_zero_gradient_leaves_master_bit_unchanged),
    ("adam t=1 closed form", pn.test_adam_first_step_closed_form),
    ("adam constant-g closed form", pn.test_adam_constant_gradient_closed_form),
    ("adam vs torch.optim.Adam", pn.test_adam_matches_torch_optim_adam),
    ("small MLP against torch.optim.Adam", pn.test_sharded_adam_on_a_small_mlp_matches_torch_adam),
]


def _all_page_values():
    for pin in pa.PINS:
        pa.test_page_printed_value(pin)


ACCOUNTING_PINS = [
    ("page-printed values", _all_page_values),
    ("16 bytes per parameter", pa.test_sixteen_bytes_per_parameter),
    ("closed forms", lambda: [pa.test_closed_forms(n, w) for n, w in
                              [(8, 4), (65536, 4), (124439808, 8), (7_500_000_000, 64)]]),
    ("traffic forms", lambda: [pa.test_traffic_ratio_and_exact_forms(n, w) for n, w in
                               [(8, 4), (65536, 4), (7_500_000_000, 64)]]),
    ("stage-3 peak", pa.test_stage3_peak_is_resident_plus_gathered_unit),
    ("prefetch peak", pa.test_prefetch_peak_two_live_units),
    ("padding readings", pa.test_padding_readings),
    ("owned ranges tile the vector", pa.test_layout_owned_ranges_tile_the_padded_vector),
    ("owner partitions", pa.test_owner_rule_gives_the_pages_contiguous_partitions),
    ("owner per-rank forms", pa.test_owner_accounting_per_rank_closed_forms),
    ("owner peak 2/64", pa.test_owner_peak_two_64ths_either_reading),
    ("owner = split when balanced", lambda: [pa.test_owner_balanced_equals_split_layout(w, k)
                                             for w, k in [(4, 1), (4, 3), (8, 4), (64, 3)]]),
    ("owner forms for any map", pa.test_owner_accounting_closed_forms_for_any_map),
    ("one count for Llama 3 70B", pa.test_one_parameter_count_reproduces_the_unprinted_model),
]

SCHEME_PINS = [
    ("world of one is plain Adam", ps.test_world_of_one_is_plain_adam_on_the_gradient),
    ("all schemes bit-identical", lambda: ps.test_all_schemes_bit_identical(
        4096, 8, "bf16", 1e-3, [1024, 512, 2048, 512])),
    ("zero gradients change nothing", ps.test_zero_gradients_leave_everything_unchanged),
    ("padding tail stays zero", lambda: [ps.test_padding_tail_stays_zero(s) for s in (1, 2, 3)]),
    ("stage-3 gathers twice", lambda: ps.test_stage3_gathers_twice_and_counts_traffic([16384] * 4)),
    ("sampled = full run", ps.test_sampled_trajectory_matches_full_run),
]


def first_failing(pins):
    """Name of the first pin that fails, or None if all pass."""
    for name, pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            return name
    return None


# ------------------------------------------------------ numerics mutants ----
def adam_variant(eps_inside=False, no_bc1=False, no_bc2=False, sign=-1.0, v_one_g=False,
                 m_uses_b2=False, no_lr=False, swap_mv=False, v_no_square_scale=False):
    """The oracle's Adam update with the named mistake planted."""
    def update(master, m, v, g, k):
        g = np.asarray(g, dtype=np.float32)
        m = (k.c2 if m_uses_b2 else k.c1) * m + (k.c2m if m_uses_b2 else k.c1m) * g
        if v_one_g:
            v = k.c2 * v + k.c2m * g
        elif v_no_square_scale:
            v = k.c2 * v + g * g
        else:
            v = k.c2 * v + (k.c2m * g) * g
        mh = m if no_bc1 else m / k.bc1
        vh = v if no_bc2 else v / k.bc2
        d = np.sqrt(vh + k.eps) if eps_inside else np.sqrt(vh) + k.eps
        u = mh / d if no_lr else (k.lr * mh) / d
        master = master + np.float32(sign) * u
        out = (master.astype(np.float32), m.astype(np.float32), v.astype(np.float32))
        return (out[0], out[2], out[1]) if swap_mv else out
    return update


def consts_variant(t_shift=0, swap_betas=False, bc_from_lr=False):
    def consts(lr, b1, b2, eps, t):
        if t < 1:
            raise ValueError("t counts from 1")
        if swap_betas:
            b1, b2 = b2, b1
        f = np.float32
        tt = t + t_shift
        bc1, bc2 = 1.0 - b1 ** tt, 1.0 - b2 ** tt
        if bc_from_lr:
            bc1 = bc2 = 1.0 - lr ** tt
        return nm.AdamConsts(f(b1), f(1.0 - b1), f(b2), f(1.0 - b2), f(bc1), f(bc2), f(lr), f(eps))
    return consts


def reduce_variant(mean_by=None, reverse=False, drop_last=False, drop_first=False, acc16=False,
                   no_mean=False):
    def reduce(rows, mean=True):
        rows = [np.asarray(r, dtype=np.float32) for r in rows]
        if reverse:
            rows = rows[::-1]
        if drop_last and len(rows) > 1:
            rows = rows[:-1]
        if drop_first and len(rows) > 1:
            rows = rows[1:]
        acc_ = rows[0].copy()
        for r in rows[1:]:
            acc_ = acc_ + r
            if acc16:                     # accumulate in bf16: round each partial sum
                acc_ = nm.widen16(nm.cast16(acc_, "bf16"), "bf16")
        if mean and not no_mean:
            n = len(rows) if mean_by is None else mean_by(len(rows))
            acc_ = acc_ / np.float32(n)
        return acc_
    return reduce


_cast16 = nm.cast16


def cast_truncate(x, dtype):
    if dtype != "bf16":
        return _cast16(x, dtype)
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def cast_ties_away(x, dtype):
    if dtype != "bf16":
        return _cast16(x, dtype)
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x8000)) >> np.uint64(16)) & np.uint64(0xFFFF)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    return np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), r).astype(np.uint16)


def cast_fp16_last_bit_flipped(x, dtype):
    if dtype != "fp16":
        return _cast16(x, dtype)
    return _cast16(x, dtype) ^ np.uint16(1)


_widen16 = nm.widen16


def widen_swapped(bits, dtype):
    return _widen16(bits, "fp16" if dtype == "bf16" else "bf16")


def widen_fp16_flush_subnormals(bits, dtype):
    out = _widen16(bits, dtype)
    if dtype == "fp16":
        b = np.ascontiguousarray(bits, dtype=np.uint16)
        sub = (b & np.uint16(0x7C00)) == 0
        out = np.where(sub, np.float32(0.0) * np.sign(out), out).astype(np.float32)
    return out


NUMERIC_MUTANTS = {
    "eps inside the square root": ("adam_update", adam_variant(eps_inside=True)),
    "no bias correction of m": ("adam_update", adam_variant(no_bc1=True)),
    "no bias correction of v": ("adam_update", adam_variant(no_bc2=True)),
    "update added instead of subtracted": ("adam_update", adam_variant(sign=+1.0)),
    "v takes g once, not g squared": ("adam_update", adam_variant(v_one_g=True)),
    "v without the (1 - b2) factor": ("adam_update", adam_variant(v_no_square_scale=True)),
    "m uses b2": ("adam_update", adam_variant(m_uses_b2=True)),
    "learning rate dropped": ("adam_update", adam_variant(no_lr=True)),
    "m and v swapped on return": ("adam_update", adam_variant(swap_mv=True)),
    "bias correction one step late (t - 1)": ("adam_consts", consts_variant(t_shift=-1)),
    "bias correction one step early (t + 1)": ("adam_consts", consts_variant(t_shift=+1)),
    "b1 and b2 swapped": ("adam_consts", consts_variant(swap_betas=True)),
    "bias correction from lr": ("adam_consts", consts_variant(bc_from_lr=True)),
    "reduce sums without the mean": ("reduce_rank_order", reduce_variant(no_mean=True)),
    "reduce divides by N - 1": ("reduce_rank_order", reduce_variant(mean_by=lambda n: max(n - 1, 1))),
    "reduce in reverse rank order": ("reduce_rank_order", reduce_variant(reverse=True)),
    "reduce drops the last rank": ("reduce_rank_order", reduce_variant(drop_last=True)),
    "reduce drops rank 0": ("reduce_rank_order", reduce_variant(drop_first=True)),
    "reduce accumulates in 16 bits": ("reduce_rank_order", reduce_variant(acc16=True)),
    "bf16 cast truncates": ("cast16", cast_truncate),
    "bf16 cast rounds ties away from zero": ("cast16", cast_ties_away),
    "fp16 cast off by one unit": ("cast16", cast_fp16_last_bit_flipped),
    "widen swaps the 16-bit formats": ("widen16", widen_swapped),
    "widen flushes fp16 subnormals": ("widen16", widen_fp16_flush_subnormals),
}


def test_control_every_pin_passes_unmutated():
    assert first_failing(NUMERIC_PINS + ACCOUNTING_PINS + SCHEME_PINS) is None


@pytest.mark.parametrize("name", list(NUMERIC_MUTANTS))
def test_numeric_mutant_is_caught(name, monkeypatch):
    attr, fn = NUMERIC_MUTANTS[name]
    monkeypatch.setattr(nm, attr, fn)
    caught = first_failing(NUMERIC_PINS + SCHEME_PINS)
    assert caught is not None, f"no pin fails with the planted mistake: {name}"


# ---------------------------------------------------- accounting mutants ----
_bytes_per_rank = acc.bytes_per_rank


def _bytes_with(change):
    """bytes_per_rank with one field rule changed after the fact."""
    def f(lay, gather_bytes=2, max_live=1, rank=None):
        b = _bytes_per_rank(lay, gather_bytes, max_live, rank)
        b2 = change(lay, b)
        if b2 is not b:
            te = b2.rs_elems + b2.ag_elems + b2.ar_elems
            b2 = dataclasses.replace(b2, traffic_elems=te, traffic_bytes=te * acc.WIRE_BYTES)
        return b2
    return f


def _stage3_one_gather(lay, b):
    if lay.stage == 3 and not lay.owner_broadcast:
        return dataclasses.replace(b, ag_elems=b.ag_elems // 2)
    return b


def _dp_one_collective(lay, b):
    return dataclasses.replace(b, ar_elems=b.ar_elems // 2) if lay.stage == 0 else b


def _traffic_all_n(lay, b):
    # N shards per collective instead of N - 1
    if lay.stage in (1, 2) and not lay.owner_broadcast and lay.world > 1:
        k = lay.world / (lay.world - 1)
        return dataclasses.replace(b, rs_elems=int(b.rs_elems * k), ag_elems=int(b.ag_elems * k))
    return b


def _peak_without_gather(lay, b):
    return dataclasses.replace(b, peak=b.resident, gathered=0) if lay.stage == 3 else b


def _resident_drops_grad(lay, b):
    return dataclasses.replace(b, res_grad=0, resident=b.resident - b.res_grad)


ACCOUNTING_MUTANTS = {
    "stage 3 counts one all-gather": ("bytes_per_rank", _bytes_with(_stage3_one_gather)),
    "data parallel counts one collective": ("bytes_per_rank", _bytes_with(_dp_one_collective)),
    "collectives send N shards, not N - 1": ("bytes_per_rank", _bytes_with(_traffic_all_n)),
    "stage-3 peak omits the gathered unit": ("bytes_per_rank", _bytes_with(_peak_without_gather)),
    "gradient band not counted": ("bytes_per_rank", _bytes_with(_resident_drops_grad)),
    "stage 2 keeps full gradients": ("SHARDED_BANDS", {**acc.SHARDED_BANDS, 2: frozenset({"master", "m", "v"})}),
    "stage 1 shards gradients": ("SHARDED_BANDS", {**acc.SHARDED_BANDS, 1: frozenset({"master", "m", "v", "grad"})}),
    "stage 3 keeps full parameters": ("SHARDED_BANDS", {**acc.SHARDED_BANDS, 3: acc.SHARDED_BANDS[2]}),
    "fp32 on the wire": ("WIRE_BYTES", 4),
    "master counted at 2 bytes": ("BAND_BYTES", {**acc.BAND_BYTES, "master": 2}),
    "gradients counted at 4 bytes": ("BAND_BYTES", {**acc.BAND_BYTES, "grad": 4}),
}


# ------------------------------------------------ layout / scheme mutants ---
_owned = lo.Layout.owned
_ceil = lo._ceil_div


def owned_off_by_one(self, rank, unit=0):
    off, n = _owned(self, rank, unit)
    return (off + 1, n) if rank == self.world - 1 and n else (off, n)


def owned_ranks_reversed(self, rank, unit=0):
    return _owned(self, self.world - 1 - rank, unit)


def owned_short_last(self, rank, unit=0):
    off, n = _owned(self, rank, unit)
    return (off, n - 1) if rank == self.world - 1 and n > 1 else (off, n)


_consts = sc._Scheme._consts


def consts_per_unit_clock(self):
    # t advanced by one more each time the constants are taken: as if the step
    # counter moved per unit or per rank instead of once per step
    self._extra = getattr(self, "_extra", 0) + 1
    return nm.adam_consts(*self.hyper, self.t + self._extra - 1)


LAYOUT_MUTANTS = {
    "last rank's shard one element late": (lo.Layout, "owned", owned_off_by_one),
    "shorter last shard": (lo.Layout, "owned", owned_short_last),
    "padding by floor, not ceil": (lo, "_ceil_div", lambda a, b: a // b),
}

# owner broadcast (stage 3 with whole units owned by single ranks)
_owner_bytes = acc._owner_bytes


def _owner_with(change):
    def f(lay, rank, gather_bytes, max_live):
        return change(lay, rank, _owner_bytes(lay, rank, gather_bytes, max_live), gather_bytes, max_live)
    return f


def _own_units_counted_as_borrowed(lay, rank, b, gather_bytes, max_live):
    k = max(1, min(max_live, len(lay.units)))
    g = gather_bytes * max(sum(lay.units[i:i + k]) for i in range(len(lay.units) - k + 1))
    return dataclasses.replace(b, gathered=g, peak=b.resident + g)


def _receives_whole_vector(lay, rank, b, gather_bytes, max_live):
    ag = 2 * lay.numel
    te = b.rs_elems + ag
    return dataclasses.replace(b, ag_elems=ag, traffic_elems=te, traffic_bytes=te * acc.WIRE_BYTES)


def _gradients_sent_twice(lay, rank, b, gather_bytes, max_live):
    rs = 2 * b.rs_elems
    te = rs + b.ag_elems
    return dataclasses.replace(b, rs_elems=rs, traffic_elems=te, traffic_bytes=te * acc.WIRE_BYTES)


def _resident_of_the_largest_owner(lay, rank, b, gather_bytes, max_live):
    big = 16 * max(lay.own_numel(r) for r in range(lay.world))
    return dataclasses.replace(b, resident=big, peak=big + b.gathered)


_unit_owners = lo.unit_owners


def owners_by_start(units, world):
    numel, out, start = sum(units), [], 0
    for size in units:
        out.append(min(world - 1, world * start // numel))
        start += size
    return tuple(out)


def owners_shifted(units, world):
    return tuple(min(world - 1, o + 1) for o in _unit_owners(units, world))


ACCOUNTING_MUTANTS.update({
    "owner: its own units counted as borrowed": ("_owner_bytes", _owner_with(_own_units_counted_as_borrowed)),
    "owner: every rank receives the whole vector": ("_owner_bytes", _owner_with(_receives_whole_vector)),
    "owner: gradients sent twice": ("_owner_bytes", _owner_with(_gradients_sent_twice)),
    "owner: resident of the largest owner": ("_owner_bytes", _owner_with(_resident_of_the_largest_owner)),
})

LAYOUT_MUTANTS.update({
    "owners shifted by one rank": (lo, "unit_owners", owners_shifted),
})


# (after the owner-broadcast mutants above are added to the dictionary)
@pytest.mark.parametrize("name", list(ACCOUNTING_MUTANTS))
def test_accounting_mutant_is_caught(name, monkeypatch):
    attr, val = ACCOUNTING_MUTANTS[name]
    monkeypatch.setattr(acc, attr, val)
    caught = first_failing(ACCOUNTING_PINS)
    assert caught is not None, f"no pin fails with the planted mistake: {name}"


def test_owner_rule_for_unequal_units_is_a_reading_not_a_pin(monkeypatch):
    """The pages show owner broadcast only on equal partitions, where taking
    a unit's owner from its start instead of its midpoint assigns the same
    ranks; so every pin accepts that rule too.  For unequal units the
    midpoint rule is a reading, and this records that no pin fixes it."""
    monkeypatch.setattr(lo, "unit_owners", owners_by_start)
    assert first_failing(ACCOUNTING_PINS + SCHEME_PINS) is None
    units = [1_050_677_248] + [218_112_000] * 32            # the Llama-3-8B shape's units
    assert owners_by_start(units, 8) != _unit_owners(units, 8)


def trajectory_variant(drop_last_rank=False, grads_of_step_before=False):
    """The sampled oracle's per-element trajectory with one planted mistake."""
    import synth

    def trajectory(p_idx, world, steps, dtype16, grad_sigma, lr, betas=(0.9, 0.999), eps=1e-8,
                   seed=0, outlier_permyriad=0, theta_sigma=0.02):
        p_idx = np.asarray(p_idx, dtype=np.int64)
        master = synth.theta0(seed, p_idx, theta_sigma)
        m = np.zeros(p_idx.shape, np.float32)
        v = np.zeros(p_idx.shape, np.float32)
        for t in range(1, steps + 1):
            gs = max(1, t - 1) if grads_of_step_before else t
            ranks = range(world - 1) if drop_last_rank and world > 1 else range(world)
            rows = [nm.widen16(synth.grad16(seed, r, gs, p_idx, grad_sigma, dtype16, outlier_permyriad),
                               dtype16) for r in ranks]
            g = nm.reduce_rank_order(rows)
            k = nm.adam_consts(lr, betas[0], betas[1], eps, t)
            master, m, v = nm.adam_update(master, m, v, g, k)
        return master, m, v, nm.cast16(master, dtype16)
    return trajectory


SCHEME_MUTANTS = {
    "ranks own each other's shards": (lo.Layout, "owned", owned_ranks_reversed),
    "step counter advances per call of Adam": (sc._Scheme, "_consts", consts_per_unit_clock),
    "sampled oracle drops the last rank": (sampled, "trajectory", trajectory_variant(drop_last_rank=True)),
    "sampled oracle reuses the previous step's gradients":
        (sampled, "trajectory", trajectory_variant(grads_of_step_before=True)),
}


@pytest.mark.parametrize("name", list(LAYOUT_MUTANTS))
def test_layout_mutant_is_caught(name, monkeypatch):
    obj, attr, val = LAYOUT_MUTANTS[name]
    monkeypatch.setattr(obj, attr, val)
    caught = first_failing(ACCOUNTING_PINS + SCHEME_PINS)
    assert caught is not None, f"no pin fails with the planted mistake: {name}"


@pytest.mark.parametrize("name", list(SCHEME_MUTANTS))
def test_scheme_mutant_is_caught(name, monkeypatch):
    obj, attr, val = SCHEME_MUTANTS[name]
    monkeypatch.setattr(obj, attr, val)
    caught = first_failing(SCHEME_PINS)
    assert caught is not None, f"no pin fails with the planted mistake: {name}"
