"""Pins of the oracle's accounting and layout against numbers printed on the pages."""
import os
import random
import shlex
from decimal import ROUND_HALF_UP, Decimal

import pytest

from oracle import accounting as acc
from oracle.layout import IndivisibleError, make_layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_accounting.txt")


def _units(tok):
    if tok == "-":
        return None
    if "x" in tok:
        k, size = tok.split("x")
        return [int(size)] * int(k)
    return [int(x) for x in tok.split(",")]


def load_pins():
    pins = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = shlex.split(line)
            pins.append(dict(id=tok[0], numel=None if tok[1] == "?" else int(tok[1]),
                             world=int(tok[2]),
                             stage=int(tok[3].rstrip("o")), owner=tok[3].endswith("o"),
                             units=_units(tok[4]),
                             pad=bool(int(tok[5])), gather_bytes=int(tok[6]), quantity=tok[7],
                             printed=Decimal(tok[8]), scale=Decimal(tok[9]), decimals=int(tok[10]),
                             source=" ".join(tok[11:])))
    return pins


def quantity(pin):
    lay = make_layout(pin["numel"], pin["world"], pin["stage"], pin["units"], pin["pad"],
                      owner_broadcast=pin["owner"])
    b = acc.bytes_per_rank(lay, gather_bytes=pin["gather_bytes"])
    q = pin["quantity"]
    if q == "resident":
        return Decimal(b.resident)
    if q == "peak":
        return Decimal(b.peak)
    if q == "opt_state":
        return Decimal(acc.optimizer_state_bytes(lay))
    if q == "res_per_param":
        return Decimal(b.resident) / Decimal(pin["numel"])
    if q == "peak_per_param":
        return Decimal(b.peak) / Decimal(pin["numel"])
    if q == "rs_elems":
        return Decimal(b.rs_elems)
    if q == "traffic_bytes_x_n_over_psi":
        return Decimal(b.traffic_bytes) * pin["world"] / ((pin["world"] - 1) * Decimal(pin["numel"]))
    if q == "peak_params_x_n_over_psi":
        held = Decimal(b.res_p16) / acc.BAND_BYTES["p16"] + Decimal(b.gathered) / pin["gather_bytes"]
        return held * pin["world"] / Decimal(pin["numel"])
    raise KeyError(q)


ALL_PINS = load_pins()
PINS = [p for p in ALL_PINS if p["numel"] is not None]
SOLVED_PINS = [p for p in ALL_PINS if p["numel"] is None]


def rounded(pin, value: Decimal) -> Decimal:
    q = Decimal(1).scaleb(-pin["decimals"])
    return (value / pin["scale"]).quantize(q, rounding=ROUND_HALF_UP)


@pytest.mark.parametrize("pin", PINS, ids=[p["id"] for p in PINS])
def test_page_printed_value(pin):
    assert rounded(pin, quantity(pin)) == pin["printed"].quantize(
        Decimal(1).scaleb(-pin["decimals"])), pin["source"]


def psi_interval(pin, value_of=None, hi=10 ** 13):
    """[a, b): the parameter counts at which the pin's rounded value equals
    the printed one.  The quantity never decreases as the count grows, so
    the counts form one interval; found by bisection."""
    value_of = value_of or (lambda psi: quantity(dict(pin, numel=psi)))
    want = pin["printed"].quantize(Decimal(1).scaleb(-pin["decimals"]))

    def first(pred):                     # smallest psi in [1, hi] with pred(psi), else hi
        a, b = 1, hi
        while a < b:
            mid = (a + b) // 2
            if pred(mid):
                b = mid
            else:
                a = mid + 1
        return a
    lo = first(lambda psi: rounded(pin, value_of(psi)) >= want)
    up = first(lambda psi: rounded(pin, value_of(psi)) > want)
    return lo, up


def solve_common_count(pins, value_of=None):
    """The counts at which every pin of one model holds: [lo, hi)."""
    lo, hi = 1, 10 ** 13
    for pin in pins:
        a, b = psi_interval(pin, value_of and (lambda psi, p=pin: value_of(p, psi)))
        lo, hi = max(lo, a), min(hi, b)
    return lo, hi


def test_one_parameter_count_reproduces_the_unprinted_model():
    # "Sharding the States.": Llama 3 70B's three per-device figures come from
    # one parameter count, about 70.5e9 (each figure alone fixes it only to a
    # band; the three bands must overlap)
    groups = {}
    for pin in SOLVED_PINS:
        groups.setdefault(pin["id"][0], []).append(pin)
    assert set(groups) == {"l"} and len(groups["l"]) == 3
    for pins in groups.values():
        lo, hi = solve_common_count(pins)
        assert lo < hi, [p["source"] for p in pins]
        assert 70.4e9 < lo < hi < 70.7e9
        for psi in (lo, (lo + hi) // 2, hi - 1):
            for pin in pins:
                assert rounded(pin, quantity(dict(pin, numel=psi))) == pin["printed"], (psi, pin["id"])


def test_sixteen_bytes_per_parameter():
    # "One Poem Suffices: ZeRO" s3.1: 2 + 2 + 3*4 = 16 bytes per parameter
    assert sum(acc.BAND_BYTES.values()) == 16
    assert acc.BAND_BYTES == {"p16": 2, "grad": 2, "master": 4, "m": 4, "v": 4}


@pytest.mark.parametrize("numel,world", [(8, 4), (65536, 4), (124439808, 8), (7_500_000_000, 64),
                                         (1_558_000_000, 16)])
def test_closed_forms(numel, world):
    # "ZeRO and FSDP" three-stage table: 16P, 4P + 12P/N, 2P + 14P/N, 16P/N (N | P)
    res = [acc.bytes_per_rank(make_layout(numel, world, s)).resident for s in range(4)]
    assert res == [16 * numel, 4 * numel + 12 * numel // world, 2 * numel + 14 * numel // world,
                   16 * numel // world]


@pytest.mark.parametrize("numel,world", [(8, 4), (65536, 4), (7_500_000_000, 64)])
def test_traffic_ratio_and_exact_forms(numel, world):
    # "ZeRO, annotated" s7 / "One Poem Suffices: ZeRO" 4.1.4: DP and stages 1-2 move
    # 2(N-1)/N * Psi, stage 3 3(N-1)/N * Psi; ratio exactly 1.5
    t = [acc.bytes_per_rank(make_layout(numel, world, s)).traffic_elems for s in range(4)]
    s = numel // world
    assert t[0] == t[1] == t[2] == 2 * (world - 1) * s
    assert t[3] == 3 * (world - 1) * s
    assert Decimal(t[3]) / Decimal(t[0]) == Decimal("1.5")
    # the 7.5B example's approximations 15.0e9 and 22.5e9 numbers per GPU
    if numel == 7_500_000_000:
        assert t[0] * world // (world - 1) == 15_000_000_000
        assert t[3] * world // (world - 1) == 22_500_000_000


def test_stage3_peak_is_resident_plus_gathered_unit():
    # "The four schemes": peak - resident is exactly the gathered copy
    lay = make_layout(65536, 4, 3, [16384] * 4)
    b = acc.bytes_per_rank(lay)
    assert b.peak - b.resident == 2 * 16384
    one = acc.bytes_per_rank(make_layout(65536, 4, 3))
    assert one.peak - one.resident == 2 * 65536
    for s in range(3):
        bs = acc.bytes_per_rank(make_layout(65536, 4, s))
        assert bs.peak == bs.resident


def test_prefetch_peak_two_live_units():
    lay = make_layout(10 + 20 + 30 + 5, 5, 3, [10, 20, 30, 5])
    b2 = acc.bytes_per_rank(lay, max_live=2)
    assert b2.gathered == 2 * (20 + 30)
    assert acc.bytes_per_rank(lay, max_live=1).gathered == 2 * 30


def test_padding_readings():
    # the prototype refuses an indivisible count; ZeroAdam pads with ceil(Psi/N)
    with pytest.raises(IndivisibleError):
        make_layout(19210, 4, 1)
    lay = make_layout(19210, 4, 1, pad=True)
    assert lay.shard_u == (4803,) and lay.padded_numel == 19212
    b = acc.bytes_per_rank(lay)
    assert b.res_p16 == 2 * 19210 and b.res_grad == 2 * 19210 and b.res_master == 4 * 4803
    with pytest.raises(IndivisibleError):
        make_layout(10, 4, 3, [5, 5])
    lay3 = make_layout(10, 4, 3, [5, 5], pad=True)
    assert lay3.shard_u == (2, 2) and lay3.padded_numel == 16


def test_layout_owned_ranges_tile_the_padded_vector():
    rnd = random.Random(7)
    for _ in range(200):
        world = rnd.randint(1, 9)
        units = [rnd.randint(1, 50) for _ in range(rnd.randint(1, 5))]
        numel = sum(units)
        for stage in (1, 2, 3):
            lay = make_layout(numel, world, stage, units, pad=True)
            seen = []
            for u in range(lay.n_units if stage == 3 else 1):
                for r in range(world):
                    off, n = lay.owned(r, u)
                    seen.extend(range(off, off + n))
            assert sorted(seen) == list(range(lay.padded_numel))
            par, ok = lay.padded_to_param(range(lay.padded_numel))
            assert sorted(par[ok].tolist()) == list(range(numel))
            assert int(ok.sum()) == numel


# ------------------------------------------------------- owner broadcast --
def test_owner_rule_gives_the_pages_contiguous_partitions():
    # "One Poem Suffices: ZeRO" s4.1.4: 64 devices, 192 blocks, 3 per device in
    # model order; "ZeRO, annotated" s7: GPU i owns shard i
    assert make_layout(192, 64, 3, [1] * 192, owner_broadcast=True).owners == \
        tuple(u // 3 for u in range(192))
    assert make_layout(8, 4, 3, [2] * 4, owner_broadcast=True).owners == (0, 1, 2, 3)


def test_pages_owner_map_and_explicit_maps():
    # the pages' partition written out: 3 consecutive blocks per device of 64
    from oracle.layout import pages_owners
    assert pages_owners(192, 64) == tuple(u // 3 for u in range(192))
    assert pages_owners(4, 4) == (0, 1, 2, 3)
    lay = make_layout(192, 64, 3, [1] * 192, owner_broadcast=True, owners=pages_owners(192, 64))
    assert lay.owners == make_layout(192, 64, 3, [1] * 192, owner_broadcast=True).owners
    with pytest.raises(ValueError):
        pages_owners(10, 4)
    for bad in ((0, 1, 2), (0, 1, 2, 4), (0, -1, 2, 3)):
        with pytest.raises(ValueError):
            make_layout(64, 4, 3, [16] * 4, owner_broadcast=True, owners=bad)
    with pytest.raises(ValueError):
        make_layout(64, 4, 3, [16] * 4, owners=(0, 1, 2, 3))


def test_owner_accounting_closed_forms_for_any_map():
    # any owner map: a rank keeps 16 B per parameter it owns, receives every
    # other parameter twice (forward and backward broadcasts), sends those
    # gradients once, and its peak adds the largest borrowed unit(s) live
    rnd = random.Random(12)
    for _ in range(200):
        world = rnd.randint(1, 9)
        units = [rnd.randint(1, 100) for _ in range(rnd.randint(1, 12))]
        owners = [rnd.randrange(world) for _ in units]
        numel = sum(units)
        lay = make_layout(numel, world, 3, units, owner_broadcast=True, owners=owners)
        for r in range(world):
            own = sum(n for n, o in zip(units, owners) if o == r)
            assert lay.own_numel(r) == own
            b = acc.bytes_per_rank(lay, rank=r)
            assert b.resident == 16 * own
            assert (b.rs_elems, b.ag_elems) == (numel - own, 2 * (numel - own))
            borrowed = [0 if o == r else n for n, o in zip(units, owners)]
            assert b.gathered == 2 * max(borrowed)
            b2 = acc.bytes_per_rank(lay, rank=r, max_live=2)
            pairs = [borrowed[i] + borrowed[i + 1] for i in range(len(units) - 1)] or borrowed
            assert b2.gathered == 2 * max(pairs)


def test_owner_peak_two_64ths_either_reading():
    # the 3 blocks a device broadcasts as one unit (max_live 1), or 192
    # single-block units with the 3 of a partition live at once: both 2/64
    for units, live in (([3000] * 64, 1), ([1000] * 192, 3)):
        b = acc.bytes_per_rank(make_layout(192000, 64, 3, units, owner_broadcast=True),
                               max_live=live)
        assert (b.res_p16 // 2 + b.gathered // 2) * 64 == 2 * 192000


@pytest.mark.parametrize("world,k", [(4, 1), (4, 3), (8, 4), (64, 3)])
def test_owner_balanced_equals_split_layout(world, k):
    # equal shares: the same bytes and the same 3(N-1)/N traffic as the
    # per-unit split (f3's claim); only the peak's gathered part differs
    size = 192                                           # divisible by every world here
    units = [size] * (k * world)
    own = acc.bytes_per_rank(make_layout(size * k * world, world, 3, units, owner_broadcast=True))
    split = acc.bytes_per_rank(make_layout(size * k * world, world, 3, units))
    assert own.resident == split.resident
    assert (own.rs_elems, own.ag_elems) == (split.rs_elems, split.ag_elems)
    assert own.gathered == 2 * size                      # one borrowed unit
    assert split.gathered == 2 * size                    # one unit, all N shards


def test_owner_accounting_per_rank_closed_forms():
    rnd = random.Random(11)
    for _ in range(200):
        world = rnd.randint(1, 9)
        units = [rnd.randint(1, 100) for _ in range(rnd.randint(1, 12))]
        numel = sum(units)
        lay = make_layout(numel, world, 3, units, owner_broadcast=True)
        assert sum(lay.own_numel(r) for r in range(world)) == numel
        assert all(lay.owners[i] <= lay.owners[i + 1] for i in range(len(units) - 1))
        per = [acc.bytes_per_rank(lay, rank=r) for r in range(world)]
        for r, b in enumerate(per):
            own = lay.own_numel(r)
            assert b.resident == 16 * own
            assert (b.rs_elems, b.ag_elems) == (numel - own, 2 * (numel - own))
            borrowed = [0 if o == r else n for n, o in zip(units, lay.owners)]
            assert b.gathered == 2 * max(borrowed)
        worst = acc.bytes_per_rank(lay)
        assert worst.peak == max(b.peak for b in per)
