"""The C-ABI library on a machine without a GPU: it loads, exports every
symbol its headers declare, and its host-only parts (layout, accounting,
argument checks, the ZeRO-3 state checks) agree with the oracle.  No call
here launches a kernel."""
import ctypes
import os
import random
import re

import pytest

import zero_sharded_mixed_reduce_amd as z
from oracle import accounting as acc
from oracle.layout import make_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(z.LIB_PATH)
    names = declared("zsmr.h")
    assert "zero_fused_step" in names and "zero_bytes_per_rank" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(z.SIGNATURES), "binding and header disagree"
    import synth.gpu as sg
    slib = ctypes.CDLL(sg.LIB_PATH)
    snames = declared("zsmr_synth.h")
    assert snames == ["zsmr_synth_fill16", "zsmr_synth_fill32"]
    for n in snames:
        assert hasattr(slib, n), n
    import ceiling
    clib = ctypes.CDLL(ceiling.LIB_PATH)
    cnames = declared("zsmr_ceiling.h")
    assert cnames == ["zsmr_ceiling_read", "zsmr_ceiling_set_balance", "zsmr_ceiling_write"]
    for n in cnames:
        assert hasattr(clib, n), n


def test_ceiling_argument_errors_return_before_any_launch():
    import ceiling
    lib = ceiling._lib()
    a16, a8 = 1 << 20, (1 << 20) + 8          # fake device addresses: never dereferenced
    assert lib.zsmr_ceiling_read(None, 16, 0, a16, None) == 1
    assert lib.zsmr_ceiling_read(a16, 16, 0, None, None) == 1
    assert lib.zsmr_ceiling_read(a16, -16, 0, a16, None) == 1
    assert lib.zsmr_ceiling_read(a16, 24, 0, a16, None) == 1
    assert lib.zsmr_ceiling_read(a16, 16, 3, a16, None) == 1
    assert lib.zsmr_ceiling_read(a8, 16, 0, a16, None) == 5
    assert lib.zsmr_ceiling_read(a16, 16, 1, a8, None) == 5
    assert lib.zsmr_ceiling_read(a16, 0, 1, a16, None) == 0
    assert lib.zsmr_ceiling_write(None, 16, 0, 0, None) == 1
    assert lib.zsmr_ceiling_write(a16, 8, 0, 0, None) == 1
    assert lib.zsmr_ceiling_write(a16, 16, 4, 0, None) == 1
    assert lib.zsmr_ceiling_write(a16, 16, -1, 0, None) == 1
    assert lib.zsmr_ceiling_set_balance(499) == 1 and lib.zsmr_ceiling_set_balance(2001) == 1
    assert lib.zsmr_ceiling_set_balance(1000) == 0 and lib.zsmr_ceiling_set_balance(1200) == 0
    assert lib.zsmr_ceiling_write(a8, 16, 1, 0, None) == 5
    assert lib.zsmr_ceiling_write(a16, 0, 0, 0, None) == 0
    assert lib.zsmr_ceiling_write(None, 0, 0, 0, None) == 0        # nothing to touch
    assert lib.zsmr_ceiling_read(None, 0, 0, None, None) == 0
    assert lib.zsmr_ceiling_read(None, 0, 5, None, None) == 1      # the shape is still checked


def test_phased_bound_is_read_time_plus_write_time():
    import ceiling
    # 7e9 bytes read at 7000 GB/s (1 ms) and 3e9 written at 6000 GB/s (0.5 ms)
    assert ceiling.phased_bound(7_000_000_000, 3_000_000_000, 7000.0, 6000.0) == pytest.approx(1.5)
    assert ceiling.phased_bound(0, 0, 1.0, 1.0) == 0


CONFIGS = [
    (65536, 4, st, [16384] * 4 if st == 3 else None) for st in range(4)
] + [
    (124_439_808, 8, 2, None), (1_558_000_000, 16, 1, None), (7_500_000_000, 64, 2, None),
    (8_030_261_248, 8, 3, [1_050_677_248] + [218_112_000] * 32),
]


def _cmp_bytes(ctx, lay, gb=2, ml=1):
    got = z.zero_bytes_per_rank(ctx, gb, ml)
    want = acc.bytes_per_rank(lay, gather_bytes=gb, max_live=ml)
    for k, v in got.items():
        assert v == getattr(want, k), k


@pytest.mark.parametrize("numel,world,stage,units", CONFIGS)
def test_layout_and_accounting_match_oracle(numel, world, stage, units):
    ctx = z.zero_init_shards(numel, world, stage, "bf16", units=units)
    lay = make_layout(numel, world, stage, units)
    info = ctx.info()
    assert info["padded_numel"] == lay.padded_numel and info["shard_numel"] == lay.shard_numel
    for u in range(lay.n_units if stage == 3 else 1):
        for r in range(world):
            off, ln, loc = z.zero_layout(ctx, r, u)
            assert (off, ln) == lay.owned(r, u)
            assert loc == (lay.local_offset(u) if stage == 3 else 0)
    _cmp_bytes(ctx, lay)
    _cmp_bytes(ctx, lay, gb=4, ml=2)


def test_random_layouts_match_oracle():
    rnd = random.Random(1234)
    for _ in range(300):
        world = rnd.randint(1, 70)
        units = [rnd.randint(1, 10 ** rnd.randint(1, 7)) for _ in range(rnd.randint(1, 6))]
        numel = sum(units)
        stage = rnd.randint(0, 3)
        ctx = z.zero_init_shards(numel, world, stage, "fp16", pad=True,
                                 units=units if stage == 3 else None)
        lay = make_layout(numel, world, stage, units if stage == 3 else None, pad=True)
        r = rnd.randrange(world)
        u = rnd.randrange(lay.n_units) if stage == 3 else 0
        assert z.zero_layout(ctx, r, u)[:2] == lay.owned(r, u)
        _cmp_bytes(ctx, lay, gb=rnd.choice([2, 4]), ml=rnd.randint(1, 3))


def test_page_pins_through_the_c_library():
    # the tiny model of "ZeRO, annotated" and the 7.5B/64 Figure-1 case
    tiny = [z.zero_bytes_per_rank(z.zero_init_shards(8, 4, s, "fp16"))["resident"] for s in range(4)]
    assert tiny == [128, 56, 44, 32]
    big = [z.zero_bytes_per_rank(z.zero_init_shards(7_500_000_000, 64, s, "bf16"))["resident"]
           for s in range(4)]
    assert big == [120_000_000_000, 31_406_250_000, 16_640_625_000, 1_875_000_000]
    assert z.zero_bytes_per_rank(z.zero_init_shards(8, 4, 1, "fp16"))["rs_elems"] == 6
    # zero_check: 57,636 bytes of optimizer state with ceil(19,210 / 4) = 4,803
    b = z.zero_bytes_per_rank(z.zero_init_shards(19210, 4, 1, "bf16", pad=True))
    assert b["res_master"] + b["res_m"] + b["res_v"] == 57636


def test_unprinted_count_pins_through_the_c_library():
    """"Sharding the States." Llama 3 70B on 64 devices: the parameter counts
    at which the C library's per-device bytes round to 295.4 / 156.5 / 17.6
    GB overlap, in the same interval the oracle finds."""
    from decimal import Decimal
    from tests import test_oracle_accounting as pa

    def c_value(pin, psi):
        ctx = z.zero_init_shards(psi, pin["world"], pin["stage"], "bf16", pad=pin["pad"])
        return Decimal(z.zero_bytes_per_rank(ctx, pin["gather_bytes"])["resident"])
    lo, hi = pa.solve_common_count(pa.SOLVED_PINS, c_value)
    assert lo < hi
    assert (lo, hi) == pa.solve_common_count(pa.SOLVED_PINS)


def test_init_errors():
    with pytest.raises(z.ZsmrError) as e:
        z.zero_init_shards(1001, 4, 2, "bf16")
    assert e.value.code == z.ZSMR_ERR_INDIVISIBLE
    with pytest.raises(z.ZsmrError) as e:
        z.zero_init_shards(10, 4, 3, "bf16", units=[5, 5])
    assert e.value.code == z.ZSMR_ERR_INDIVISIBLE
    for bad in [dict(numel=0, world=1, stage=0), dict(numel=8, world=0, stage=0),
                dict(numel=8, world=2, stage=5), dict(numel=8, world=2, stage=3, units=[4, 5])]:
        with pytest.raises(z.ZsmrError) as e:
            z.zero_init_shards(bad["numel"], bad["world"], bad["stage"], "bf16", units=bad.get("units"))
        assert e.value.code == z.ZSMR_ERR_ARG
    h = ctypes.c_void_p()
    assert z.load().zero_init_shards(ctypes.byref(h), 8, 2, 1, 3, 2, 0, None, 0) == z.ZSMR_ERR_DTYPE


def test_argument_errors_return_before_any_launch():
    ctx = z.zero_init_shards(64, 4, 2, "bf16")
    ok = 1 << 20                          # an aligned, never-dereferenced address
    with pytest.raises(z.ZsmrError) as e:     # rank out of range
        z.zero_fused_step(ctx, 4, 0, ok, 64, 0, ok, ok, ok, ok, 1, 1e-3, stream=0)
    assert e.value.code == z.ZSMR_ERR_ARG
    with pytest.raises(z.ZsmrError) as e:     # t < 1
        z.zero_fused_step(ctx, 0, 0, ok, 64, 0, ok, ok, ok, ok, 0, 1e-3, stream=0)
    assert e.value.code == z.ZSMR_ERR_ARG
    with pytest.raises(z.ZsmrError) as e:     # beta1 >= 1
        z.zero_fused_step(ctx, 0, 0, ok, 64, 0, ok, ok, ok, ok, 1, 1e-3, betas=(1.0, 0.999), stream=0)
    assert e.value.code == z.ZSMR_ERR_ARG
    with pytest.raises(z.ZsmrError) as e:     # rows overlap (stride < shard)
        z.zero_fused_step(ctx, 0, 0, ok, 8, 0, ok, ok, ok, ok, 1, 1e-3, stream=0)
    assert e.value.code == z.ZSMR_ERR_ARG
    with pytest.raises(z.ZsmrError) as e:     # odd address for a 16-bit row
        z.zero_fused_step(ctx, 0, 0, ok + 1, 64, 0, ok, ok, ok, ok, 1, 1e-3, stream=0)
    assert e.value.code == z.ZSMR_ERR_ALIGN
    with pytest.raises(z.ZsmrError) as e:     # fp32 master not 4-byte aligned
        z.zero_fused_step(ctx, 0, 0, ok, 64, 0, ok + 2, ok, ok, ok, 1, 1e-3, stream=0)
    assert e.value.code == z.ZSMR_ERR_ALIGN
    with pytest.raises(z.ZsmrError) as e:     # null g_out
        z.zero_reduce_shard(ctx, 0, 0, ok, 64, 0, True, 0, stream=0)
    assert e.value.code == z.ZSMR_ERR_ARG
    with pytest.raises(z.ZsmrError) as e:     # overlapping copy
        z.zero_gather_copy(ctx, 0, ok, ok + 8, 100, stream=0)
    assert e.value.code == z.ZSMR_ERR_ARG
    far = ok + (1 << 30)
    for args in ((ok, far, 100, 2, 99),          # blocks overlap (stride < n)
                 (ok, ok + 8, 10, 3, 100),        # source and destination spans overlap
                 (ok, far, 10, 65536, 100),       # more blocks than a grid holds
                 (ok, far, 10, 3, 1 << 62),       # the span overflows
                 (ok, far, -1, 3, 100),
                 (ok, far, 10, -1, 100),
                 (0, far, 10, 3, 100)):
        with pytest.raises(z.ZsmrError) as e:
            z.zero_gather_copy_blocks(ctx, 0, *args, stream=0)
        assert e.value.code == z.ZSMR_ERR_ARG, args
    with pytest.raises(z.ZsmrError) as e:         # odd address of a 16-bit block
        z.zero_gather_copy_blocks(ctx, 0, ok + 1, far, 10, 3, 100, stream=0)
    assert e.value.code == z.ZSMR_ERR_ALIGN
    z.zero_gather_copy_blocks(ctx, 0, ok, far, 0, 3, 100, stream=0)    # nothing to copy
    z.zero_gather_copy_blocks(ctx, 0, ok, far, 10, 0, 100, stream=0)
    z.zero_adam_step(ok, ok, ok, ok, 0, 1, 1e-3, stream=0)       # n = 0 is a no-op
    z.zero_gather_copy(ctx, 0, ok, ok, 0, stream=0)
    for rank in range(4):                                          # nothing was counted
        assert z.zero_counters(ctx, rank)["traffic_elems"] == 0


def test_stage3_state_errors_on_the_host():
    ctx = z.zero_init_shards(64, 4, 3, "bf16", units=[32, 32])
    with pytest.raises(z.ZsmrError) as e:
        z.zero_stage3_unit_release(ctx, 0)
    assert e.value.code == z.ZSMR_ERR_STATE
    with pytest.raises(z.ZsmrError) as e:
        z.zero_stage3_unit_release(ctx, 2)
    assert e.value.code == z.ZSMR_ERR_ARG
    with pytest.raises(z.ZsmrError) as e:     # a null shard pointer is refused before launching
        z.zero_stage3_unit_gather(ctx, 0, [1 << 20, 0, 1 << 20, 1 << 20], 1 << 21, stream=0)
    assert e.value.code == z.ZSMR_ERR_ARG
    U, slot = 1 << 21, 8 * 2                  # unit buffer; S_u = 8 bf16 elements per shard
    far = [1 << 24, (1 << 24) + 4096, (1 << 24) + 8192, (1 << 24) + 12288]
    for r, bad in ((1, U + 3 * slot), (0, U + 8), (3, U - 8)):
        ptrs = list(far)
        ptrs[r] = bad                         # overlaps the unit buffer, not at its own slot
        with pytest.raises(z.ZsmrError) as e:
            z.zero_stage3_unit_gather(ctx, 0, ptrs, U, stream=0)
        assert e.value.code == z.ZSMR_ERR_ARG
    assert z.zero_stage3_unit_state(ctx, 0) == (False, 0, 0)
    z.zero_stage3_set_max_live(ctx, 2)
    with pytest.raises(z.ZsmrError) as e:
        z.zero_stage3_set_max_live(ctx, 0)
    assert e.value.code == z.ZSMR_ERR_ARG
    nz = z.zero_init_shards(64, 4, 2, "bf16")
    with pytest.raises(z.ZsmrError) as e:     # not a stage-3 context
        z.zero_stage3_unit_release(nz, 0)
    assert e.value.code == z.ZSMR_ERR_ARG
    with pytest.raises(z.ZsmrError) as e:
        z.zsmr_set_launch_shape(-1, 4, 5, 32)
    with pytest.raises(z.ZsmrError) as e:
        z.zsmr_set_launch_shape(65, 4, 5, 32)
    with pytest.raises(z.ZsmrError) as e:
        z.zsmr_set_launch_shape(2, 4, 6, 32)
    with pytest.raises(z.ZsmrError) as e:
        z.zsmr_set_launch_shape(2, 4, 5, 0)
    with pytest.raises(z.ZsmrError) as e:
        z.zsmr_set_launch_shape(2, -1, 3, 16)
    with pytest.raises(z.ZsmrError) as e:
        z.zsmr_set_launch_shape(2, 65, 3, 16)
    assert e.value.code == z.ZSMR_ERR_ARG
    z.zsmr_set_launch_shape(2, 1, 3, 16)      # a grid-stride copy grid
    z.zsmr_set_launch_shape()                 # back to the defaults (one burst per wave)


def test_fused_range_bounds_are_checked_on_the_host():
    ctx = z.zero_init_shards(64, 4, 2, "bf16")
    ok = 1 << 20
    for begin, count in ((-1, 4), (0, -1), (10, 7), (17, 0), (0, 17)):
        with pytest.raises(z.ZsmrError) as e:
            z.zero_fused_step_range(ctx, 0, 0, begin, count, ok, 16, 0, ok, ok, ok, ok, 1, 1e-3,
                                    stream=0)
        assert e.value.code == z.ZSMR_ERR_ARG, (begin, count)
    for begin in (0, 7, 16):                   # empty ranges inside the piece are no-ops
        z.zero_fused_step_range(ctx, 1, 0, begin, 0, ok, 16, 0, ok, ok, ok, ok, 1, 1e-3, stream=0)
    assert z.zero_counters(ctx, 1)["traffic_elems"] == 0


def test_write_window_arguments():
    for bad in ((999, 100, 0, 0), (10_000_001, 100, 0, 0), (32000, 0, 0, 0), (32000, 4000, -1, 0),
                (32000, 30000, 2000, 0), (32000, 4000, 0, 4000), (32000, 4000, 0, -1),
                (0, -1, 0, 0), (0, 0, -1, 0), (0, 0, 0, -1)):
        with pytest.raises(z.ZsmrError) as e:
            z.zsmr_set_write_window(*bad)
        assert e.value.code == z.ZSMR_ERR_ARG, bad
    z.zsmr_set_write_window(0, 0, 0, 0)
    z.zsmr_set_write_window(1000, 2, 997, 1)
    z.zsmr_set_write_window()                 # back to the defaults


def test_context_world_is_kept():
    """The binding reads N once per context and keeps it for its row-size
    checks; it equals what the library reports, and a short gradient
    buffer is still refused before any call."""
    import torch
    for world in (1, 4, 64):
        ctx = z.zero_init_shards(64 * world, world, 2, "bf16")
        assert ctx.world == z.zero_layout_info(ctx)["world"] == world
        g = torch.empty(64 * world, dtype=torch.bfloat16)
        if world > 1:
            with pytest.raises(ValueError):
                z._rows_fit(ctx, g, 64 * world, 0, 64, "grads")   # rows of stride Psi overrun the buffer
        z._rows_fit(ctx, g, 64, 0, 64, "grads")                   # N rows of stride 64 fit


def test_xcd_balance_arguments():
    for bad in (0, 499, 2001, -1000):
        with pytest.raises(z.ZsmrError) as e:
            z.zsmr_set_xcd_balance(bad)
        assert e.value.code == z.ZSMR_ERR_ARG, bad
    for good in (500, 1000, 2000):
        z.zsmr_set_xcd_balance(good)
    z.zsmr_set_xcd_balance()                  # back to the default



def _owner_case(numel, world, units):
    ctx = z.zero_init_shards(numel, world, z.ZSMR_ZERO3_OWNER, "bf16", units=units)
    lay = make_layout(numel, world, 3, units, owner_broadcast=True)
    return ctx, lay


@pytest.mark.parametrize("numel,world,units", [
    (8, 4, [2] * 4), (192_000, 64, [3000] * 64), (192_000, 64, [1000] * 192),
    (8_030_261_248, 8, [1_050_677_248] + [218_112_000] * 32),
    (6000, 5, [1000, 7, 2993, 1500, 500]),
])
def test_owner_layout_and_accounting_match_oracle(numel, world, units):
    ctx, lay = _owner_case(numel, world, units)
    info = ctx.info()
    assert info["padded_numel"] == numel and info["shard_numel"] == lay.shard_numel
    assert info["max_unit_numel"] == max(units)
    for u in range(len(units)):
        assert z.zero_unit_owner(ctx, u) == lay.owners[u]
        for r in range(world):
            off, ln, loc = z.zero_layout(ctx, r, u)
            assert (off, ln) == lay.owned(r, u)
            assert loc == lay.local_offset(u)
    for gb, ml in ((2, 1), (4, 2), (2, 3)):
        for r in range(world):
            got = z.zero_bytes_of_rank(ctx, r, gb, ml)
            want = acc.bytes_per_rank(lay, gather_bytes=gb, max_live=ml, rank=r)
            for k, v in got.items():
                assert v == getattr(want, k), (r, k)
        worst = z.zero_bytes_per_rank(ctx, gb, ml)
        want = acc.bytes_per_rank(lay, gather_bytes=gb, max_live=ml)
        for k, v in worst.items():
            assert v == getattr(want, k), k


def test_owner_random_layouts_match_oracle():
    rnd = random.Random(99)
    for _ in range(300):
        world = rnd.randint(1, 40)
        units = [rnd.randint(1, 10 ** rnd.randint(1, 6)) for _ in range(rnd.randint(1, 20))]
        ctx, lay = _owner_case(sum(units), world, units)
        for u in range(len(units)):
            assert z.zero_unit_owner(ctx, u) == lay.owners[u]
        r = rnd.randrange(world)
        got = z.zero_bytes_of_rank(ctx, r, 2, rnd.randint(1, 3))
        assert got["resident"] == 16 * lay.own_numel(r)


def test_explicit_owner_maps_match_oracle():
    """Owners chosen by the caller (any map, not only the midpoint default):
    the library's index map and per-rank accounting equal the oracle's for
    the same map; the pages' own partition (k consecutive equal units per
    rank) is one of them."""
    from oracle.layout import pages_owners
    rnd = random.Random(5)
    cases = [(192_000, 64, [1000] * 192, list(pages_owners(192, 64))),
             (6000, 5, [1000, 7, 2993, 1500, 500], [3, 0, 3, 1, 4]),
             (8_030_261_248, 8, [1_050_677_248] + [218_112_000] * 32,
              [0] + [1] * 5 + [2] * 5 + [3] * 5 + [4] * 5 + [5] * 4 + [6] * 4 + [7] * 4)]
    for _ in range(200):
        world = rnd.randint(1, 12)
        units = [rnd.randint(1, 10 ** rnd.randint(1, 5)) for _ in range(rnd.randint(1, 15))]
        cases.append((sum(units), world, units, [rnd.randrange(world) for _ in units]))
    for numel, world, units, owners in cases:
        ctx = z.zero_init_shards(numel, world, z.ZSMR_ZERO3_OWNER, "bf16", units=units)
        z.zero_set_unit_owners(ctx, owners)
        lay = make_layout(numel, world, 3, units, owner_broadcast=True, owners=owners)
        assert ctx.info()["shard_numel"] == lay.shard_numel
        for u in range(len(units)):
            assert z.zero_unit_owner(ctx, u) == owners[u] == lay.owners[u]
            for r in range(world):
                off, ln, loc = z.zero_layout(ctx, r, u)
                assert (off, ln) == lay.owned(r, u)
                if ln:
                    assert loc == lay.local_offset(u)
        for ml in (1, 2):
            for r in range(world):
                got = z.zero_bytes_of_rank(ctx, r, 2, ml)
                want = acc.bytes_per_rank(lay, max_live=ml, rank=r)
                assert got == {k: getattr(want, k) for k in got}, (owners, r)
            worst = z.zero_bytes_per_rank(ctx, 2, ml)
            want = acc.bytes_per_rank(lay, max_live=ml)
            assert worst == {k: getattr(want, k) for k in worst}


def test_owner_map_errors():
    ctx, _ = _owner_case(64, 4, [16] * 4)
    for bad in ([0, 1, 2], [0, 1, 2, 4], [0, -1, 2, 3]):
        with pytest.raises(z.ZsmrError) as e:
            z.zero_set_unit_owners(ctx, bad)
        assert e.value.code == z.ZSMR_ERR_ARG
    split = z.zero_init_shards(64, 4, 3, "bf16", units=[32, 32])
    with pytest.raises(z.ZsmrError) as e:
        z.zero_set_unit_owners(split, [0, 1])
    assert e.value.code == z.ZSMR_ERR_ARG
    # a fresh context takes any map, and may be given another before its first use
    # (a map is refused once a call has counted something: the host driver's check)
    z.zero_set_unit_owners(ctx, [0, 0, 1, 1])
    z.zero_set_unit_owners(ctx, [3, 2, 1, 0])
    assert [z.zero_unit_owner(ctx, u) for u in range(4)] == [3, 2, 1, 0]


def test_integer_arrays_that_do_not_fit_their_c_type_are_refused():
    """Unit sizes (int64) and owners (int32) are checked before the call:
    ctypes would store 2**32 + 1 in an int32 array as 1, a valid owner."""
    ctx, _ = _owner_case(64, 4, [16] * 4)
    with pytest.raises(ValueError, match="owners"):
        z.zero_set_unit_owners(ctx, [0, 1, 2, (1 << 32) + 1])
    assert [z.zero_unit_owner(ctx, u) for u in range(4)] == [0, 1, 2, 3]   # unchanged
    with pytest.raises(ValueError, match="units"):
        z.zero_init_shards(64, 4, 3, "bf16", units=[(1 << 64) + 32, 32])


def test_stage3_gather_refuses_a_short_pointer_list():
    """The library reads N shard pointers at stage 3: the binding refuses a
    shorter list before any call."""
    ctx = z.zero_init_shards(64, 4, 3, "bf16", units=[32, 32])
    with pytest.raises(ValueError, match="shard pointers"):
        z.zero_stage3_unit_gather(ctx, 0, [1 << 20, 1 << 21], 1 << 22, stream=0)
    own, _ = _owner_case(64, 4, [16] * 4)
    with pytest.raises(ValueError, match="shard pointers"):
        z.zero_stage3_unit_gather(own, 0, [], 1 << 22, stream=0)


def test_owner_argument_errors():
    ctx, _ = _owner_case(64, 4, [16] * 4)
    with pytest.raises(z.ZsmrError) as e:     # a null owner copy is refused before launching
        z.zero_stage3_unit_gather(ctx, 0, [0], 1 << 21, stream=0)
    assert e.value.code == z.ZSMR_ERR_ARG
    with pytest.raises(z.ZsmrError) as e:     # owner copy and unit buffer overlap
        z.zero_stage3_unit_gather(ctx, 0, [1 << 20], (1 << 20) + 8, stream=0)
    assert e.value.code == z.ZSMR_ERR_ARG
    with pytest.raises(z.ZsmrError) as e:
        z.zero_unit_owner(ctx, 4)
    assert e.value.code == z.ZSMR_ERR_ARG
    split = z.zero_init_shards(64, 4, 3, "bf16", units=[32, 32])
    with pytest.raises(z.ZsmrError) as e:     # no owners in the split layout
        z.zero_unit_owner(split, 0)
    assert e.value.code == z.ZSMR_ERR_ARG
    with pytest.raises(z.ZsmrError) as e:
        z.zero_bytes_of_rank(ctx, 4)
    assert e.value.code == z.ZSMR_ERR_ARG
    ok = 1 << 20                              # a non-owner's fused call is an empty no-op
    z.zero_fused_step(ctx, 1, 0, ok, 16, 0, ok, ok, ok, ok, 1, 1e-3, stream=0)
    assert z.zero_counters(ctx, 0)["traffic_elems"] == 0
    assert z.zero_stage3_unit_state(ctx, 0) == (False, 0, 0)


def test_a_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library every entry point raises."""
    import ceiling
    import synth.gpu as sg
    gone = str(tmp_path / "libgone.so")
    monkeypatch.setattr(z, "LIB_PATH", gone)
    monkeypatch.setattr(z, "_LIB", None)
    with pytest.raises(ImportError):
        z.load()
    with pytest.raises(ImportError):
        z.zero_init_shards(64, 4, 2, "bf16")
    monkeypatch.setattr(sg, "LIB_PATH", gone)
    monkeypatch.setattr(sg, "_LIB", None)
    with pytest.raises(ImportError):
        sg.fill32(1 << 20, 4, 0, 4, 0, 0, 0, 1, 1.0, stream=0)
    monkeypatch.setattr(ceiling, "LIB_PATH", gone)
    monkeypatch.setattr(ceiling, "_LIB", None)
    with pytest.raises(ImportError):
        ceiling.write(1 << 20, 16, 0, 0, stream=0)


def test_host_tensors_are_refused_before_any_call():
    """A CPU tensor's address must never reach a kernel as a device address."""
    import torch
    import ceiling
    import synth.gpu as sg
    ctx = z.zero_init_shards(64, 4, 2, "bf16")
    h16 = torch.zeros(64, dtype=torch.bfloat16)
    h32 = torch.zeros(64, dtype=torch.float32)
    with pytest.raises(ValueError):
        z.zero_gather_copy(ctx, 0, h16, 1 << 20, 10, stream=0)
    with pytest.raises(ValueError):
        z.zero_fused_step(ctx, 0, 0, 1 << 20, 64, 0, h32, 1 << 21, 1 << 22, 1 << 23, 1, 1e-3, stream=0)
    with pytest.raises(ValueError):
        z.zero_init_state(ctx, 0, 0, h32, h32, h32, h32, h16, stream=0)
    with pytest.raises(ValueError):
        sg.fill16(h16, 1, 64, 64, 0, 64, 0, 0, 0, 1, 1.0, "bf16", stream=0)
    with pytest.raises(ValueError):
        ceiling.write(h32, 16, 0, 0, stream=0)
    for rank in range(4):
        assert z.zero_counters(ctx, rank)["traffic_elems"] == 0


class _FakeDeviceTensor:
    """Stands in for a device tensor of `nbytes` bytes at a never-dereferenced
    address (the binding's size checks run before any library call)."""

    def __init__(self, elems, elem_bytes=2, contiguous=True):
        import types
        self.device = types.SimpleNamespace(type="cuda")
        self._n, self._b, self._c = elems, elem_bytes, contiguous

    def numel(self):
        return self._n

    def element_size(self):
        return self._b

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return 1 << 20


def test_undersized_or_strided_tensors_are_refused_before_any_call():
    F = _FakeDeviceTensor
    ctx = z.zero_init_shards(64, 4, 2, "bf16")                  # S = 16 per rank
    with pytest.raises(ValueError, match="dst"):
        z.zero_gather_copy(ctx, 0, F(100), F(99), 100, stream=0)
    with pytest.raises(ValueError, match="not contiguous"):
        z.zero_gather_copy(ctx, 0, F(100, contiguous=False), F(100), 100, stream=0)
    with pytest.raises(ValueError, match="src"):
        z.zero_gather_copy_blocks(ctx, 0, F(3 * 50 + 9), F(1000), 10, 4, 50, stream=0)
    with pytest.raises(ValueError, match="grads"):                # rows 0..3 of stride 16 from base 16
        z.zero_fused_step(ctx, 1, 0, F(16 + 3 * 16 + 15), 16, 16, F(16, 4), F(16, 4), F(16, 4),
                          F(16), 1, 1e-3, stream=0)
    with pytest.raises(ValueError, match="master"):
        z.zero_fused_step(ctx, 1, 0, F(16 + 3 * 16 + 16), 16, 16, F(15, 4), F(16, 4), F(16, 4),
                          F(16), 1, 1e-3, stream=0)
    with pytest.raises(ValueError, match="p16_dst"):               # an fp32 master where bytes count
        z.zero_gather_cast(ctx, 0, 0, F(16, 4), F(8, 2), stream=0)
    with pytest.raises(ValueError, match="g_out"):
        z.zero_reduce_shard(ctx, 0, 0, F(64), 16, 0, True, F(15, 4), stream=0)
    with pytest.raises(ValueError, match="p16_dst"):               # a range reaching element 16
        z.zero_fused_step_range(ctx, 0, 0, 10, 6, F(64), 16, 0, F(16, 4), F(16, 4), F(16, 4),
                                F(15), 1, 1e-3, stream=0)
    s3 = z.zero_init_shards(64, 4, 3, "bf16", units=[32, 32])      # S_u = 8
    with pytest.raises(ValueError, match="unit_buf"):
        z.zero_stage3_unit_gather(s3, 1, [F(8)] * 4, F(31), stream=0)
    with pytest.raises(ValueError, match="shard 2"):
        z.zero_stage3_unit_gather(s3, 1, [F(8), F(8), F(7), F(8)], F(32), stream=0)
    for c in (ctx, s3):
        for rank in range(4):
            assert z.zero_counters(c, rank)["traffic_elems"] == 0
    assert z.zero_stage3_unit_state(s3, 1) == (False, 0, 0)


def test_integers_that_do_not_fit_their_c_type_are_refused():
    """ctypes would pass 2**32 + 4 as an int32_t 4: the bindings refuse it."""
    import ceiling
    import synth.gpu as sg
    with pytest.raises(ValueError, match="argument 2"):
        z.zero_init_shards(64, (1 << 32) + 4, 2, "bf16")
    with pytest.raises(ValueError, match="argument 1"):
        z.zero_init_shards(1 << 64, 4, 2, "bf16")
    ctx = z.zero_init_shards(64, 4, 2, "bf16")
    with pytest.raises(ValueError, match="argument 1"):
        z.zero_layout(ctx, (1 << 32) + 1, 0)
    with pytest.raises(ValueError, match="argument 10"):           # t
        z.zero_fused_step(ctx, 0, 0, 1 << 20, 64, 0, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                          (1 << 32) + 1, 1e-3, stream=0)
    with pytest.raises(ValueError, match="argument 5"):            # count of blocks
        z.zero_gather_copy_blocks(ctx, 0, 1 << 20, 1 << 40, 10, (1 << 32) + 2, 100, stream=0)
    with pytest.raises(ValueError, match="argument 4"):            # seed
        sg.fill32(1 << 20, 4, 0, 4, 1 << 32, 0, 0, 1, 1.0, stream=0)
    with pytest.raises(ValueError, match="argument 1"):
        ceiling.read(1 << 20, -(1 << 63) - 1, 0, 1 << 21, stream=0)
    for rank in range(4):
        assert z.zero_counters(ctx, rank)["traffic_elems"] == 0


def test_size_limits_of_a_context():
    """Sizes past the documented limits are refused before anything is
    allocated; at the limits every byte and traffic figure is exact."""
    MAX_NUMEL, MAX_WORLD, MAX_UNITS = 1 << 56, 1 << 20, 1 << 20
    for numel, world in ((MAX_NUMEL + 1, 4), ((1 << 63) - 1, 3), (8, MAX_WORLD + 1)):
        for stage in range(5):
            with pytest.raises(z.ZsmrError) as e:
                z.zero_init_shards(numel, world, stage, "bf16", pad=True)
            assert e.value.code == z.ZSMR_ERR_ARG
    h = ctypes.c_void_p()
    arr = (ctypes.c_int64 * 1)(8)
    assert z.load().zero_init_shards(ctypes.byref(h), 8, 1, 3, 2, 2, 0, arr, MAX_UNITS + 1) \
        == z.ZSMR_ERR_ARG and not h.value
    ctx = z.zero_init_shards(MAX_NUMEL, 64, 3, "bf16")
    b = z.zero_bytes_per_rank(ctx, gather_bytes=8, max_live=2)
    S = MAX_NUMEL // 64
    assert b["resident"] == 16 * S and b["gathered"] == 8 * MAX_NUMEL
    assert b["traffic_bytes"] == 2 * 3 * 63 * S
    with pytest.raises(z.ZsmrError) as e:
        z.zero_bytes_per_rank(ctx, gather_bytes=9)
    assert e.value.code == z.ZSMR_ERR_ARG


def test_peak_over_every_window_length_matches_oracle():
    """The gathered peak with max_live units live at once, for every
    max_live from 1 to past the unit count, split (stage 3) and owner
    (stage 4) layouts on random units and owner maps: the library equals the
    oracle's window-by-window sums."""
    rnd = random.Random(17)
    for _ in range(60):
        world = rnd.randint(1, 9)
        units = [world * rnd.randint(1, 10 ** rnd.randint(1, 4)) for _ in range(rnd.randint(1, 12))]
        numel = sum(units)
        split = z.zero_init_shards(numel, world, 3, "bf16", units=units)
        lay3 = make_layout(numel, world, 3, units)
        owners = [rnd.randrange(world) for _ in units]
        own = z.zero_init_shards(numel, world, z.ZSMR_ZERO3_OWNER, "bf16", units=units)
        z.zero_set_unit_owners(own, owners)
        lay4 = make_layout(numel, world, 3, units, owner_broadcast=True, owners=owners)
        for ml in range(1, len(units) + 3):
            got = z.zero_bytes_per_rank(split, 2, ml)
            want = acc.bytes_per_rank(lay3, max_live=ml)
            assert got == {k: getattr(want, k) for k in got}, (units, ml)
            for r in range(world):
                got = z.zero_bytes_of_rank(own, r, 4, ml)
                want = acc.bytes_per_rank(lay4, gather_bytes=4, max_live=ml, rank=r)
                assert got == {k: getattr(want, k) for k in got}, (units, owners, r, ml)


def test_peak_of_many_units_is_one_pass():
    """2^20 units (the most a context takes) with half of them live at once:
    the accounting is one pass over the units, not one per window."""
    import time
    n_units = 1 << 20
    units = [1 + (u % 7) for u in range(n_units)]
    ctx = z.zero_init_shards(sum(units), 2, z.ZSMR_ZERO3_OWNER, "bf16", units=units)
    t0 = time.perf_counter()
    b = z.zero_bytes_per_rank(ctx, 2, n_units // 2)
    assert time.perf_counter() - t0 < 5.0
    assert b["gathered"] > 0
