"""Pins of the oracle's scheme simulation: invariants the pages state (all
schemes compute the same model; ZeRO-2 is ZeRO-1 with one flag; ZeRO-3 must
gather twice per unit per step) and the accounting they must reproduce."""
import numpy as np
import pytest

import synth
from oracle import accounting as acc
from oracle import numerics as nm
from oracle import sampled
from oracle import schemes as sc
from oracle.layout import IndivisibleError, make_layout


def grads_fn(numel, world, dtype, sigma, seed=0, outlier=0):
    p = np.arange(numel)

    def f(t):
        return [synth.grad16(seed, r, t, p, sigma, dtype, outlier) for r in range(world)]
    return f


def run_all(numel, world, dtype, sigma, steps, lr, units=None, pad=False):
    theta = synth.theta0(0, np.arange(numel))
    g = grads_fn(numel, world, dtype, sigma)
    out = {}
    for stage in range(4):
        u = units if stage == 3 else None
        out[stage] = sc.run(stage, numel, world, theta, g, steps, dtype, lr, units=u, pad=pad)
    return out


def bits(x):
    return np.ascontiguousarray(x).view(np.uint32)


@pytest.mark.parametrize("numel,world,dtype,sigma,units", [
    (65536, 4, "fp16", 1e-2, [16384] * 4),          # the 65,536 / N = 4 / fp16 workload
    (4096, 8, "bf16", 1e-3, [1024, 512, 2048, 512]),
])
def test_all_schemes_bit_identical(numel, world, dtype, sigma, units):
    res = run_all(numel, world, dtype, sigma, steps=5, lr=1e-2, units=units)
    ref = res[0]
    for stage in (1, 2, 3):
        s = res[stage]
        assert np.array_equal(bits(s.full_master()), bits(ref.full_master()))
        assert np.array_equal(bits(s.full_m()), bits(ref.full_m()))
        assert np.array_equal(bits(s.full_v()), bits(ref.full_v()))
        assert np.array_equal(s.working_copy(), ref.working_copy())
    # every rank's working copy is the same bits; it is the cast of the master
    for r in range(world):
        assert np.array_equal(res[1].working_copy(r), res[1].working_copy(0))
    assert np.array_equal(ref.working_copy(), nm.cast16(ref.full_master(), dtype))
    # and the update actually moved every element
    assert np.all(ref.full_master() != synth.theta0(0, np.arange(numel)))


def test_zero2_is_zero1():
    res = run_all(8192, 4, "bf16", 1e-3, steps=3, lr=1e-3)
    a, b = res[1], res[2]
    for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v)):
        for r in range(4):
            assert np.array_equal(bits(x[r]), bits(y[r]))
    assert np.array_equal(a.p16[0], b.p16[0])
    la, lb = make_layout(8192, 4, 1), make_layout(8192, 4, 2)
    assert acc.bytes_per_rank(la).res_grad == 4 * acc.bytes_per_rank(lb).res_grad


def test_world_of_one_is_plain_adam_on_the_gradient():
    numel = 3000
    theta = synth.theta0(0, np.arange(numel))
    g = grads_fn(numel, 1, "bf16", 1e-3)
    s = sc.run(2, numel, 1, theta, g, 4, "bf16", 1e-3)
    master, m, v = theta.copy(), np.zeros(numel, np.float32), np.zeros(numel, np.float32)
    for t in range(1, 5):
        k = nm.adam_consts(1e-3, 0.9, 0.999, 1e-8, t)
        master, m, v = nm.adam_update(master, m, v, nm.widen16(g(t)[0], "bf16"), k)
    assert np.array_equal(bits(s.full_master()), bits(master))


def test_zero_gradients_leave_everything_unchanged():
    numel, world = 2048, 4
    theta = synth.theta0(0, np.arange(numel))
    zero = lambda t: [np.zeros(numel, np.uint16) for _ in range(world)]
    for stage in range(4):
        s = sc.run(stage, numel, world, theta, zero, 3, "bf16", 1e-2,
                   units=[1024, 1024] if stage == 3 else None)
        assert np.array_equal(bits(s.full_master()), bits(theta))
        assert not s.full_m().any() and not s.full_v().any()


@pytest.mark.parametrize("stage", [1, 2, 3])
def test_padding_tail_stays_zero(stage):
    numel, world = 1001, 4
    units = [500, 501] if stage == 3 else None
    theta = synth.theta0(0, np.arange(numel))
    g = grads_fn(numel, world, "bf16", 1e-3)
    with pytest.raises(IndivisibleError):
        sc.run(stage, numel, world, theta, g, 1, "bf16", 1e-3, units=units)
    s = sc.run(stage, numel, world, theta, g, 3, "bf16", 1e-3, units=units, pad=True)
    lay = s.lay
    par, ok = lay.padded_to_param(np.arange(lay.padded_numel))
    if stage == 3:
        padded = s._padded(s.master)
        padded16 = s._padded(s.p16)
        padded_mv = (s._padded(s.m), s._padded(s.v))
    else:
        padded = np.concatenate(s.master)
        padded16 = s.p16[0]
        padded_mv = (np.concatenate(s.m), np.concatenate(s.v))
    assert (~ok).sum() > 0
    assert not padded[~ok].any() and not padded16[~ok].any()
    assert not padded_mv[0][~ok].any() and not padded_mv[1][~ok].any()
    dp = sc.run(0, numel, world, theta, g, 3, "bf16", 1e-3)
    assert np.array_equal(bits(s.full_master()), bits(dp.full_master()))


def test_fp32_gather_then_cast_equals_16bit_gather():
    # the prototype all-gathers fp32 masters and casts after; the cast is elementwise
    rng = np.random.default_rng(1)
    shards = [rng.normal(0, 0.02, 1000).astype(np.float32) for _ in range(4)]
    for dt in ("bf16", "fp16"):
        a = nm.cast16(np.concatenate(shards), dt)
        b = np.concatenate([nm.cast16(s, dt) for s in shards])
        assert np.array_equal(a, b)


def test_sampled_trajectory_matches_full_run():
    numel, world, T = 5000, 8, 4
    res = sc.run(2, numel, world, synth.theta0(0, np.arange(numel)),
                 grads_fn(numel, world, "bf16", 1e-3, outlier=100), T, "bf16", 1e-4)
    idx = np.array([0, 1, 7, 624, 625, 4999, 2500])
    m, mm, vv, p16 = sampled.trajectory(idx, world, T, "bf16", 1e-3, 1e-4, outlier_permyriad=100)
    assert np.array_equal(bits(m), bits(res.full_master()[idx]))
    assert np.array_equal(bits(mm), bits(res.full_m()[idx]))
    assert np.array_equal(bits(vv), bits(res.full_v()[idx]))
    assert np.array_equal(p16, res.working_copy()[idx])


# ------------------------------------------------------- ZeRO-3 schedule -----

def schedule_matches_accounting(s: sc.ZeRO3, steps: int) -> bool:
    """What a correct ZeRO-3 run must show after ``steps`` steps."""
    lay = s.lay
    b = acc.bytes_per_rank(lay)
    sch = s.schedule
    return (all(g == 2 * steps for g in sch.gathers)
            and all(r == 2 * steps for r in sch.releases)
            and not sch.live
            and all(x == steps * b.ag_elems for x in s.ag_elems)
            and all(x == steps * b.rs_elems for x in s.rs_elems)
            and sch.peak_live_bytes == b.gathered
            and acc.bytes_per_rank(lay).resident + sch.peak_live_bytes == b.peak)


@pytest.mark.parametrize("units", [[65536], [16384] * 4, [5000, 20000, 40536]])
def test_stage3_gathers_twice_and_counts_traffic(units):
    numel, world, T = 65536, 4, 3
    seen = []

    def use(phase, u, buf):
        seen.append((phase, u))
        lay = s.lay
        q, w = lay.unit_pstart[u], world * lay.shard_u[u]
        assert np.array_equal(buf, s._padded(s.p16)[q:q + w])
    theta = synth.theta0(0, np.arange(numel))
    lay = make_layout(numel, world, 3, units)
    s = sc.ZeRO3(lay, theta, "fp16", 1e-2, use=use)
    g = grads_fn(numel, world, "fp16", 1e-2)
    for t in range(1, T + 1):
        s.step(g(t))
    assert schedule_matches_accounting(s, T)
    U = len(units)
    order = [("forward", u) for u in range(U)] + [("backward", u) for u in reversed(range(U))]
    assert seen == order * T
    b = acc.bytes_per_rank(lay)
    assert b.traffic_elems == 3 * (world - 1) * lay.shard_numel


class _GatherOnce(sc.ZeRO3):
    """A planted mistake: gather each unit once and keep it through backward."""

    def step(self, grads16):
        self.t += 1
        lay, w = self.lay, self.lay.world
        rows = self._rows(grads16)
        k = self._consts()
        for u in range(lay.n_units):
            self.gather(u)
        for u in reversed(range(lay.n_units)):
            for r in range(w):
                off, n = lay.owned(r, u)
                gr = nm.reduce_rank_order([row[off:off + n] for row in rows])
                self.rs_elems[r] += (w - 1) * n
                self.master[r][u], self.m[r][u], self.v[r][u] = nm.adam_update(
                    self.master[r][u], self.m[r][u], self.v[r][u], gr, k)
                self.p16[r][u] = nm.cast16(self.master[r][u], self.dtype)
            self.release(u)
        for r in range(w):
            self.ag_elems[r] = self.schedule.ag_elems


def test_gather_once_mistake_is_caught():
    numel, world, T = 4096, 4, 2
    theta = synth.theta0(0, np.arange(numel))
    g = grads_fn(numel, world, "bf16", 1e-3)
    # one unit: the schedule allows it, the counters expose it (2P traffic, not 3P)
    s = _GatherOnce(make_layout(numel, world, 3), theta, "bf16", 1e-3, max_live=1)
    for t in range(1, T + 1):
        s.step(g(t))
    assert not schedule_matches_accounting(s, T)
    assert s.schedule.ag_elems == T * (world - 1) * s.lay.shard_numel
    # the same arithmetic result, which is why the mistake hides ("right loss, wrong numbers")
    good = sc.run(3, numel, world, theta, g, T, "bf16", 1e-3)
    assert np.array_equal(bits(s.full_master()), bits(good.full_master()))
    # several units with one live at a time: the state machine refuses it outright
    s2 = _GatherOnce(make_layout(numel, world, 3, [2048, 2048]), theta, "bf16", 1e-3)
    with pytest.raises(sc.ScheduleError):
        s2.step(g(1))


def test_schedule_errors():
    lay = make_layout(64, 4, 3, [32, 32])
    sch = sc.Stage3Schedule(lay)
    with pytest.raises(sc.ScheduleError):
        sch.release(0)
    sch.gather(0)
    with pytest.raises(sc.ScheduleError):
        sch.gather(0)
    with pytest.raises(sc.ScheduleError):
        sch.gather(1)                       # max_live = 1
    sch.release(0)
    pre = sc.Stage3Schedule(lay, max_live=2)
    pre.gather(0)
    pre.gather(1)
    assert pre.peak_live_bytes == acc.bytes_per_rank(lay, max_live=2).gathered


# ------------------------------------------------------- owner broadcast --
@pytest.mark.parametrize("numel,world,units", [
    (8, 4, [2, 2, 2, 2]),                          # the pages' tiny model, GPU i owns layer i
    (65536, 4, [16384] * 4),
    (6000, 5, [1000, 7, 2993, 1500, 500]),         # uneven units: rank 1 owns none
    (4096, 3, [4096]),                             # one unit: rank 1 owns everything
    (777, 1, [300, 477]),                          # a world of one
])
def test_owner_broadcast_computes_the_same_model(numel, world, units):
    # "One Poem Suffices: ZeRO" s4.1.4 / "ZeRO, annotated" s7: the owner
    # layout changes who stores and sends what, never the arithmetic
    theta = synth.theta0(0, np.arange(numel))
    g = grads_fn(numel, world, "bf16", 1e-2)
    own = sc.run(3, numel, world, theta, g, 3, "bf16", 1e-3, units=units, owner_broadcast=True)
    dp = sc.run(0, numel, world, theta, g, 3, "bf16", 1e-3)
    for a, b in ((own.full_master(), dp.full_master()), (own.full_m(), dp.full_m()),
                 (own.full_v(), dp.full_v())):
        assert np.array_equal(bits(a), bits(b))
    assert np.array_equal(own.working_copy(), dp.working_copy())


@pytest.mark.parametrize("owners", [[3, 0, 3, 1, 4], [0, 0, 0, 0, 0], [4, 3, 2, 1, 0]])
def test_owner_broadcast_with_any_owner_map_computes_the_same_model(owners):
    # who owns a unit changes who stores and sends it, never the arithmetic
    numel, world, units = 6000, 5, [1000, 7, 2993, 1500, 500]
    theta = synth.theta0(0, np.arange(numel))
    g = grads_fn(numel, world, "bf16", 1e-2)
    own = sc.run(3, numel, world, theta, g, 2, "bf16", 1e-3, units=units, owner_broadcast=True,
                 owners=owners)
    dp = sc.run(0, numel, world, theta, g, 2, "bf16", 1e-3)
    assert np.array_equal(bits(own.full_master()), bits(dp.full_master()))
    assert np.array_equal(own.working_copy(), dp.working_copy())
    for r in range(world):
        b = acc.bytes_per_rank(own.lay, rank=r)
        assert (own.rs_elems[r], own.ag_elems[r]) == (2 * b.rs_elems, 2 * b.ag_elems)


def test_owner_broadcast_schedule_and_counters():
    numel, world, T = 6000, 5, 3
    units = [1000, 7, 2993, 1500, 500]
    lay = make_layout(numel, world, 3, units, owner_broadcast=True)
    seen = []

    def use(phase, u, buf):
        seen.append((phase, u))
        p, n = lay.unit_start[u], lay.units[u]
        assert np.array_equal(buf, s.working_copy()[p:p + n])     # the owner's copy
    theta = synth.theta0(0, np.arange(numel))
    s = sc.ZeRO3Owner(lay, theta, "bf16", 1e-3, use=use)
    g = grads_fn(numel, world, "bf16", 1e-3)
    for t in range(1, T + 1):
        s.step(g(t))
    U = len(units)
    order = [("forward", u) for u in range(U)] + [("backward", u) for u in reversed(range(U))]
    assert seen == order * T
    assert s.schedule.gathers == [2 * T] * U == s.schedule.releases
    for r in range(world):
        b = acc.bytes_per_rank(lay, rank=r)
        assert (s.rs_elems[r], s.ag_elems[r]) == (T * b.rs_elems, T * b.ag_elems)
        assert s.schedule.peak_live_bytes[r] == b.gathered
    # the owners hold no buffer for their own units: rank 0 owns units 0 and 1,
    # so its largest borrowed unit is unit 2, a non-owner's is unit 2 as well
    assert s.schedule.peak_live_bytes == [2 * 2993, 2 * 2993, 2 * 1500, 2 * 2993, 2 * 2993]


def test_owner_schedule_errors_and_prefetch():
    lay = make_layout(64, 4, 3, [16] * 4, owner_broadcast=True)
    sch = sc.OwnerSchedule(lay)
    with pytest.raises(sc.ScheduleError):
        sch.release(0)
    sch.gather(0)
    with pytest.raises(sc.ScheduleError):
        sch.gather(0)
    with pytest.raises(sc.ScheduleError):
        sch.gather(1)                       # max_live = 1
    sch.release(0)
    pre = sc.OwnerSchedule(lay, max_live=2)
    pre.gather(0)                           # a forward pass with the next unit prefetched
    for u in range(1, 4):
        pre.gather(u)
        pre.release(u - 1)
    pre.release(3)
    for r in range(4):
        assert pre.peak_live_bytes[r] == acc.bytes_per_rank(lay, max_live=2, rank=r).gathered
    with pytest.raises(ValueError):
        sc.ZeRO3Owner(make_layout(64, 4, 3, [16] * 4), np.zeros(64, np.float32), "bf16")
