"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, at
sizes the oracle finishes in seconds: all four schemes on the 65,536-element
/ 4-rank / fp16 workload, ragged and padded sizes, every alignment variant of
the kernels, mixed 16-bit formats, fused against unfused, and the counters
against the accounting."""
import numpy as np
import pytest
import torch

import synth
import zero_sharded_mixed_reduce_amd as z
from oracle import accounting as acc
from oracle import numerics as nm
from oracle import schemes as sc
from oracle.layout import make_layout
from tests.gpu_helpers import compare, dev16, host16, host32, param_map, say

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(params=[5, 0], ids=["deferred", "direct"])
def fused_path(request):
    """Run a test with the fused step's deferred-write kernel (a ring of 5
    tiles, from one gradient row on) and with the kernel that writes at once;
    both must give the same bits.  Where an operand rules out the vector
    path (unaligned rows or state) both ids run the one-element kernel."""
    z.zsmr_set_launch_shape(0, 0, request.param, 1)
    yield request.param
    z.zsmr_set_launch_shape()


def gpu_scheme(stage, numel, world, dt, T, lr, units=None, pad=False, fused=True, gsig=1e-2,
               check_gathers=True, seed=0):
    """Run a scheme over N simulated ranks through the C ABI only."""
    say(f"[gpu_scheme] stage={stage} numel={numel} world={world} dt={dt} T={T} units={units} "
        f"pad={pad} fused={fused}")
    units3 = list(units) if (units and stage == 3) else None
    ctx = z.zero_init_shards(numel, world, stage, dt, pad=pad, units=units3)
    info = ctx.info()
    P = info["padded_numel"]
    pm = param_map(ctx, units3)
    ok = pm >= 0
    p = np.arange(numel)
    theta = synth.theta0(seed, p)

    def padded(x, fill=0):
        out = np.full(P, fill, dtype=x.dtype)
        out[ok] = x[pm[ok]]
        return out

    def grads_dev(t):
        rows = np.stack([padded(synth.grad16(seed, r, t, p, gsig, dt)) for r in range(world)])
        return dev16(rows.ravel())

    reps = world if stage == 0 else 1                 # DP: one full replica per rank
    th = torch.from_numpy(padded(theta)).cuda()
    master = [torch.empty(P, dtype=torch.float32, device="cuda") for _ in range(reps)]
    m = [torch.empty_like(master[0]) for _ in range(reps)]
    v = [torch.empty_like(master[0]) for _ in range(reps)]
    p16 = [torch.empty(P, dtype=TDT[dt], device="cuda") for _ in range(reps)]
    pieces = []
    for u in range(info["n_units"] if stage == 3 else 1):
        for r in range(world):
            off, ln, _ = z.zero_layout(ctx, r, u)
            pieces.append((r, u, off, ln))
    for (r, u, off, ln) in pieces:
        i = r if stage == 0 else 0
        z.zero_init_state(ctx, r, u, th[off:], master[i][off:], m[i][off:], v[i][off:], p16[i][off:])
    g_tmp = torch.empty(max(pc[3] for pc in pieces), dtype=torch.float32, device="cuda")
    unit_buf = torch.empty(info["max_unit_numel"], dtype=TDT[dt], device="cuda")
    gather_bad = 0

    def update(t, G, r, u, off, ln):
        i = r if stage == 0 else 0
        if fused:
            z.zero_fused_step(ctx, r, u, G, P, off, master[i][off:], m[i][off:], v[i][off:],
                              p16[i][off:], t, lr)
        else:
            z.zero_reduce_shard(ctx, r, u, G, P, off, True, g_tmp)
            z.zero_adam_step(master[i][off:], m[i][off:], v[i][off:], g_tmp, ln, t, lr)
            z.zero_gather_cast(ctx, r, u, master[i][off:], p16[i][off:])

    def gather(u):
        nonlocal gather_bad
        offs = [z.zero_layout(ctx, r, u) for r in range(world)]
        z.zero_stage3_unit_gather(ctx, u, [p16[0][o:] for (o, _, _) in offs], unit_buf)
        if check_gathers:
            q0, su = offs[0][0], offs[0][1]
            gather_bad += not torch.equal(unit_buf[:world * su].view(torch.int16),
                                          p16[0][q0:q0 + world * su].view(torch.int16))

    for t in range(1, T + 1):
        G = grads_dev(t)
        if stage != 3:
            for (r, u, off, ln) in pieces:
                update(t, G, r, u, off, ln)
        else:
            U = info["n_units"]
            for u in range(U):
                gather(u)
                z.zero_stage3_unit_release(ctx, u)
            for u in reversed(range(U)):
                gather(u)
                for (r, uu, off, ln) in pieces:
                    if uu == u:
                        update(t, G, r, u, off, ln)
                z.zero_stage3_unit_release(ctx, u)
    torch.cuda.synchronize()
    assert gather_bad == 0, "a gathered unit differs from its shards"

    res = {"ctx": ctx, "P": P, "pm": pm}
    res["reps"] = [{"master": _unpad(host32(master[i]), pm, ok, numel),
                    "m": _unpad(host32(m[i]), pm, ok, numel),
                    "v": _unpad(host32(v[i]), pm, ok, numel),
                    "p16": _unpad(host16(p16[i]), pm, ok, numel),
                    "pad_master": host32(master[i])[~ok], "pad_p16": host16(p16[i])[~ok]}
                   for i in range(reps)]
    return res


def _unpad(x, pm, ok, numel):
    out = np.empty(numel, dtype=x.dtype)
    out[pm[ok]] = x[ok]
    return out


def oracle_scheme(stage, numel, world, dt, T, lr, units=None, pad=False, gsig=1e-2, seed=0):
    p = np.arange(numel)
    theta = synth.theta0(seed, p)

    def g(t):
        return [synth.grad16(seed, r, t, p, gsig, dt) for r in range(world)]
    return sc.run(stage, numel, world, theta, g, T, dt, lr, units=units if stage == 3 else None,
                  pad=pad)


def check_against_oracle(res, ref, what):
    for i, rep in enumerate(res["reps"]):
        compare({"master": rep["master"], "m": rep["m"], "v": rep["v"]},
                {"master": ref.full_master(), "m": ref.full_m(), "v": ref.full_v()},
                rep["p16"], ref.working_copy(), f"{what} replica {i}")
        assert not rep["pad_master"].any() and not rep["pad_p16"].any(), "pad is not zero"


def check_counters(res, stage, numel, world, units, pad, T):
    lay = make_layout(numel, world, stage, units if stage == 3 else None, pad)
    want = acc.bytes_per_rank(lay)
    for r in range(world):
        c = z.zero_counters(res["ctx"], r)
        assert c["rs_elems"] == T * want.rs_elems
        assert c["ag_elems"] == T * want.ag_elems
        assert c["ar_elems"] == T * want.ar_elems
        assert c["traffic_bytes"] == T * want.traffic_bytes
    c = z.zero_counters(res["ctx"], 0)
    if stage == 3:
        U = lay.n_units
        assert c["stage3_gathers"] == 2 * U * T and c["stage3_releases"] == 2 * U * T
        assert c["live_units"] == 0 and c["peak_live_bytes"] == want.gathered
        for u in range(U):
            assert z.zero_stage3_unit_state(res["ctx"], u) == (False, 2 * T, 2 * T)


# --------------------------------------------- the 65,536 / N = 4 workload --
@pytest.mark.parametrize("stage", [0, 1, 2, 3])
@pytest.mark.parametrize("fused", [True, False])
def test_psi65k_all_schemes(stage, fused, fused_path):
    numel, world, dt, T, lr, units = 65536, 4, "fp16", 5, 1e-2, [16384] * 4
    res = gpu_scheme(stage, numel, world, dt, T, lr, units, fused=fused)
    ref = oracle_scheme(stage, numel, world, dt, T, lr, units)
    check_against_oracle(res, ref, f"psi65k stage {stage} fused={fused}")
    check_counters(res, stage, numel, world, units, False, T)


def test_psi65k_stage3_one_unit_is_whole_vector_gather():
    res = gpu_scheme(3, 65536, 4, "fp16", 5, 1e-2, [65536])
    ref = oracle_scheme(3, 65536, 4, "fp16", 5, 1e-2, [65536])
    check_against_oracle(res, ref, "psi65k stage 3, one unit")
    check_counters(res, 3, 65536, 4, [65536], False, 5)


# ------------------------------------------------ ragged and padded sizes --
@pytest.mark.parametrize("numel,world,stage,units,dt", [
    (1001, 4, 1, None, "bf16"),                 # pad: S = 251, rows not 16-byte aligned
    (1001, 3, 2, None, "fp16"),
    (40_003, 5, 2, None, "bf16"),               # several tiles, ragged tail, odd world
    (40_003, 7, 3, [10_001, 7, 29_991, 1, 2, 1], "bf16"),   # tiny units, all padded
    (123_457, 8, 3, [100_000, 23_457], "fp16"),
    (777, 1, 2, None, "bf16"),                  # a world of one
    (7, 1, 1, None, "bf16"),                    # fewer elements than one vector
    (9, 3, 3, [9], "fp16"),                     # padding inside a single unit
    (65_544, 8, 0, None, "bf16"),               # data parallel, not a multiple of 64
    (40_003, 11, 2, None, "fp16"),              # > 8 rows: the deferred kernel, ragged
    (50_001, 16, 3, [30_000, 20_001], "bf16"),  # > 8 rows, stage 3, padded units
])
def test_ragged_and_padded(numel, world, stage, units, dt, fused_path):
    pad = True
    for fused in (True, False):
        res = gpu_scheme(stage, numel, world, dt, 3, 1e-3, units, pad=pad, fused=fused, gsig=1e-2)
        ref = oracle_scheme(stage, numel, world, dt, 3, 1e-3, units, pad=pad)
        check_against_oracle(res, ref, f"ragged {numel}/{world}/stage {stage} fused={fused}")
        check_counters(res, stage, numel, world, units, pad, 3)


# -------------------------------------------------- single-piece variants --
def _piece_inputs(n, world, gdt, seed=0, step=1, sigma=1e-2, outlier=0):
    p = np.arange(n)
    rows = np.stack([synth.grad16(seed, r, step, p, sigma, gdt, outlier) for r in range(world)])
    theta = synth.theta0(seed, p)
    return rows, theta


def _oracle_piece(rows, theta, gdt, pdt, T, lr, steps_rows=None):
    master, m, v = theta.copy(), np.zeros_like(theta), np.zeros_like(theta)
    for t in range(1, T + 1):
        r16 = rows if steps_rows is None else steps_rows[t]
        g = nm.reduce_rank_order([nm.widen16(r, gdt) for r in r16])
        master, m, v = nm.adam_update(master, m, v, g, nm.adam_consts(lr, 0.9, 0.999, 1e-8, t))
    return master, m, v, nm.cast16(master, pdt)


@pytest.mark.parametrize("shift16,shift32,gshift", [
    (0, 0, 0),      # 128-bit everywhere
    (4, 0, 0),      # 16-bit destination 8-byte aligned: 64-bit stores
    (2, 0, 0),      # 4-byte aligned: 32-bit stores
    (1, 0, 0),      # 2-byte aligned: 16-bit stores
    (3, 0, 0),
    (0, 1, 0),      # fp32 state not 16-byte aligned: one element per lane
    (0, 0, 1),      # gradient rows not 16-byte aligned: one element per lane
    (5, 3, 2),
])
@pytest.mark.parametrize("n", [8 * 256 * 3 + 5, 1, 7, 8, 9])
def test_alignment_variants(shift16, shift32, gshift, n, fused_path):
    world, gdt, pdt, T, lr = 12, "bf16", "bf16", 2, 1e-3
    ctx = z.zero_init_shards(n * world, world, 2, gdt, pdt)
    rows, theta = _piece_inputs(n, world, gdt)
    stride = n + 8 + (8 - n % 8) % 8                       # rows 16-byte aligned apart
    gbuf = np.zeros(gshift + world * stride, np.uint16)
    for r in range(world):
        gbuf[gshift + r * stride: gshift + r * stride + n] = rows[r]
    G = dev16(gbuf)
    mk32 = lambda: torch.zeros(n + 8, dtype=torch.float32, device="cuda")
    mb, mm, vb = mk32(), mk32(), mk32()
    pb = torch.zeros(n + 16, dtype=torch.bfloat16, device="cuda")
    th = torch.zeros(n + 8, dtype=torch.float32, device="cuda")
    th[shift32:shift32 + n] = torch.from_numpy(theta).cuda()
    s, s16 = shift32, shift16
    z.zero_init_state(ctx, 0, 0, th[s:], mb[s:], mm[s:], vb[s:], pb[s16:])
    for t in range(1, T + 1):
        z.zero_fused_step(ctx, 0, 0, G[gshift:], stride, 0, mb[s:], mm[s:], vb[s:], pb[s16:], t, lr)
    torch.cuda.synchronize()
    master, m, v, p16 = _oracle_piece(rows, theta, gdt, pdt, T, lr)
    got16 = host16(pb)
    compare({"master": host32(mb)[s:s + n], "m": host32(mm)[s:s + n], "v": host32(vb)[s:s + n]},
            {"master": master, "m": m, "v": v}, got16[s16:s16 + n], p16,
            f"alignment shift16={shift16} shift32={shift32} gshift={gshift} n={n}")
    # nothing outside the piece was written
    assert not got16[:s16].any() and not got16[s16 + n:].any()
    assert not host32(mb)[:s].any() and not host32(mb)[s + n:].any()



@pytest.mark.parametrize("shape", [0, 1, 2, 5])
@pytest.mark.parametrize("n", [512 * 300 + 77, 512 * 4000 + 5])
def test_step_grid_shapes(shape, n):
    """The step kernels' grid (one wave tile per wave, or grid-stride with
    1, 2 or 5 workgroups per CU) changes nothing: the fused step (direct
    kernel, 6 rows) and the reduce, Adam and cast launches all match the
    oracle, with heads (the piece 24 elements into a line) and tails."""
    world, gdt, lr, off = 6, "bf16", 1e-3, 24
    say(f"[step grid] shape={shape} n={n}")
    z.zsmr_set_launch_shape(shape, 0, 3, 16)
    try:
        rows, theta, G, stride, th, mb, mm, vb, gb, pb = _line_buffers(n, world, gdt, off, off, off)
        ctx = z.zero_init_shards(n * world, world, 2, gdt)
        z.zero_init_state(ctx, 0, 0, th[off:], mb[off:], mm[off:], vb[off:], pb[off:])
        for t in (1, 2):
            z.zero_fused_step(ctx, 0, 0, G[off:], stride, 0, mb[off:], mm[off:], vb[off:], pb[off:], t, lr)
        z.zero_reduce_shard(ctx, 0, 0, G[off:], stride, 0, True, gb[off:])
        z.zero_adam_step(mb[off:], mm[off:], vb[off:], gb[off:], n, 3, lr)
        z.zero_gather_cast(ctx, 0, 0, mb[off:], pb[off:])
        torch.cuda.synchronize()
    finally:
        z.zsmr_set_launch_shape()
    master, m, v, p16 = _oracle_piece(rows, theta, gdt, gdt, 3, lr)
    got16 = host16(pb)
    compare({"master": host32(mb)[off:off + n], "m": host32(mm)[off:off + n], "v": host32(vb)[off:off + n]},
            {"master": master, "m": m, "v": v}, got16[off:off + n], p16, f"step grid shape={shape} n={n}")
    assert not got16[:off].any() and not got16[off + n:].any()
    for b in (mb, mm, vb):
        assert not host32(b)[:off].any() and not host32(b)[off + n:].any()

# (gradient rows, fp32 state, 16-bit copy) offsets in elements from a 128-byte line
LINE_OFFSETS = [
    (0, 0, 0),
    (24, 24, 24),     # a rank's shard at r*S with S = 24 mod 64 (1.558e9 elements on 16 ranks)
    (8, 8, 8),
    (56, 56, 56),
    (40, 0, 0),       # rows and state on different lines: the tiles follow the rows
    (4, 0, 4),        # rows 8-byte aligned: after a head of 60 all on a line
    (4, 0, 0),        # ... and the 16-bit copy then 8-byte aligned (64-bit stores)
    (0, 12, 0),       # state off its line, rows on theirs: no head
    (8, 2, 8),        # state 8-byte aligned: one element per lane, no head
]


def _line_buffers(n, world, gdt, goff, soff, poff):
    rows, theta = _piece_inputs(n, world, gdt, seed=3)
    stride = n + 64 - n % 64                                # rows 128 bytes apart
    gbuf = np.zeros(goff + world * stride, np.uint16)
    for r in range(world):
        gbuf[goff + r * stride: goff + r * stride + n] = rows[r]
    mk32 = lambda: torch.zeros(n + 64, dtype=torch.float32, device="cuda")
    th = mk32()
    th[soff:soff + n] = torch.from_numpy(theta).cuda()
    return rows, theta, dev16(gbuf), stride, th, mk32(), mk32(), mk32(), mk32(), \
        torch.zeros(n + 64, dtype=torch.bfloat16, device="cuda")


@pytest.mark.parametrize("goff,soff,poff", LINE_OFFSETS)
@pytest.mark.parametrize("world", [4, 16])
def test_line_heads_fused(goff, soff, poff, world, fused_path):
    """Pieces that do not start on a 128-byte line: the vector body's tiles
    start on the line of the gradient rows, and the elements before it run
    one by one.  Results match the oracle; nothing outside the piece is
    written."""
    n, gdt, T, lr = 512 * 40 + 77, "bf16", 2, 1e-3
    say(f"[line heads fused] offsets={goff},{soff},{poff} world={world} defer={fused_path}")
    rows, theta, G, stride, th, mb, mm, vb, _, pb = _line_buffers(n, world, gdt, goff, soff, poff)
    ctx = z.zero_init_shards(n * world, world, 2, gdt)
    s, q = soff, poff
    z.zero_init_state(ctx, 0, 0, th[s:], mb[s:], mm[s:], vb[s:], pb[q:])
    for t in range(1, T + 1):
        z.zero_fused_step(ctx, 0, 0, G[goff:], stride, 0, mb[s:], mm[s:], vb[s:], pb[q:], t, lr)
    torch.cuda.synchronize()
    master, m, v, p16 = _oracle_piece(rows, theta, gdt, gdt, T, lr)
    got16 = host16(pb)
    compare({"master": host32(mb)[s:s + n], "m": host32(mm)[s:s + n], "v": host32(vb)[s:s + n]},
            {"master": master, "m": m, "v": v}, got16[q:q + n], p16,
            f"line heads offsets={goff},{soff},{poff} world={world}")
    assert not got16[:q].any() and not got16[q + n:].any()
    for b in (mb, mm, vb):
        assert not host32(b)[:s].any() and not host32(b)[s + n:].any()


@pytest.mark.parametrize("goff,soff,poff", LINE_OFFSETS)
def test_line_heads_three_kernels(goff, soff, poff):
    """The same pieces through the reduce, Adam and cast kernels: the reduce
    aligns on the gradient rows, Adam and the cast on the fp32 master."""
    n, world, gdt, lr = 512 * 40 + 77, 6, "bf16", 1e-3
    say(f"[line heads three kernels] offsets={goff},{soff},{poff}")
    rows, theta, G, stride, th, mb, mm, vb, gb, pb = _line_buffers(n, world, gdt, goff, soff, poff)
    ctx = z.zero_init_shards(n * world, world, 2, gdt)
    s, q = soff, poff
    z.zero_init_state(ctx, 0, 0, th[s:], mb[s:], mm[s:], vb[s:], pb[q:])
    z.zero_reduce_shard(ctx, 0, 0, G[goff:], stride, 0, True, gb[s:])
    z.zero_adam_step(mb[s:], mm[s:], vb[s:], gb[s:], n, 1, lr)
    z.zero_gather_cast(ctx, 0, 0, mb[s:], pb[q:])
    torch.cuda.synchronize()
    g = nm.reduce_rank_order([nm.widen16(r, gdt) for r in rows])
    assert np.array_equal(host32(gb)[s:s + n].view(np.uint32), g.view(np.uint32))
    master, m, v, p16 = _oracle_piece(rows, theta, gdt, gdt, 1, lr)
    got16 = host16(pb)
    compare({"master": host32(mb)[s:s + n], "m": host32(mm)[s:s + n], "v": host32(vb)[s:s + n]},
            {"master": master, "m": m, "v": v}, got16[q:q + n], p16,
            f"line heads (three kernels) offsets={goff},{soff},{poff}")
    assert not got16[:q].any() and not got16[q + n:].any()
    for b in (mb, mm, vb, gb):
        assert not host32(b)[:s].any() and not host32(b)[s + n:].any()



@pytest.mark.parametrize("gdt,pdt", [("fp16", "bf16"), ("bf16", "fp16"), ("fp16", "fp16")])
def test_mixed_formats(gdt, pdt, fused_path):
    n, world, T, lr = 3 * 2048 + 3, 17, 3, 1e-2
    ctx = z.zero_init_shards(n * world, world, 1, gdt, pdt)
    steps_rows = {t: _piece_inputs(n, world, gdt, step=t)[0] for t in range(1, T + 1)}
    theta = synth.theta0(0, np.arange(n))
    th = torch.from_numpy(theta).cuda()
    mb = torch.empty(n, dtype=torch.float32, device="cuda")
    mm, vb = torch.empty_like(mb), torch.empty_like(mb)
    pb = torch.empty(n, dtype=TDT[pdt], device="cuda")
    z.zero_init_state(ctx, 0, 0, th, mb, mm, vb, pb)
    for t in range(1, T + 1):
        z.zero_fused_step(ctx, 0, 0, dev16(steps_rows[t].ravel()), n, 0, mb, mm, vb, pb, t, lr)
    torch.cuda.synchronize()
    master, m, v, p16 = _oracle_piece(None, theta, gdt, pdt, T, lr, steps_rows)
    compare({"master": host32(mb), "m": host32(mm), "v": host32(vb)},
            {"master": master, "m": m, "v": v}, host16(pb), p16, f"mixed {gdt}->{pdt}")


def _padded_rows(rows: np.ndarray, stride: int) -> torch.Tensor:
    """rows (N x n 16-bit) on the device, row r at r*stride."""
    buf = np.zeros((rows.shape[0], stride), np.uint16)
    buf[:, :rows.shape[1]] = rows
    return dev16(buf.ravel())


def _expect_kernel(ctx, grads, stride, master, m, v, p16, kernel, ring=None, windowed=None,
                   store=None):
    """Ask the library which kernel these buffers select and insist on it, so
    that a test meant for one kernel cannot silently run another."""
    plan = z.zsmr_fused_step_plan(ctx, 0, 0, grads, stride, 0, master, m, v, p16)
    assert plan["kernel"] == kernel, plan
    if ring is not None:
        assert plan["ring_tiles"] == ring, plan
    if windowed is not None:
        assert bool(plan["windowed"]) == windowed, plan
    if store is not None:
        assert plan["store_elems"] == store, plan
    return plan


@pytest.mark.parametrize("tiles", [5, 3, 1])
def test_deferred_kernel_many_rounds(tiles):
    """The deferred-write kernel with each wave's LDS ring filled several
    times over (1,024 waves, about 10 tiles each) and a ragged tail, 9 rows
    (one whole row batch and a batch of one row), against the oracle."""
    z.zsmr_set_launch_shape(0, 0, tiles, 1)
    try:
        n = 1024 * 10 * 512 + 3 * 512 + 77
        stride = (n + 63) // 64 * 64                       # rows on 128-byte lines, n ragged
        world, T, lr = 9, 2, 1e-3
        ctx = z.zero_init_shards(n * world, world, 2, "bf16")
        steps_rows = {t: _piece_inputs(n, world, "bf16", step=t)[0] for t in range(1, T + 1)}
        theta = synth.theta0(0, np.arange(n))
        mb = torch.from_numpy(theta.copy()).cuda()
        mm, vb = torch.empty_like(mb), torch.empty_like(mb)
        pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        z.zero_init_state(ctx, 0, 0, mb.clone(), mb, mm, vb, pb)
        for t in range(1, T + 1):
            G = _padded_rows(steps_rows[t], stride)
            # 9 rows: no windows, so a ring of at most 2 tiles
            _expect_kernel(ctx, G, stride, mb, mm, vb, pb, "deferred", ring=min(tiles, 2),
                           windowed=False)
            z.zero_fused_step(ctx, 0, 0, G, stride, 0, mb, mm, vb, pb, t, lr)
        torch.cuda.synchronize()
        master, m, v, p16 = _oracle_piece(None, theta, "bf16", "bf16", T, lr, steps_rows)
        compare({"master": host32(mb), "m": host32(mm), "v": host32(vb)},
                {"master": master, "m": m, "v": v}, host16(pb), p16, f"deferred tiles={tiles} n={n}")
    finally:
        z.zsmr_set_launch_shape()


def _fused_run(n, rows, T, defer, window, guard=64, p16_shift=0, expect=None):
    """T fused steps on one n-element piece with rows gradient rows made by
    the device generator (row stride n rounded up to 64 elements, so the
    vector kernels run); returns the outputs with `guard` untouched elements
    on both sides of every buffer.  p16_shift moves the 16-bit copy that many
    elements off its 8-byte alignment (2: 32-bit stores, 1: 16-bit stores).
    expect: the kernel the buffers must select (checked with the library's
    plan query)."""
    import synth.gpu as sgpu
    z.zsmr_set_launch_shape(0, 0, defer, 1)
    z.zsmr_set_write_window(*window)
    try:
        stride = (n + 63) // 64 * 64
        ctx = z.zero_init_shards(n * rows, rows, 2, "bf16")
        G = torch.empty(rows * stride, dtype=torch.int16, device="cuda")
        th = torch.empty(n, dtype=torch.float32, device="cuda")
        sgpu.fill32(th, n, 0, n, 7, synth.TAG_THETA, 0, 0, 0.02)
        buf = lambda dt, extra=0: torch.full((n + 2 * guard + extra,), -3, dtype=dt, device="cuda")
        mb, mm, vb = buf(torch.float32), buf(torch.float32), buf(torch.float32)
        pb_all = buf(torch.int16, 4)
        pb = pb_all[p16_shift:p16_shift + n + 2 * guard]
        sl = slice(guard, guard + n)
        if expect is not None:
            _expect_kernel(ctx, G, stride, mb[sl], mm[sl], vb[sl], pb[sl], **expect)
        z.zero_init_state(ctx, 0, 0, th, mb[sl], mm[sl], vb[sl], pb[sl])
        for t in range(1, T + 1):
            sgpu.fill16(G, rows, stride, n, 0, n, 7, synth.TAG_GRAD, 0, t, 1e-2, "bf16")
            z.zero_fused_step(ctx, 0, 0, G, stride, 0, mb[sl], mm[sl], vb[sl], pb[sl], t, 1e-3)
        torch.cuda.synchronize()
        return mb, mm, vb, pb
    finally:
        z.zsmr_set_launch_shape()
        z.zsmr_set_write_window()


WINDOWS = {
    "default": z.WRITE_WINDOW_DEFAULT,
    "off": (0, 0, 0, 0),
    "short": (1000, 300, 0, 0),                # many windows per tile: partial sums cross them
    "margin": (4000, 500, 700, 200),           # scaled to 1,506 ns at 16 rows
    "long": (200000, 20000, 0, 5000),          # the ring fills long before a window
}


@pytest.mark.parametrize("window", list(WINDOWS), ids=list(WINDOWS))
@pytest.mark.parametrize("kd", [1, 2, 3, 5])
@pytest.mark.parametrize("rows", [1, 4, 5, 8, 9, 16, 33, 64])
def test_deferred_windows_match_direct_bits(window, kd, rows):
    """Write windows and ring sizes change only when results are stored:
    the deferred kernel gives the direct kernel's bits, and writes nothing
    outside the piece.  With 4 rows or fewer a tile is one row batch (its
    first and last); windows apply from 16 rows, their cycle scaled to the
    row count (without windows the ring holds at most 2 tiles)."""
    n = 1024 * 6 * 512 + 2 * 512 + 131           # ~6 tiles per wave, a ragged tail
    say(f"[deferred] window={window} kd={kd} rows={rows} n={n}")
    windowed = window != "off" and rows >= 16
    ref = _fused_run(n, rows, 2, 0, WINDOWS["off"], expect={"kernel": "direct"})
    got = _fused_run(n, rows, 2, kd, WINDOWS[window],
                     expect={"kernel": "deferred", "windowed": windowed,
                             "ring": kd if windowed else min(kd, 2)})
    for name, a, b in zip(("master", "m", "v", "p16"), ref, got):
        ai = a.view(torch.int32) if a.dtype == torch.float32 else a
        bi = b.view(torch.int32) if b.dtype == torch.float32 else b
        diff = int((ai != bi).sum())
        assert diff == 0, f"{name}: {diff} elements differ"
    g = 64
    for b in got:
        bi = b.view(torch.int32) if b.dtype == torch.float32 else b
        fill = torch.full((g,), -3, dtype=b.dtype, device="cuda")
        fi = fill.view(torch.int32) if b.dtype == torch.float32 else fill
        assert torch.equal(bi[:g], fi) and torch.equal(bi[-g:], fi)


@pytest.mark.parametrize("rows,kd,p16_shift", [
    (64, 5, 0), (64, 3, 0),
    (64, 3, 2), (64, 3, 1),       # 16-bit copy 4-byte and 2-byte aligned (32- and 16-bit stores)
    (16, 3, 2), (16, 3, 1),       # the fewest rows with windows
    (24, 3, 0), (33, 3, 1),
])
def test_deferred_sampled_against_oracle(rows, kd, p16_shift):
    """Windowed deferred runs (default windows, rings of 3 and 5 tiles, 16-bit
    stores of every width) against the oracle on every element of three
    whole tiles, a wave's later tiles and the tail."""
    n, T = 1024 * 6 * 512 + 2 * 512 + 131, 2
    say(f"[deferred sampled] rows={rows} kd={kd} p16_shift={p16_shift}")
    store = {0: 4, 2: 2, 1: 1}[p16_shift]
    mb, mm, vb, pb = _fused_run(n, rows, T, kd, WINDOWS["default"], p16_shift=p16_shift,
                                expect={"kernel": "deferred", "ring": kd, "windowed": True,
                                        "store": store})
    g = 64
    # tiles 0, 1023-1024, a wave's second and third tiles (2,048 waves in the
    # windowed grid of 2 workgroups per CU) and the tail
    pos = np.concatenate([np.arange(0, 512), np.arange(512 * 1023, 512 * 1025),
                          np.arange(512 * 2048, 512 * 2049), np.arange(512 * 4096, 512 * 4097),
                          np.arange(n - 1200, n)])
    p = pos.astype(np.int64)
    theta = synth.theta0(7, p)
    master, m, v = theta.copy(), np.zeros_like(theta), np.zeros_like(theta)
    for t in range(1, T + 1):
        r16 = [synth.grad16(7, r, t, p, 1e-2, "bf16") for r in range(rows)]
        gr = nm.reduce_rank_order([nm.widen16(r, "bf16") for r in r16])
        master, m, v = nm.adam_update(master, m, v, gr, nm.adam_consts(1e-3, 0.9, 0.999, 1e-8, t))
    at = lambda x: host32(x)[g + pos] if x.dtype == torch.float32 else host16(x)[g + pos]
    compare({"master": at(mb), "m": at(mm), "v": at(vb)}, {"master": master, "m": m, "v": v},
            at(pb), nm.cast16(master, "bf16"), f"deferred windowed sampled rows={rows} kd={kd} "
            f"p16_shift={p16_shift}")


@pytest.mark.parametrize("rows", [8, 9, 12, 13, 14, 16, 17, 20, 23])
def test_direct_kernel_row_batches_against_oracle(rows):
    """The direct kernel loads 12 gradient rows per batch at 9-13 and 16-23
    rows and 8 otherwise (the library's plan says which): every element
    against the oracle, two steps, a ragged tail."""
    n, T, lr = 512 * 40 + 77, 2, 1e-3
    z.zsmr_set_launch_shape(0, 0, 0, 24)            # no deferred kernel: the direct one at any rows
    try:
        ctx = z.zero_init_shards(n * rows, rows, 2, "bf16")
        stride = (n + 63) // 64 * 64
        steps_rows = {t: _piece_inputs(n, rows, "bf16", step=t, seed=4)[0] for t in range(1, T + 1)}
        theta = synth.theta0(4, np.arange(n))
        mb = torch.from_numpy(theta.copy()).cuda()
        mm, vb = torch.empty_like(mb), torch.empty_like(mb)
        pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        z.zero_init_state(ctx, 0, 0, mb.clone(), mb, mm, vb, pb)
        want_rb = 12 if 9 <= rows <= 13 or 16 <= rows <= 23 else 8
        for t in range(1, T + 1):
            G = _padded_rows(steps_rows[t], stride)
            plan = _expect_kernel(ctx, G, stride, mb, mm, vb, pb, "direct")
            assert plan["row_batch"] == want_rb, plan
            z.zero_fused_step(ctx, 0, 0, G, stride, 0, mb, mm, vb, pb, t, lr)
        torch.cuda.synchronize()
    finally:
        z.zsmr_set_launch_shape()
    theta = synth.theta0(4, np.arange(n))
    master, m, v, p16 = _oracle_piece(None, theta, "bf16", "bf16", T, lr, steps_rows)
    compare({"master": host32(mb), "m": host32(mm), "v": host32(vb)},
            {"master": master, "m": m, "v": v}, host16(pb), p16, f"direct rows={rows}")


@pytest.mark.parametrize("world", [16, 12, 64])     # the mean multiplies by 1/N for 16 and 64
@pytest.mark.parametrize("gdt", ["bf16", "fp16"])
def test_reduce_sum_and_mean(gdt, world):
    n = 10_000 + 3
    ctx = z.zero_init_shards(n * world, world, 2, gdt)
    rows, _ = _piece_inputs(n, world, gdt, sigma=1e-1, outlier=100)
    G = dev16(rows.ravel())
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    for mean in (False, True):
        z.zero_reduce_shard(ctx, 0, 0, G, n, 0, mean, out)
        torch.cuda.synchronize()
        want = nm.reduce_rank_order([nm.widen16(r, gdt) for r in rows], mean=mean)
        assert np.array_equal(host32(out).view(np.uint32), want.view(np.uint32)), f"mean={mean}"


def test_zero_gradient_leaves_master_and_adam_only_matches():
    n = 5000
    theta = synth.theta0(0, np.arange(n))
    g = np.zeros(n, np.float32)
    mb = torch.from_numpy(theta.copy()).cuda()
    mm, vb = torch.zeros_like(mb), torch.zeros_like(mb)
    for t in range(1, 4):
        z.zero_adam_step(mb, mm, vb, torch.from_numpy(g).cuda(), n, t, 1e-2)
    torch.cuda.synchronize()
    assert np.array_equal(host32(mb).view(np.uint32), theta.view(np.uint32))
    assert not host32(mm).any() and not host32(vb).any()
    # Adam alone against the oracle on a wide range of magnitudes
    rng = np.random.default_rng(2)
    gg = (rng.normal(0, 1, n) * 10.0 ** rng.uniform(-9, 1, n)).astype(np.float32)
    mb = torch.from_numpy(theta.copy()).cuda()
    mm, vb = torch.zeros_like(mb), torch.zeros_like(mb)
    master, m, v = theta.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 6):
        z.zero_adam_step(mb, mm, vb, torch.from_numpy(gg).cuda(), n, t, 3e-3, (0.8, 0.95), 1e-6)
        master, m, v = nm.adam_update(master, m, v, gg, nm.adam_consts(3e-3, 0.8, 0.95, 1e-6, t))
    torch.cuda.synchronize()
    for got, want in ((mb, master), (mm, m), (vb, v)):
        assert np.array_equal(host32(got).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_cast_special_values(dt):
    vals = np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65520.0, 1e30, -1e30, np.inf, -np.inf, 6e-8,
                     3e-45, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11,
                     3.4e38, 5.96e-8, 2.98e-8, 1.5e-38], np.float32)
    rng = np.random.default_rng(9)
    rand = rng.integers(0, 1 << 32, 1 << 16, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([vals, rand[np.isfinite(rand)]]).astype(np.float32)
    ctx = z.zero_init_shards(x.size, 1, 2, dt)
    out = torch.empty(x.size, dtype=TDT[dt], device="cuda")
    z.zero_gather_cast(ctx, 0, 0, torch.from_numpy(x).cuda(), out)
    torch.cuda.synchronize()
    assert np.array_equal(host16(out), nm.cast16(x, dt))


def test_gather_copy_alignments():
    n = 100_003
    src = np.arange(n + 32, dtype=np.uint16)
    ctx = z.zero_init_shards(64, 2, 2, "bf16")
    for so, do in [(0, 0), (4, 4), (1, 1), (2, 6), (3, 0), (0, 5)]:
        S = dev16(src)
        D = torch.zeros(n + 32, dtype=torch.int16, device="cuda")
        z.zero_gather_copy(ctx, 1, S[so:], D[do:], n)
        torch.cuda.synchronize()
        got = host16(D)
        assert np.array_equal(got[do:do + n], src[so:so + n])
        assert not got[:do].any() and not got[do + n:].any()
    assert z.zero_counters(ctx, 1)["ag_elems"] == 6 * n


@pytest.mark.parametrize("n,count,stride", [
    (1, 1, 1), (7, 3, 7), (2_000_003, 5, 2_000_003),     # blocks end to end; every block aligned differently
    (100_003, 63, 117_003), (1_048_576, 4, 1_048_580),   # gaps between blocks
    (16_384, 2, 16_384 + 64), (33, 17, 40),
])
@pytest.mark.parametrize("soff,doff", [(0, 0), (3, 3), (40, 40),   # 16-byte vectors
                                       (4, 0), (2, 0), (1, 0), (0, 7)])   # 8-, 4-, 2-byte
def test_gather_copy_blocks(n, count, stride, soff, doff):
    """count blocks of n elements, block k at k*stride: the same bytes as
    count single copies, nothing written between or around the blocks, and
    count*n elements counted; source and destination equally aligned or not
    (the copy's vector width follows their distance)."""
    say(f"[copy blocks] n={n} count={count} stride={stride} soff={soff} doff={doff}")
    span = (count - 1) * stride + n
    rng = np.random.default_rng(n + count)
    src = rng.integers(1, 1 << 16, span + 128, dtype=np.uint64).astype(np.uint16)
    S = dev16(src)
    D = torch.zeros(span + 128, dtype=torch.int16, device="cuda")
    ctx = z.zero_init_shards(64, 2, 2, "bf16")
    z.zero_gather_copy_blocks(ctx, 1, S[soff:], D[doff:], n, count, stride)
    torch.cuda.synchronize()
    got = host16(D)
    want = np.zeros_like(src)
    for k in range(count):
        want[doff + k * stride:doff + k * stride + n] = src[soff + k * stride:soff + k * stride + n]
    assert np.array_equal(got, want)
    assert z.zero_counters(ctx, 1)["ag_elems"] == count * n


def test_stage3_gather_with_shards_already_in_their_slots():
    """Shards that already sit at their own slots of the unit buffer (an
    in-place gather) are left as they are; the others are copied in."""
    world, units = 4, [40_000, 12_345]
    ctx = z.zero_init_shards(sum(units), world, 3, "bf16", pad=True, units=units)
    for u in range(len(units)):
        each = z.zero_layout(ctx, 0, u)[1]
        rng = np.random.default_rng(u)
        want = rng.integers(0, 1 << 16, world * each, dtype=np.uint64).astype(np.uint16)
        buf = torch.zeros(world * each + 64, dtype=torch.int16, device="cuda")
        unit_buf = buf[32:32 + world * each]
        inplace = {0, 2}
        for r in inplace:                     # shards 0 and 2 are already in place
            unit_buf[r * each:(r + 1) * each] = dev16(want[r * each:(r + 1) * each])
        others = {r: dev16(want[r * each:(r + 1) * each]) for r in range(world) if r not in inplace}
        ptrs = [unit_buf[r * each:] if r in inplace else others[r] for r in range(world)]
        say(f"[gather in place] unit {u} each={each}")
        z.zero_stage3_unit_gather(ctx, u, ptrs, unit_buf)
        torch.cuda.synchronize()
        got = host16(buf)
        assert np.array_equal(got[32:32 + world * each], want)
        assert not got[:32].any() and not got[32 + world * each:].any()
        z.zero_stage3_unit_release(ctx, u)


@pytest.mark.parametrize("n", [1, 7, 8, 9, 16_383, 16_384, 16_385, 3 * 16_384 + 5,
                               (1 << 24) + 777, 256 * 4 * 2 * 16_384 + 3])
@pytest.mark.parametrize("off", [0, 3, 40])     # 40: a 24-element head to a 128-byte line
@pytest.mark.parametrize("shape", [0, 1, 3])   # one burst per wave; grid-stride 1 and 3 per CU
def test_burst_copy_sizes(n, off, shape):
    """The 16-byte copy moves 2,048-vector chunks per wave (16,384 elements);
    sizes around one chunk, several chunks per wave and a partial last chunk,
    with a head (off = 3: equal misalignment of source and destination), in
    the default one-burst-per-wave grid and in grid-stride grids."""
    say(f"[copy] n={n} off={off} shape={shape}")
    z.zsmr_set_launch_shape(0, shape, 3, 16)
    try:
        _copy_case(n, off)
    finally:
        z.zsmr_set_launch_shape()


@pytest.mark.parametrize("n", [100, 3 * 16_384 + 5, (1 << 20) + 77])
@pytest.mark.parametrize("grid_off", [0, 128, 18_304, 65_536 - 128, 131_072 - 128])
def test_copy_chunk_grid_offsets(n, grid_off):
    """The burst copy lays its 32 KB chunks out from the destination's 128 KB
    boundary below the vector body: destinations at chosen distances past
    such a boundary (partial first chunks of every size), small and large
    copies, a source at another offset modulo 128 KB; bytes exact, nothing
    outside written."""
    say(f"[copy grid] n={n} grid_off={grid_off}")
    ctx = z.zero_init_shards(64, 2, 2, "bf16")
    rng = np.random.default_rng(n + grid_off)
    src = rng.integers(0, 1 << 16, n + 4096, dtype=np.uint16)
    S = dev16(src)
    D = torch.zeros(n + (1 << 17), dtype=torch.int16, device="cuda")
    # element offset putting D[off] grid_off bytes past a 128 KB boundary
    off = ((grid_off - D.data_ptr()) % (1 << 17)) // 2
    soff = 1000                                   # source 16-byte aligned like the destination
    soff += ((D.data_ptr() + 2 * off) - (S.data_ptr() + 2 * soff)) % 16 // 2
    z.zero_gather_copy(ctx, 1, S[soff:], D[off:], n)
    torch.cuda.synchronize()
    got = host16(D)
    assert np.array_equal(got[off:off + n], src[soff:soff + n])
    assert not got[:off].any() and not got[off + n:].any()

def _copy_case(n, off):
    rng = np.random.default_rng(n + off)
    src = rng.integers(0, 1 << 16, n + 2 * off + 16, dtype=np.uint16)
    ctx = z.zero_init_shards(64, 2, 2, "bf16")
    S = dev16(src)
    D = torch.zeros(n + 2 * off + 16, dtype=torch.int16, device="cuda")
    z.zero_gather_copy(ctx, 1, S[off:], D[off:], n)
    torch.cuda.synchronize()
    got = host16(D)
    assert np.array_equal(got[off:off + n], src[off:off + n])
    assert not got[:off].any() and not got[off + n:].any()


@pytest.mark.parametrize("permille", [500, 1000, 2000])
def test_copies_cover_every_region_at_any_xcd_weight(permille):
    """However the copies weight the even XCDs against the odd ones, every
    element is copied once: the receive, the block receive and the ZeRO-3
    gather are byte-exact, nothing around them is written, and the counters
    do not depend on the weight."""
    say(f"[xcd balance] permille={permille}")
    z.zsmr_set_xcd_balance(permille)
    try:
        rng = np.random.default_rng(permille)
        for n, off in ((1, 0), (33, 3), (1_000_003, 0), (4_194_304 + 77, 5), (40_000_000, 8)):
            src = rng.integers(1, 1 << 16, n + 64, dtype=np.uint64).astype(np.uint16)
            S = dev16(src)
            D = torch.zeros(n + 64, dtype=torch.int16, device="cuda")
            ctx = z.zero_init_shards(64, 2, 2, "bf16")
            z.zero_gather_copy(ctx, 1, S[off:], D[off:], n)
            torch.cuda.synchronize()
            got = host16(D)
            assert np.array_equal(got[off:off + n], src[off:off + n]), n
            assert not got[:off].any() and not got[off + n:].any(), n
            assert z.zero_counters(ctx, 1)["ag_elems"] == n
        n, count, stride = 100_003, 63, 117_003
        span = (count - 1) * stride + n
        src = rng.integers(1, 1 << 16, span, dtype=np.uint64).astype(np.uint16)
        D = torch.zeros(span, dtype=torch.int16, device="cuda")
        ctx = z.zero_init_shards(64, 2, 2, "bf16")
        z.zero_gather_copy_blocks(ctx, 1, dev16(src), D, n, count, stride)
        torch.cuda.synchronize()
        want = np.zeros_like(src)
        for k in range(count):
            want[k * stride:k * stride + n] = src[k * stride:k * stride + n]
        assert np.array_equal(host16(D), want)
        units = [8 * 300_001, 8 * 5]
        s3 = z.zero_init_shards(sum(units), 8, 3, "bf16", units=units)
        for u, total in enumerate(units):
            each = total // 8
            shards = [dev16(rng.integers(1, 1 << 16, each, dtype=np.uint64).astype(np.uint16))
                      for _ in range(8)]
            buf = torch.zeros(total + 16, dtype=torch.int16, device="cuda")
            z.zero_stage3_unit_gather(s3, u, shards, buf)
            torch.cuda.synchronize()
            got = host16(buf)
            assert np.array_equal(got[:total], np.concatenate([host16(x) for x in shards]))
            assert not got[total:].any()
            z.zero_stage3_unit_release(s3, u)
    finally:
        z.zsmr_set_xcd_balance()
