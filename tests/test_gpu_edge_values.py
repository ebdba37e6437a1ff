"""Inputs the generator never produces, through the kernels, bit for bit
against the oracle ("The four schemes", Base._adam and the 16-bit casts):

* fp32-subnormal and tiny gradients (1e-45 .. 1e-30) and fp32-subnormal m
  and v, where a flush to zero or an inexact division or square root would
  part from NumPy's gradual underflow;
* 16-bit gradients near and below the smallest normal (bf16 about 1e-38,
  fp16 about 6e-5), summed over the ranks;
* NaN and +-Inf gradient entries;
* zero gradients with zero moments next to all of these, which must leave
  the master bit-unchanged.

Every element of master, m, v and the 16-bit copy must carry the oracle's
bits, except that a NaN matches any NaN (the pages fix no NaN payload).  The
fused step runs in each of its kernels (one element per lane, the direct
kernel, the deferred-write kernel with and without write windows); the
library's plan query confirms which one ran.
"""
import numpy as np
import pytest
import torch

import zero_sharded_mixed_reduce_amd as z
from oracle import numerics as nm
from tests.gpu_helpers import dev16, host16, host32, say

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def same_f32(got, want, what):
    """Bit-equal, or NaN on both sides."""
    got, want = np.asarray(got, np.float32), np.asarray(want, np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    bad = np.flatnonzero(gn != wn)
    assert bad.size == 0, f"{what}: NaN at {bad[:5]} on one side only"
    neq = np.flatnonzero(got.view(np.uint32)[~gn] != want.view(np.uint32)[~wn])
    assert neq.size == 0, (f"{what}: {neq.size} elements differ, e.g. got "
                           f"{got[~gn][neq[:3]]} want {want[~wn][neq[:3]]}")
    return int(gn.sum())


def nan16(bits, dtype):
    b = bits.astype(np.uint32) & 0x7FFF
    return b > (0x7F80 if dtype == "bf16" else 0x7C00)


def same_16(got, want, dtype, what):
    gn, wn = nan16(got, dtype), nan16(want, dtype)
    assert np.array_equal(gn, wn), f"{what}: NaN on one side only"
    neq = np.flatnonzero(got[~gn] != want[~wn])
    assert neq.size == 0, f"{what}: {neq.size} 16-bit values differ"


def f32_from_bits(u):
    return np.asarray(u, np.uint32).view(np.float32)


def special_f32(rng, n):
    """fp32 values: subnormals, tiny normals up to 1e-30, zeros, NaN, +-Inf,
    and ordinary values, with random signs."""
    kinds = rng.integers(0, 8, n)
    sub = rng.integers(1, 0x00800000, n, dtype=np.uint64).astype(np.uint32)
    tiny = rng.integers(0x00800000, 0x0DA24260, n, dtype=np.uint64).astype(np.uint32)   # up to ~1e-30
    ordinary = rng.integers(0x30000000, 0x3F800000, n, dtype=np.uint64).astype(np.uint32)
    bits = np.where(kinds < 3, sub, np.where(kinds < 5, tiny, ordinary))
    bits = np.where(kinds == 6, 0, bits)
    sign = rng.integers(0, 2, n).astype(np.uint32) << 31
    x = f32_from_bits(bits | sign).copy()
    k = rng.integers(0, n, max(1, n // 200))
    x[k[0::3]] = np.nan
    x[k[1::3]] = np.inf
    x[k[2::3]] = -np.inf
    return x


def subnormal_f32(rng, n, signed=True):
    bits = rng.integers(0, 0x00800000, n, dtype=np.uint64).astype(np.uint32)
    if signed:
        bits |= rng.integers(0, 2, n).astype(np.uint32) << 31
    return f32_from_bits(bits).copy()


def special_rows16(rng, world, n, dtype):
    """16-bit gradient rows around the smallest normal of the format (bf16:
    subnormals and normals up to about 1e-36; fp16: subnormals and normals up
    to about 2e-4), a few NaN and +-Inf entries, zeros."""
    top = 0x0400 if dtype == "bf16" else 0x0C00
    bits = rng.integers(0, top, (world, n), dtype=np.uint64).astype(np.uint16)
    bits |= (rng.integers(0, 2, (world, n)).astype(np.uint16) << 15)
    inf, qnan, snan = (0x7F80, 0x7FC0, 0x7F81) if dtype == "bf16" else (0x7C00, 0x7E00, 0x7C01)
    for r in range(world):
        k = rng.integers(0, n, max(1, n // 500))
        bits[r, k[0::4]] = inf
        bits[r, k[1::4]] = inf | 0x8000
        bits[r, k[2::4]] = qnan
        bits[r, k[3::4]] = snan
    return bits


def oracle_run(rows_by_step, dtype16, pdt, theta, m0, v0, lr, betas=(0.9, 0.999), eps=1e-8):
    master, m, v = theta.copy(), m0.copy(), v0.copy()
    with np.errstate(all="ignore"):
        for t, rows in enumerate(rows_by_step, start=1):
            g = nm.reduce_rank_order([nm.widen16(r, dtype16) for r in rows])
            master, m, v = nm.adam_update(master, m, v, g, nm.adam_consts(lr, *betas, eps, t))
        return master, m, v, nm.cast16(master, pdt)


@pytest.mark.parametrize("lr,betas,eps", [(1e-3, (0.9, 0.999), 1e-8), (1e-2, (0.8, 0.95), 0.0),
                                          (3e-4, (0.9, 0.999), 1e-30)])
def test_adam_step_subnormal_tiny_and_nonfinite(lr, betas, eps):
    """zero_adam_step with fp32 gradients from 1e-45 to 1e-30, NaN and +-Inf,
    m and v seeded subnormal, 4 steps; eps = 0 and eps = 1e-30 put the
    subnormal square roots themselves in the denominator."""
    rng = np.random.default_rng(int(lr * 1e6))
    n = 512 * 37 + 11                                  # whole tiles and a ragged tail
    theta = (rng.normal(0, 0.02, n)).astype(np.float32)
    m0, v0 = subnormal_f32(rng, n), np.abs(subnormal_f32(rng, n))
    zero = rng.integers(0, n, n // 50)                 # zero gradient and zero moments here
    m0[zero] = 0
    v0[zero] = 0
    gs = []
    mb = torch.from_numpy(theta.copy()).cuda()
    mm, vb = torch.from_numpy(m0.copy()).cuda(), torch.from_numpy(v0.copy()).cuda()
    master, m, v = theta.copy(), m0.copy(), v0.copy()
    with np.errstate(all="ignore"):
        for t in range(1, 5):
            g = special_f32(rng, n)
            g[zero] = 0
            gs.append(g)
            z.zero_adam_step(mb, mm, vb, torch.from_numpy(g).cuda(), n, t, lr, betas, eps)
            master, m, v = nm.adam_update(master, m, v, g, nm.adam_consts(lr, *betas, eps, t))
    torch.cuda.synchronize()
    nans = same_f32(host32(mb), master, "master")
    same_f32(host32(mm), m, "m")
    same_f32(host32(vb), v, "v")
    # a zero gradient with zero moments leaves the master exactly as it was
    # (with eps = 0 the update there is 0/0: NaN on both sides, as checked)
    if eps > 0:
        assert np.array_equal(host32(mb)[zero].view(np.uint32), theta[zero].view(np.uint32))
    say(f"[edge adam] lr={lr} eps={eps}: bit-exact, {nans} NaN masters")
    sub = np.abs(m) < np.float32(2.0 ** -126)
    assert (sub & (m != 0)).any(), "no subnormal m survived: the case tests nothing"


KERNELS = {
    # name: (launch shape (defer tiles, min rows), write window, rows, fp32 element shift)
    "scalar": ((3, 24), None, 5, 1),
    "direct": ((0, 24), None, 12, 0),
    "deferred": ((3, 1), (0, 0, 0, 0), 12, 0),
    "deferred_windowed": ((3, 1), None, 24, 0),
}


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("kernel", list(KERNELS))
def test_fused_step_edge_values(kernel, dtype):
    """The fused step on 16-bit gradients around the format's smallest
    normal, with NaN and +-Inf entries, on subnormal m and v, 3 steps, in
    each kernel."""
    (defer, min_rows), window, world, shift = KERNELS[kernel]
    rng = np.random.default_rng(7 + len(kernel))
    n = 512 * 64 + 77
    stride = (n + 63) // 64 * 64
    say(f"[edge fused] kernel={kernel} dtype={dtype} rows={world}")
    z.zsmr_set_launch_shape(0, 0, defer, min_rows)
    if window is not None:
        z.zsmr_set_write_window(*window)
    try:
        ctx = z.zero_init_shards(n * world, world, 2, dtype)
        theta = rng.normal(0, 0.02, n).astype(np.float32)
        m0, v0 = subnormal_f32(rng, n), np.abs(subnormal_f32(rng, n))
        quiet = rng.integers(0, n, n // 50)             # zero gradient in every row, zero moments
        m0[quiet] = 0
        v0[quiet] = 0
        mk = lambda x: torch.from_numpy(np.concatenate([np.zeros(shift, np.float32), x])).cuda()
        th, mb, mm, vb = mk(theta), mk(theta), mk(m0), mk(v0)
        pb = torch.zeros(n, dtype=TDT[dtype], device="cuda")
        s = shift
        z.zero_init_state(ctx, 0, 0, th[s:], mb[s:], torch.empty_like(mm)[s:], torch.empty_like(vb)[s:],
                          pb)
        rows_by_step = []
        for t in range(1, 4):
            rows = special_rows16(rng, world, n, dtype)
            rows[:, quiet] = 0
            rows_by_step.append(rows)
            buf = np.zeros((world, stride), np.uint16)
            buf[:, :n] = rows
            G = dev16(buf.ravel())
            plan = z.zsmr_fused_step_plan(ctx, 0, 0, G, stride, 0, mb[s:], mm[s:], vb[s:], pb)
            assert plan["kernel"] == kernel.split("_")[0], plan
            assert bool(plan["windowed"]) == (kernel == "deferred_windowed"), plan
            z.zero_fused_step(ctx, 0, 0, G, stride, 0, mb[s:], mm[s:], vb[s:], pb, t, 1e-3)
        torch.cuda.synchronize()
    finally:
        z.zsmr_set_launch_shape()
        z.zsmr_set_write_window()
    master, m, v, p16 = oracle_run(rows_by_step, dtype, dtype, theta, m0, v0, 1e-3)
    nans = same_f32(host32(mb)[s:], master, "master")
    same_f32(host32(mm)[s:], m, "m")
    same_f32(host32(vb)[s:], v, "v")
    same_16(host16(pb), p16, dtype, "working copy")
    assert np.array_equal(host32(mb)[s:][quiet].view(np.uint32), theta[quiet].view(np.uint32))
    assert 0 < nans < n, "the case should mix NaN and finite results"
    say(f"[edge fused] kernel={kernel} dtype={dtype}: bit-exact, {nans} NaN masters of {n}")


def test_reduce_of_subnormal_rows_is_exact():
    """The reduce alone on bf16 and fp16 rows of subnormals and tiny normals
    (sums that stay subnormal, cross into the normal range, and cancel), sum
    and mean, 16 and 12 ranks (the mean multiplies by 1/16, divides by 12)."""
    rng = np.random.default_rng(3)
    n = 10_003
    for dtype in ("bf16", "fp16"):
        for world in (16, 12):
            ctx = z.zero_init_shards(n * world, world, 2, dtype)
            top = 0x0100 if dtype == "bf16" else 0x0500
            rows = rng.integers(0, top, (world, n), dtype=np.uint64).astype(np.uint16)
            rows |= rng.integers(0, 2, (world, n)).astype(np.uint16) << 15
            G = dev16(rows.ravel())
            out = torch.empty(n, dtype=torch.float32, device="cuda")
            for mean in (False, True):
                z.zero_reduce_shard(ctx, 0, 0, G, n, 0, mean, out)
                torch.cuda.synchronize()
                want = nm.reduce_rank_order([nm.widen16(r, dtype) for r in rows], mean=mean)
                same_f32(host32(out), want, f"reduce {dtype} N={world} mean={mean}")
                if dtype == "bf16":
                    # bf16 shares fp32's exponent range: sums and means of
                    # these rows include fp32 subnormals
                    assert (np.abs(want[want != 0]) < np.float32(2.0 ** -126)).any()
                else:
                    # fp16 subnormals are normal fp32 values: the case is the
                    # exact widening of fp16 subnormal inputs
                    assert ((rows & 0x7C00) == 0).any() and ((rows & 0x03FF) != 0).any()
