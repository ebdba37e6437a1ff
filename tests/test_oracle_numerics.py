"""Pins of the oracle's elementwise arithmetic against things other than itself:
torch's casts (library routines), exact rational sums (brute force), closed
forms of Adam, torch.optim.Adam (the check "ZeRO and FSDP" runs in
zero_check.py) and that page's own sharded-vs-unsharded experiment."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import numerics as nm
from oracle.layout import make_layout
from oracle import accounting as acc


# ---------------------------------------------------------------- casts -----

def _structured_f32_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1FFF, 0x2000, 0x2001, 0x3FFF,
                     0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xC000, 0xE000, 0xF000, 0xFFFF,
                     0x6000, 0x5FFF, 0x4000, 0x4001], dtype=np.uint32)
    rng = np.random.default_rng(3)
    lows = np.concatenate([lows, rng.integers(0, 1 << 16, 12, dtype=np.uint32)])
    pat = (hi[:, None] | lows[None, :]).ravel()
    rand = rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([pat, rand]).view(np.float32)


@pytest.mark.parametrize("dtype,tdtype", [("bf16", torch.bfloat16), ("fp16", torch.float16)])
def test_cast16_matches_torch_rne(dtype, tdtype):
    x = _structured_f32_patterns()
    ours = nm.cast16(x, dtype)
    ref = torch.from_numpy(x.copy()).to(tdtype).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    back = nm.widen16(ours[nan], dtype)
    assert np.all(np.isnan(back))


def test_cast16_ties_go_to_even():
    # 1 + 2^-8 is halfway between two bf16 values: ties to the even one (1.0)
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11], np.float32)
    b = nm.widen16(nm.cast16(x[:2], "bf16"), "bf16")
    h = nm.widen16(nm.cast16(x[2:], "fp16"), "fp16")
    assert b.tolist() == [1.0, 1 + 4 * 2.0 ** -8] and h.tolist() == [1.0, 1 + 4 * 2.0 ** -11]


@pytest.mark.parametrize("dtype,tdtype", [("bf16", torch.bfloat16), ("fp16", torch.float16)])
def test_widen16_all_patterns(dtype, tdtype):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = nm.widen16(bits, dtype)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(tdtype).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# --------------------------------------------------------------- reduce -----

def test_reduce_brute_force_error_bound():
    rng = np.random.default_rng(11)
    for world in (1, 2, 3, 4, 8, 16, 64):
        rows16 = [rng.integers(0, 1 << 16, 257, dtype=np.uint32).astype(np.uint16) for _ in range(world)]
        rows16 = [np.where(np.isfinite(nm.widen16(r, "bf16")), r, 0).astype(np.uint16) for r in rows16]
        rows = [nm.widen16(r, "bf16") for r in rows16]
        with np.errstate(over="ignore"):
            got = nm.reduce_rank_order(rows, mean=False)
        for j in range(0, 257, 16):
            vals = [Fraction(float(r[j])) for r in rows]
            exact = sum(vals)
            bound = Fraction(world - 1) * Fraction(2) ** -24 * sum(abs(v) for v in vals)
            if math.isfinite(float(got[j])):
                assert abs(Fraction(float(got[j])) - exact) <= bound


def test_reduce_is_rank_order_fp32():
    one, tiny = np.float32(1.0), np.float32(2.0 ** -24)
    rows = [np.array([one]), np.array([tiny]), np.array([tiny])]
    # rank order: (1 + 2^-24) rounds to 1, then again -> 1; reversed order would give 1 + 2^-23
    assert nm.reduce_rank_order(rows, mean=False)[0] == one
    assert nm.reduce_rank_order(rows[::-1], mean=False)[0] == np.float32(1 + 2.0 ** -23)
    # fp32 (not 16-bit) accumulation: 1 + 2^-10 survives in fp32, not in bf16
    rows = [np.array([one]), np.array([np.float32(2.0 ** -10)])]
    assert nm.reduce_rank_order(rows, mean=False)[0] == np.float32(1 + 2.0 ** -10)


def test_reduce_special_cases():
    x = np.array([0.5, -3.25, 1e-3, 7.0], np.float32)
    assert np.array_equal(nm.reduce_rank_order([x]), x)                       # N = 1
    assert np.all(nm.reduce_rank_order([x, -x], mean=False) == 0)             # x + (-x)
    got = nm.reduce_rank_order([x, x, x, x])                                   # mean of equal rows
    assert np.array_equal(got, x)


# ----------------------------------------------------------------- Adam -----

HP = dict(lr=1e-2, b1=0.9, b2=0.999, eps=1e-8)


def test_adam_zero_gradient_leaves_master_bit_unchanged():
    rng = np.random.default_rng(0)
    master = rng.normal(0, 0.02, 4096).astype(np.float32)
    m = np.zeros_like(master)
    v = np.zeros_like(master)
    for t in range(1, 6):
        k = nm.adam_consts(HP["lr"], HP["b1"], HP["b2"], HP["eps"], t)
        new, m, v = nm.adam_update(master, m, v, np.zeros_like(master), k)
        assert np.array_equal(new.view(np.uint32), master.view(np.uint32))
    assert not m.any() and not v.any()


def test_adam_first_step_closed_form():
    # t = 1: m_hat = g, v_hat = g^2, so the step is lr * g / (|g| + eps) (eps outside the sqrt)
    g = np.float32(10.0) ** np.linspace(-10, -1, 64).astype(np.float32)
    g = np.concatenate([g, -g]).astype(np.float32)
    master = np.zeros_like(g)
    k = nm.adam_consts(HP["lr"], HP["b1"], HP["b2"], HP["eps"], 1)
    new, m, v = nm.adam_update(master, np.zeros_like(g), np.zeros_like(g), g, k)
    g64 = g.astype(np.float64)
    want = -HP["lr"] * g64 / (np.abs(g64) + HP["eps"])
    assert np.allclose(new, want, rtol=4e-7, atol=0)


def test_adam_constant_gradient_closed_form():
    g = np.array([3e-3, -2e-4, 5e-9, -1e-7, 1.0], np.float32)
    master = np.full_like(g, 0.25)
    m = np.zeros_like(g)
    v = np.zeros_like(g)
    T = 7
    for t in range(1, T + 1):
        k = nm.adam_consts(1e-3, 0.9, 0.999, 1e-8, t)
        master, m, v = nm.adam_update(master, m, v, g, k)
    g64 = g.astype(np.float64)
    want = 0.25 - T * 1e-3 * g64 / (np.abs(g64) + 1e-8)
    assert np.allclose(master.astype(np.float64) - 0.25, want - 0.25, rtol=2e-5, atol=1e-9)


def test_adam_matches_torch_optim_adam():
    # "ZeRO and FSDP" checks its sharded Adam against torch.optim.Adam to 1e-5
    rng = np.random.default_rng(5)
    theta = rng.normal(0, 0.02, 10000).astype(np.float32)
    p = torch.nn.Parameter(torch.from_numpy(theta.copy()))
    opt = torch.optim.Adam([p], lr=1e-2, betas=(0.9, 0.999), eps=1e-8, foreach=False)
    master, m, v = theta.copy(), np.zeros_like(theta), np.zeros_like(theta)
    scale_m = np.zeros_like(theta)
    scale_v = np.zeros_like(theta)
    for t in range(1, 6):
        g = (rng.normal(0, 1e-2, theta.size) * 10.0 ** rng.uniform(-6, 0, theta.size)).astype(np.float32)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        k = nm.adam_consts(1e-2, 0.9, 0.999, 1e-8, t)
        master, m, v = nm.adam_update(master, m, v, g, k)
        scale_m = np.maximum(scale_m, np.maximum(np.abs(m), np.abs(g)))
        scale_v = np.maximum(scale_v, np.maximum(v, g * g))
    ref = p.detach().numpy()
    assert np.max(np.abs(master - ref)) < 1e-5
    st = opt.state[p]
    # torch forms m with lerp, which rounds differently where g and m cancel:
    # compare against the magnitudes that entered the update
    assert np.all(np.abs(m - st["exp_avg"].numpy()) <= 1e-5 * scale_m)
    assert np.all(np.abs(v - st["exp_avg_sq"].numpy()) <= 1e-5 * scale_v)


def test_zero_check_replay():
    """The experiment of "ZeRO and FSDP" (zero_check.py): 4 ranks, each with a
    quarter of a 32-sample batch, reduce-scatter mean + Adam on padded shards,
    against single-process torch.optim.Adam on the full batch: < 1e-5 after
    3 steps, and 57,636 bytes of optimizer state per rank."""
    torch.manual_seed(0)
    ref = torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(), torch.nn.Linear(256, 10))
    torch.manual_seed(0)
    model = torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(), torch.nn.Linear(256, 10))
    torch.manual_seed(123)
    X, Y = torch.randn(32, 64), torch.randint(0, 10, (32,))
    loss_fn = torch.nn.CrossEntropyLoss()
    world = 4
    params = list(model.parameters())
    numel = sum(p.numel() for p in params)
    lay = make_layout(numel, world, 1, pad=True)
    assert numel == 19210 and acc.optimizer_state_bytes(lay) == 57636
    flat = np.zeros(lay.padded_numel, np.float32)
    flat[:numel] = torch.cat([p.detach().flatten() for p in params]).numpy()
    shards = [flat[lay.owned(r)[0]:lay.owned(r)[0] + lay.owned(r)[1]].copy() for r in range(world)]
    ms = [np.zeros_like(s) for s in shards]
    vs = [np.zeros_like(s) for s in shards]
    opt_ref = torch.optim.Adam(ref.parameters(), lr=1e-2, foreach=False)
    for t in range(1, 4):
        opt_ref.zero_grad()
        loss_fn(ref(X), Y).backward()
        opt_ref.step()
        rows = []
        for r in range(world):
            model.zero_grad()
            sl = slice(r * 32 // world, (r + 1) * 32 // world)
            loss_fn(model(X[sl]), Y[sl]).backward()
            g = np.zeros(lay.padded_numel, np.float32)
            g[:numel] = torch.cat([p.grad.flatten() for p in params]).numpy()
            rows.append(g)
        k = nm.adam_consts(1e-2, 0.9, 0.999, 1e-8, t)
        for r in range(world):
            off, n = lay.owned(r)
            gr = nm.reduce_rank_order([row[off:off + n] for row in rows])
            shards[r], ms[r], vs[r] = nm.adam_update(shards[r], ms[r], vs[r], gr, k)
        full = np.concatenate(shards)
        assert not full[numel:].any()                       # the pad stays zero
        off = 0
        with torch.no_grad():
            for p in params:
                p.copy_(torch.from_numpy(full[off:off + p.numel()].reshape(p.shape)))
                off += p.numel()
    diff = max((a - b).abs().max().item() for a, b in zip(ref.parameters(), model.parameters()))
    assert diff < 1e-5
