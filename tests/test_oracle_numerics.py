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


def test_sharded_adam_on_a_small_mlp_matches_torch_adam():
    """The experiment "ZeRO and FSDP" runs with zero_check.py, re-done with
    the oracle: a two-layer perceptron with 64 inputs, 256 GELU units and 10
    outputs (Psi = 19,210 parameters) on a 32-sample batch; 4 ranks each take
    a quarter of the batch, the rank-order mean of their gradients drives
    Adam on zero-padded shards of ceil(Psi / 4) = 4,803 elements, and after 3
    steps every parameter is within 1e-5 of torch.optim.Adam run on the
    whole batch; each rank then holds 57,636 bytes of optimizer state (the
    page prints both).  The weights, data and labels are this test's own
    seeded draws: the check holds for any."""
    gen = torch.Generator().manual_seed(2024)
    shapes = [(256, 64), (256,), (10, 256), (10,)]
    start = [(torch.rand(sh, generator=gen) * 2 - 1) * (1.0 / sh[-1] ** 0.5) for sh in shapes]
    inputs = torch.randn(32, 64, generator=gen)
    targets = torch.randint(0, 10, (32,), generator=gen)
    sizes = [int(np.prod(sh)) for sh in shapes]
    numel, world, steps, lr = sum(sizes), 4, 3, 1e-2

    def grads_of(flat, rows):
        """fp32 gradient, as one flat vector, of the mean cross-entropy over
        the batch rows `rows` at parameters `flat`."""
        parts = torch.from_numpy(flat[:numel].copy()).split(sizes)
        ps = [t.reshape(sh).requires_grad_(True) for t, sh in zip(parts, shapes)]
        hidden = torch.nn.functional.gelu(inputs[rows] @ ps[0].T + ps[1])
        loss = torch.nn.functional.cross_entropy(hidden @ ps[2].T + ps[3], targets[rows])
        return torch.cat([g.reshape(-1) for g in torch.autograd.grad(loss, ps)]).numpy()

    # torch.optim.Adam on the whole batch
    ref = [t.clone().requires_grad_(True) for t in start]
    adam = torch.optim.Adam(ref, lr=lr, betas=(0.9, 0.999), eps=1e-8, foreach=False)
    for _ in range(steps):
        flat_now = torch.cat([t.detach().reshape(-1) for t in ref]).numpy()
        g_all = torch.from_numpy(grads_of(flat_now, slice(0, 32))).split(sizes)
        for t, g in zip(ref, g_all):
            t.grad = g.reshape(t.shape).clone()
        adam.step()
    want = torch.cat([t.detach().reshape(-1) for t in ref]).numpy()

    # the oracle: padded shards, one per rank, each rank a quarter of the batch
    lay = make_layout(numel, world, 1, pad=True)
    assert numel == 19210 and lay.shard_u == (4803,) and acc.optimizer_state_bytes(lay) == 57636
    flat = np.zeros(lay.padded_numel, np.float32)
    flat[:numel] = torch.cat([t.reshape(-1) for t in start]).numpy()
    state = []
    for r in range(world):
        off, n = lay.owned(r)
        state.append([flat[off:off + n].copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)])
    for t in range(1, steps + 1):
        rows = []
        for r in range(world):
            g = np.zeros(lay.padded_numel, np.float32)
            g[:numel] = grads_of(flat, slice(8 * r, 8 * (r + 1)))
            rows.append(g)
        k = nm.adam_consts(lr, 0.9, 0.999, 1e-8, t)
        for r in range(world):
            off, n = lay.owned(r)
            g_r = nm.reduce_rank_order([row[off:off + n] for row in rows])
            state[r] = list(nm.adam_update(state[r][0], state[r][1], state[r][2], g_r, k))
        flat = np.concatenate([st[0] for st in state])
        assert not flat[numel:].any()                          # the pad stays zero
    assert np.max(np.abs(flat[:numel] - want)) < 1e-5
    start_flat = torch.cat([t.reshape(-1) for t in start]).numpy()
    assert np.max(np.abs(want - start_flat)) > 1e-2                  # and the steps moved it
