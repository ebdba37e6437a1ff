"""The seeded input generator: its definition, distributions and pad rule."""
import numpy as np
import pytest

import synth

MASK = (1 << 64) - 1


def splitmix64_int(x: int) -> int:
    # SplitMix64 (Steele, Lea, Flood 2014) in Python integers
    z = (x + 0x9E3779B97F4A7C15) & MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def test_splitmix64_vectorised_matches_integer_definition():
    rng = np.random.default_rng(0)
    xs = rng.integers(0, 1 << 63, 1000, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    xs = np.concatenate([xs, np.array([0, 1, MASK, 1 << 63], dtype=np.uint64)])
    got = synth.splitmix64(xs)
    for x, y in zip(xs.tolist(), got.tolist()):
        assert y == splitmix64_int(x)


def test_normal_is_integer_irwin_hall_times_sigma():
    p = np.arange(0, 4000, 7)
    key = synth.stream_key(0, synth.TAG_GRAD, 3, 2)
    x = synth.normal_f32(0, synth.TAG_GRAD, 3, 2, p, 1e-3)
    for i, pi in enumerate(p[:50].tolist()):
        s = 0
        for j in range(3):
            d = splitmix64_int((key + 4 * pi + j) & MASK)
            s += sum((d >> (16 * q)) & 0xFFFF for q in range(4))
        z = np.float32(s - 393210) * np.float32(2.0 ** -16)
        assert x[i] == np.float32(z * np.float32(1e-3))


def test_distribution_and_outliers():
    p = np.arange(1 << 20)
    x = synth.normal_f32(0, synth.TAG_GRAD, 0, 1, p, 1e-3)
    assert abs(x.mean()) < 1e-5 and abs(x.std() - 1e-3) < 2e-5
    assert np.abs(x).max() <= 6e-3
    y = synth.normal_f32(0, synth.TAG_GRAD, 0, 1, p, 1e-3, outlier_permyriad=100)
    hit = y != x
    assert 0.009 < hit.mean() < 0.011
    assert np.array_equal(y[hit], x[hit] * np.float32(100))
    # different streams differ; the same stream repeats
    z = synth.normal_f32(0, synth.TAG_GRAD, 1, 1, p[:1000], 1e-3)
    assert not np.array_equal(z, x[:1000])
    assert np.array_equal(synth.normal_f32(0, synth.TAG_GRAD, 0, 1, p[:1000], 1e-3), x[:1000])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_trunc16_truncates_toward_zero(dtype):
    x = synth.normal_f32(0, synth.TAG_GRAD, 0, 1, np.arange(1 << 18), 1e-2)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, -1.0, 6e-8, 3e-5, 65504.0, 1e5])])
    h = synth.trunc16(x, dtype)
    if dtype == "bf16":
        v = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        up = ((h.astype(np.uint32) + 1) << 16).view(np.float32).astype(np.float64)
    else:
        v = h.view(np.float16).astype(np.float64)
        up = (h + np.uint16(1)).view(np.float16).astype(np.float64)
    ax = np.abs(x.astype(np.float64))
    assert np.all(np.abs(v) <= ax)
    fin = ax < 65504
    assert np.all(np.abs(up[fin]) > ax[fin])


def test_fill_rows_pad_rule():
    a = synth.fill_rows16(0, synth.TAG_GRAD, 5, 3, 2, 100, 40, 33, 1e-3, "bf16")
    assert a.shape == (3, 40) and not a[:, 33:].any()
    for r in range(3):
        assert np.array_equal(a[r, :33], synth.grad16(0, 5 + r, 2, np.arange(100, 133), 1e-3, "bf16"))
    f = synth.fill_f32(0, synth.TAG_THETA, 0, 0, 10, 20, 15, 0.02)
    assert not f[15:].any() and np.array_equal(f[:15], synth.theta0(0, np.arange(10, 25)))
