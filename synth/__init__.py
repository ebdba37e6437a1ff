"""Seeded synthetic inputs for the ZeRO shard step: the fp32 initial parameters
and the per-rank 16-bit gradients (and the staged peer slices of a single-rank
run).

This module is shared by the CPU oracle's tests, the GPU tests and the
benchmark.  It holds none of the method's arithmetic: no reduction, no Adam and
no fp32 -> 16-bit round-to-nearest cast.  It only answers "what is the input
value at parameter index p for (tag, rank, step)".  The GPU fill kernels in
``synth/synth_fill.hip`` implement the same definition and are tested against
this file bit for bit.

Definition (every step is integer arithmetic up to one or two IEEE fp32
multiplies, so any element can be regenerated on its own and both sides agree
exactly):

* ``splitmix64(x)``: the public-domain SplitMix64 output function of Steele,
  Lea and Flood (OOPSLA 2014): add the golden-ratio increment
  0x9E3779B97F4A7C15, then the variant-13 finaliser (xor-shift 30, multiply
  0xBF58476D1CE4E5B9, xor-shift 27, multiply 0x94D049BB133111EB, xor-shift 31),
  all modulo 2**64.
* stream key ``k = splitmix64(seed ^ tag<<56 ^ rank<<40 ^ step<<32)`` with
  ``seed`` < 2**32, ``step`` < 256, ``rank`` < 65536.
* for parameter index ``p`` the draws are ``d_j = splitmix64(k + 4p + j)``,
  j = 0..3.  d_0..d_2 give twelve 16-bit integers u_0..u_11; their sum ``s``
  minus 393210 (the exact mean of the sum) over 65536 is an Irwin-Hall(12)
  approximation of a standard normal, exact in fp32, truncated at +-6.
* value ``x = fl32(z * fl32(sigma))``.  With outliers enabled (the 1.5B
  workload: one entry in a hundred scaled by 100) the entry is an outlier iff
  ``d_3 mod 10000 < outlier_permyriad`` and then ``x = fl32(x * 100)``.
* 16-bit inputs are the fp32 value **truncated** toward zero (bf16: the upper
  16 bits; fp16: exponent re-biased, mantissa shifted right, subnormals by the
  same shift, no overflow at these magnitudes).  Truncation is a property of
  the input recipe, chosen so that the generator shares no rounding code with
  either side of the method's cast.

Distributions follow the workloads: theta0 ~ N(0, 0.02) in fp32, gradients
~ N(0, 1e-2) (fp16) or N(0, 1e-3) (bf16); sigma is the standard deviation.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TAG_THETA = 1
TAG_GRAD = 2
TAG_PEER = 3

BF16 = "bf16"
FP16 = "fp16"

_IH_MEAN = 393210          # 12 * 65535 / 2, the exact mean of the 12-draw sum
_CHUNK = 1 << 22


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(x) -> np.ndarray:
    """SplitMix64 output for state ``x`` (uint64 array or scalar), mod 2**64."""
    with np.errstate(over="ignore"):
        return _mix64(np.asarray(x, dtype=np.uint64) + GAMMA)


def stream_key(seed: int, tag: int, rank: int, step: int) -> int:
    if not (0 <= seed < 1 << 32 and 0 <= step < 256 and 0 <= rank < 1 << 16 and 0 <= tag < 256):
        raise ValueError("seed/tag/rank/step out of range")
    x = seed ^ (tag << 56) ^ (rank << 40) ^ (step << 32)
    return int(splitmix64(np.uint64(x)))


def _normal_chunk(key: int, p: np.ndarray, sigma: float, outlier_permyriad: int) -> np.ndarray:
    with np.errstate(over="ignore"):
        base = np.uint64(key) + p.astype(np.uint64) * np.uint64(4)
        s = np.zeros(p.shape, dtype=np.int64)
        mask16 = np.uint64(0xFFFF)
        for j in range(3):
            d = splitmix64(base + np.uint64(j))
            for q in range(4):
                s += ((d >> np.uint64(16 * q)) & mask16).astype(np.int64)
        z = (s - _IH_MEAN).astype(np.float32) * np.float32(2.0 ** -16)   # exact
        x = z * np.float32(sigma)                                          # one rounding
        if outlier_permyriad:
            d3 = splitmix64(base + np.uint64(3))
            hit = (d3 % np.uint64(10000)) < np.uint64(outlier_permyriad)
            x = np.where(hit, x * np.float32(100.0), x).astype(np.float32)
    return x


def normal_f32(seed: int, tag: int, rank: int, step: int, p, sigma: float,
               outlier_permyriad: int = 0) -> np.ndarray:
    """fp32 samples at parameter indices ``p`` (int array) for one stream."""
    p = np.asarray(p, dtype=np.int64).ravel()
    key = stream_key(seed, tag, rank, step)
    out = np.empty(p.shape, dtype=np.float32)
    for lo in range(0, p.size, _CHUNK):
        out[lo:lo + _CHUNK] = _normal_chunk(key, p[lo:lo + _CHUNK], sigma, outlier_permyriad)
    return out


def trunc16(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> 16-bit pattern by truncation toward zero (input encoding only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if dtype == BF16:
        return (u >> np.uint32(16)).astype(np.uint16)
    if dtype != FP16:
        raise ValueError(dtype)
    sign = ((u >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint32)
    e = ((u >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64)
    mant = (u & np.uint32(0x7FFFFF)).astype(np.int64)
    big = e - 127 + 15
    normal = (sign | (np.clip(big, 0, 30).astype(np.uint32) << np.uint32(10))
              | (mant >> 13).astype(np.uint32))
    sh = np.clip(126 - e, 0, 63)
    sub = sign | np.where(sh < 32, (mant | 0x800000) >> sh, 0).astype(np.uint32)
    h = np.where(big >= 31, sign | np.uint32(0x7BFF),
                 np.where(big >= 1, normal, np.where(e == 0, sign, sub)))
    return h.astype(np.uint16)


def theta0(seed: int, p, sigma: float = 0.02) -> np.ndarray:
    """Initial fp32 parameters at parameter indices ``p``."""
    return normal_f32(seed, TAG_THETA, 0, 0, p, sigma)


def grad16(seed: int, rank: int, step: int, p, sigma: float, dtype: str,
           outlier_permyriad: int = 0) -> np.ndarray:
    """16-bit gradient of ``rank`` at Adam step ``step`` for parameter indices ``p``."""
    return trunc16(normal_f32(seed, TAG_GRAD, rank, step, p, sigma, outlier_permyriad), dtype)


def peer16(seed: int, p, dtype: str, sigma: float = 0.02) -> np.ndarray:
    """Staged 16-bit peer values (what other ranks' all-gather would deliver)."""
    return trunc16(normal_f32(seed, TAG_PEER, 0, 0, p, sigma), dtype)


def fill_rows16(seed: int, tag: int, rank0: int, rows: int, step: int, p0: int, n: int,
                p_valid: int, sigma: float, dtype: str, outlier_permyriad: int = 0) -> np.ndarray:
    """[rows, n] uint16: row r, column k holds the value for rank ``rank0+r`` at
    parameter ``p0+k`` if ``k < p_valid`` and zero otherwise (the pad).  Same
    contract as the GPU fill entry point ``zsmr_synth_fill16``."""
    out = np.zeros((rows, n), dtype=np.uint16)
    k = np.arange(min(n, max(p_valid, 0)), dtype=np.int64)
    for r in range(rows):
        out[r, :k.size] = trunc16(normal_f32(seed, tag, rank0 + r, step, p0 + k, sigma,
                                             outlier_permyriad), dtype)
    return out


def fill_f32(seed: int, tag: int, rank: int, step: int, p0: int, n: int, p_valid: int,
             sigma: float) -> np.ndarray:
    """[n] fp32 with the same pad rule as ``fill_rows16`` (GPU: ``zsmr_synth_fill32``)."""
    out = np.zeros(n, dtype=np.float32)
    k = np.arange(min(n, max(p_valid, 0)), dtype=np.int64)
    out[:k.size] = normal_f32(seed, tag, rank, step, p0 + k, sigma)
    return out
