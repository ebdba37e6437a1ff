"""Elementwise arithmetic of the ZeRO shard step, in plain NumPy fp32.

Test infrastructure only (see the package header).  Each function is one step
of the pages' method, written out with one NumPy operation per rounding.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BF16 = "bf16"
FP16 = "fp16"


def widen16(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit pattern -> fp32 value.  Exact for both formats: bf16 is the upper
    half of an fp32 word, and every fp16 value (subnormals included) is an fp32
    value."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == FP16:
        return bits.view(np.float16).astype(np.float32)
    raise ValueError(dtype)


def reduce_rank_order(rows, mean: bool = True) -> np.ndarray:
    """The arithmetic of the gradient reduce-scatter for one owned slice.

    ``rows`` holds one fp32 array per rank (the widened 16-bit contributions).
    The sum is accumulated in fp32 strictly in rank order 0, 1, ..., N-1 (one
    rounding per addition) and then divided by N: the pages' collectives are
    a mean ("The four schemes", ``reduce_scatter_mean``; "ZeRO and FSDP",
    ``ZeroAdam.step`` sums with the reduce-scatter then divides by the world
    size).  ``mean=False`` returns the raw sum.
    """
    rows = list(rows)
    if not rows:
        raise ValueError("need at least one rank")
    acc = np.array(rows[0], dtype=np.float32, copy=True)
    for r in range(1, len(rows)):
        acc = acc + np.asarray(rows[r], dtype=np.float32)
    if mean:
        acc = acc / np.float32(len(rows))
    return acc


@dataclass(frozen=True)
class AdamConsts:
    c1: np.float32      # beta1
    c1m: np.float32     # 1 - beta1
    c2: np.float32      # beta2
    c2m: np.float32     # 1 - beta2
    bc1: np.float32     # 1 - beta1**t
    bc2: np.float32     # 1 - beta2**t
    lr: np.float32
    eps: np.float32


def adam_consts(lr: float, b1: float, b2: float, eps: float, t: int) -> AdamConsts:
    """Scalar constants of one Adam step.

    The pages' prototype writes them as Python (double) expressions that
    multiply or divide fp32 arrays ("The four schemes", ``Base._adam``), so
    each is evaluated in double and rounded to fp32 once at use.  ``t`` counts
    optimizer steps from 1 and is the same for every rank and unit.
    """
    if t < 1:
        raise ValueError("t counts from 1")
    f = np.float32
    return AdamConsts(f(b1), f(1.0 - b1), f(b2), f(1.0 - b2),
                      f(1.0 - b1 ** t), f(1.0 - b2 ** t), f(lr), f(eps))


def adam_update(master: np.ndarray, m: np.ndarray, v: np.ndarray, g: np.ndarray,
                k: AdamConsts):
    """Mixed-precision Adam on an owned slice; returns new (master, m, v).

    In the prototype's order ("The four schemes", ``Base._adam``; the same
    update as ``ZeroAdam.step`` in "ZeRO and FSDP"):
        m  = b1*m + (1-b1)*g
        v  = b2*v + ((1-b2)*g)*g
        mh = m / (1-b1^t),   vh = v / (1-b2^t)
        master = master - (lr*mh) / (sqrt(vh) + eps)
    every operation rounded to fp32.
    """
    g = np.asarray(g, dtype=np.float32)
    m = k.c1 * m + k.c1m * g
    v = k.c2 * v + (k.c2m * g) * g
    mh = m / k.bc1
    vh = v / k.bc2
    d = np.sqrt(vh) + k.eps
    u = (k.lr * mh) / d
    master = master - u
    return master.astype(np.float32), m.astype(np.float32), v.astype(np.float32)


def cast16(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> 16-bit working copy, round to nearest with ties to even.

    The prototype's cast of the master into the 16-bit copy is NumPy's
    ``astype(float16)`` ("The four schemes", ``Base.__init__`` and the schemes'
    ``step``), which rounds to nearest even and overflows to infinity; bf16 is
    treated the same way.  NaN maps to a quiet NaN of the same sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == FP16:
        with np.errstate(over="ignore", invalid="ignore"):
            return x.astype(np.float16).view(np.uint16)
    if dtype != BF16:
        raise ValueError(dtype)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    quiet = (u >> np.uint64(16)) | np.uint64(0x0040)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)
