"""Per-element trajectories at chosen parameter indices.

Test infrastructure only (see the package header).

Every step of the method is elementwise once the rank-order reduce is done, so
the final master, m, v and 16-bit working copy at a parameter index depend
only on theta0 and the N gradients of that index at each step.  This module
regenerates exactly those inputs (``synth``) and applies ``numerics`` to
them, which lets a 10**10-element run be checked at any sample of indices.
That all four schemes give the same per-element result is itself pinned by
the scheme tests ("ZeRO and FSDP": sharded Adam matches full Adam; "The four
schemes": ZeRO-2 is ZeRO-1 with one flag changed).
"""
from __future__ import annotations

import numpy as np

import synth
from . import numerics as nm


def trajectory(p_idx, world: int, steps: int, dtype16: str, grad_sigma: float, lr: float,
               betas=(0.9, 0.999), eps: float = 1e-8, seed: int = 0,
               outlier_permyriad: int = 0, theta_sigma: float = 0.02):
    """(master, m, v, working-copy bits) after ``steps`` steps at ``p_idx``."""
    p_idx = np.asarray(p_idx, dtype=np.int64)
    master = synth.theta0(seed, p_idx, theta_sigma)
    m = np.zeros(p_idx.shape, np.float32)
    v = np.zeros(p_idx.shape, np.float32)
    for t in range(1, steps + 1):
        rows = [nm.widen16(synth.grad16(seed, r, t, p_idx, grad_sigma, dtype16,
                                        outlier_permyriad), dtype16)
                for r in range(world)]
        g = nm.reduce_rank_order(rows)
        k = nm.adam_consts(lr, betas[0], betas[1], eps, t)
        master, m, v = nm.adam_update(master, m, v, g, k)
    return master, m, v, nm.cast16(master, dtype16)
