"""Shared helpers of the GPU tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np
import torch

import zero_sharded_mixed_reduce_amd as z
from tests.progress import say  # noqa: F401  (the GPU tests import it from here)

REL_TOL = 1e-5      # fp32 master/m/v: max relative error against the oracle
ULP_TOL = 1         # 16-bit working copy: max distance in units in the last place


def dev16(bits: np.ndarray) -> torch.Tensor:
    """16-bit patterns to a device int16 tensor (the library reads raw bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()


def host16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host32(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def ordered16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def compare(got_f32: dict, want_f32: dict, got16: np.ndarray, want16: np.ndarray, what: str):
    """Assert the acceptance bar and return exactness statistics."""
    stats = {}
    for k in want_f32:
        g = np.asarray(got_f32[k], dtype=np.float32)
        w = np.asarray(want_f32[k], dtype=np.float32)
        assert g.shape == w.shape, (what, k, g.shape, w.shape)
        rel = np.abs(g.astype(np.float64) - w) / np.maximum(np.abs(w.astype(np.float64)), 2.0 ** -126)
        assert np.all(np.isfinite(g)), (what, k)
        mx = float(rel.max()) if rel.size else 0.0
        assert mx <= REL_TOL, f"{what} {k}: max rel err {mx:.3g}"
        stats[k] = (mx, int(np.count_nonzero(g.view(np.uint32) != w.view(np.uint32))))
    d = np.abs(ordered16(got16) - ordered16(want16))
    mx16 = int(d.max()) if d.size else 0
    assert mx16 <= ULP_TOL, f"{what} working copy: max {mx16} ulp"
    stats["p16"] = (mx16, int(np.count_nonzero(got16 != want16)))
    say(f"[parity] {what}: " + ", ".join(f"{k} max={v[0]:.3g} differing={v[1]}" for k, v in stats.items()))
    return stats


def param_map(ctx, units=None) -> np.ndarray:
    """Padded position -> parameter index (-1 for pad), built from the
    library's own index map (zero_layout) and the true unit sizes."""
    info = ctx.info()
    P, numel, world, stage = info["padded_numel"], info["numel"], info["world"], info["stage"]
    out = np.full(P, -1, dtype=np.int64)
    if stage in (0, 1, 2):
        out[:numel] = np.arange(numel)
        return out
    units = list(units) if units else [numel]
    p_start = 0
    for u, size in enumerate(units):
        q0, su, _ = z.zero_layout(ctx, 0, u)
        k = np.arange(world * su, dtype=np.int64)
        out[q0:q0 + world * su] = np.where(k < size, p_start + k, -1)
        p_start += size
    return out
