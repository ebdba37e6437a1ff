"""The oracle's fp32 -> 16-bit cast on every one of the 2^32 fp32 bit
patterns, against torch's CPU casts (a library routine that rounds to nearest
even): the same 16 bits for every non-NaN input, and a NaN for every NaN
input.  The sweep runs in 256 slices of 2^24 patterns (one per value of the
top byte) over a pool of spawned worker processes."""
import multiprocessing as mp
import os

import numpy as np
import pytest

SLICE_BITS = 24


def _check_slice(args):
    """(dtype, top byte) -> number of patterns that disagree."""
    import torch
    from oracle import numerics as nm
    dtype, top = args
    torch.set_num_threads(1)
    bits = np.arange(1 << SLICE_BITS, dtype=np.uint32) | np.uint32(top << SLICE_BITS)
    x = bits.view(np.float32)
    ours = nm.cast16(x, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    ref = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    bad = int(np.count_nonzero(ours[~nan] != ref[~nan]))
    back = nm.widen16(ours[nan], dtype)
    bad += int(np.count_nonzero(~np.isnan(back)))
    return bad


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_cast16_on_every_fp32_pattern(dtype):
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")       # no fork of a process that holds thread pools
    with ctx.Pool(workers) as pool:
        bad = pool.map(_check_slice, [(dtype, top) for top in range(256)], chunksize=4)
    assert sum(bad) == 0, [(top, b) for top, b in enumerate(bad) if b]
