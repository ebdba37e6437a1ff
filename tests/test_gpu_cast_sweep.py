"""The device cast (fp32 -> 16-bit, round to nearest even) on every one of
the 2^32 fp32 bit patterns, through zero_gather_cast, in 16 launches of 2^28
patterns each.  Every non-NaN pattern must give the 16 bits of torch's CPU
cast, which the CPU suite pins equal to the oracle's cast on all 2^32
patterns.  Every NaN pattern must give a NaN (the pages fix no payload); for
bf16 it must also be the oracle's quiet NaN (the sign and the top payload
bits kept, the quiet bit set), the rule the kernel implements as well."""
import numpy as np
import pytest
import torch

import zero_sharded_mixed_reduce_amd as z
from oracle import numerics as nm
from tests.gpu_helpers import host16, say

pytestmark = pytest.mark.gpu

CHUNK_BITS = 28
TDT = {"bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_device_cast_on_every_fp32_pattern(dtype):
    n = 1 << CHUNK_BITS
    ctx = z.zero_init_shards(n, 1, 2, dtype)
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    base = np.arange(n, dtype=np.uint32)
    for c in range(1 << (32 - CHUNK_BITS)):
        say(f"[cast sweep] {dtype} patterns {c << CHUNK_BITS:#010x}..")
        bits = base | np.uint32(c << CHUNK_BITS)
        x = bits.view(np.float32)
        z.zero_gather_cast(ctx, 0, 0, torch.from_numpy(x).cuda(), out)
        got = host16(out)
        ref = torch.from_numpy(x).to(TDT[dtype]).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(x)
        bad = np.flatnonzero((got != ref) & ~nan)
        assert bad.size == 0, f"{bad.size} patterns differ, first {bits[bad[0]]:#010x}"
        if nan.any():
            assert np.isnan(nm.widen16(got[nan], dtype)).all()
            if dtype == "bf16":
                assert np.array_equal(got[nan], nm.cast16(x[nan], dtype))
    assert z.zero_counters(ctx, 0)["traffic_elems"] == 0     # one rank: no gather traffic
