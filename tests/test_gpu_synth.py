"""The GPU fill kernels of the input generator agree bit for bit with its
NumPy definition (so oracle inputs regenerated on the host are exactly the
GPU run's inputs)."""
import numpy as np
import pytest
import torch

import synth
import synth.gpu as sgpu
from tests.gpu_helpers import host16, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,sigma,outlier", [("bf16", 1e-3, 0), ("bf16", 1e-3, 100),
                                                 ("fp16", 1e-2, 0), ("fp16", 0.02, 0)])
def test_fill16_matches_numpy(dtype, sigma, outlier):
    rows, n, p0, p_valid, stride = 3, 50_001, (1 << 33) + 17, 49_000, 50_008
    say(f"[synth] fill16 {dtype} sigma={sigma} outlier={outlier}")
    buf = torch.full((rows * stride,), 7, dtype=torch.int16, device="cuda")
    sgpu.fill16(buf, rows, stride, n, p0, p_valid, 0, synth.TAG_GRAD, 5, 3, sigma, dtype, outlier)
    torch.cuda.synchronize()
    got = host16(buf).reshape(rows, stride)
    want = synth.fill_rows16(0, synth.TAG_GRAD, 5, rows, 3, p0, n, p_valid, sigma, dtype, outlier)
    assert np.array_equal(got[:, :n], want)
    assert np.all(got[:, n:] == 7)                 # nothing written past n


def test_fill32_matches_numpy():
    n, p0, p_valid = 100_003, 7_499_999_000, 99_000
    buf = torch.full((n + 5,), -1.0, dtype=torch.float32, device="cuda")
    sgpu.fill32(buf, n, p0, p_valid, 0, synth.TAG_THETA, 0, 0, 0.02)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    want = synth.fill_f32(0, synth.TAG_THETA, 0, 0, p0, n, p_valid, 0.02)
    assert np.array_equal(got[:n].view(np.uint32), want.view(np.uint32))
    assert np.all(got[n:] == -1.0)


def test_peer_values():
    n = 4096
    buf = torch.empty(n, dtype=torch.int16, device="cuda")
    sgpu.fill16(buf, 1, n, n, 123_456_789, n, 0, synth.TAG_PEER, 0, 0, 0.02, "bf16")
    torch.cuda.synchronize()
    assert np.array_equal(host16(buf), synth.peer16(0, np.arange(123_456_789, 123_456_789 + n), "bf16"))
