"""The pure-read and pure-write reference streams the benchmark times beside
the shard step: the write stream stores its value into exactly the bytes it
is given, in every shape, and the read stream leaves every buffer as it was."""
import pytest
import torch

import ceiling
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

# element counts (int32 words): empty, one vector, ragged tails around one
# 32 KB burst and one 8 KB region burst, several bursts plus a tail
SIZES = [0, 4, 2044, 2048, 2052, 8192 * 3 + 4, 65536 * 5 + 12, (1 << 22) + 36]


@pytest.mark.parametrize("shape", [ceiling.BURSTS, ceiling.PLAIN, ceiling.BURSTS_BALANCED,
                                   ceiling.PLAIN_BALANCED])
@pytest.mark.parametrize("words", SIZES)
def test_write_covers_exactly_its_bytes(words, shape):
    say(f"[ceiling] write words={words} shape={shape}")
    guard = 4096
    buf = torch.full((words + 2 * guard,), -1, dtype=torch.int32, device="cuda")
    body = buf[guard:guard + words]
    ceiling.write(body, 4 * words, shape, 0x12345678)
    torch.cuda.synchronize()
    assert bool((body == 0x12345678).all())
    assert bool((buf[:guard] == -1).all()) and bool((buf[guard + words:] == -1).all())


@pytest.mark.parametrize("shape", [ceiling.BURSTS, ceiling.REGIONS, ceiling.BURSTS_BALANCED])
@pytest.mark.parametrize("words", SIZES)
def test_read_changes_nothing(words, shape):
    say(f"[ceiling] read words={words} shape={shape}")
    src = torch.arange(words, dtype=torch.int32, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    before = src.clone()
    ceiling.read(src, 4 * words, shape, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, before)
    assert sink.tolist() == [7, 7, 7, 7]      # the XOR of 0..n-1 never matches the fixed value


@pytest.mark.parametrize("permille", [500, 1000, 2000])
def test_balanced_write_covers_exactly_its_bytes_at_any_weight(permille):
    """Every chunk block is written once whatever the XCDs' weights."""
    words = (1 << 22) + 36
    say(f"[ceiling] balanced write permille={permille}")
    ceiling.set_balance(permille)
    try:
        guard = 4096
        buf = torch.full((words + 2 * guard,), -1, dtype=torch.int32, device="cuda")
        body = buf[guard:guard + words]
        ceiling.write(body, 4 * words, ceiling.PLAIN_BALANCED, 0x0BADCAFE)
        torch.cuda.synchronize()
        assert bool((body == 0x0BADCAFE).all())
        assert bool((buf[:guard] == -1).all()) and bool((buf[guard + words:] == -1).all())
    finally:
        ceiling.set_balance(1200)


def test_measure_reports_both_directions():
    say("[ceiling] measure 256 MiB")
    buf = torch.empty(1 << 26, dtype=torch.int32, device="cuda")
    out = ceiling.measure(buf, 1 << 28, reps=2)
    assert set(out["read"]) == set(ceiling.READ_SHAPES) and set(out["write"]) == set(ceiling.WRITE_SHAPES)
    assert out["read_GBps"] > 0 and out["write_GBps"] > 0
