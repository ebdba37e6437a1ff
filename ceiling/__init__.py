"""ctypes binding of ``ceiling/libzsmr_ceiling.so``: pure-read and pure-write
reference streams over HBM (C ABI in ``include/zsmr_ceiling.h``).

Measurement only.  ``phased_bound`` turns the two pure rates into the least
time a kernel that reads R bytes and writes W bytes can take on the same
device: R / read rate + W / write rate (no time lost turning HBM between
reads and writes).
"""
from __future__ import annotations

import ctypes
import os

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libzsmr_ceiling.so")
BURSTS, REGIONS, PLAIN, BURSTS_BALANCED, PLAIN_BALANCED = 0, 1, 1, 2, 3
READ_SHAPES = {"bursts": BURSTS, "regions": REGIONS, "bursts_balanced": BURSTS_BALANCED}
WRITE_SHAPES = {"bursts_nt": BURSTS, "bursts_plain": PLAIN, "bursts_nt_balanced": BURSTS_BALANCED,
                "bursts_plain_balanced": PLAIN_BALANCED}
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m zero_sharded_mixed_reduce_amd.build`")
        from zero_sharded_mixed_reduce_amd import checked_library
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        _LIB = checked_library(LIB_PATH, {
            "zsmr_ceiling_read": (i32, [vp, i64, i32, vp, vp]),
            "zsmr_ceiling_write": (i32, [vp, i64, i32, ctypes.c_uint32, vp]),
            "zsmr_ceiling_set_balance": (i32, [i32]),
        })
    return _LIB


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _ptr(x):
    """Device address of a tensor or a raw address; host tensors are refused."""
    if isinstance(x, int):
        return x
    dev = getattr(x, "device", None)
    if dev is not None and getattr(dev, "type", "cuda") != "cuda":
        raise ValueError(f"a {dev.type} tensor was passed where device memory is required")
    return x.data_ptr()


def read(src, nbytes: int, shape: int, sink, stream=None) -> None:
    code = _lib().zsmr_ceiling_read(_ptr(src), nbytes, shape, _ptr(sink), _stream(stream))
    if code:
        raise RuntimeError(f"zsmr_ceiling_read failed with code {code}")


def write(dst, nbytes: int, shape: int, value: int, stream=None) -> None:
    code = _lib().zsmr_ceiling_write(_ptr(dst), nbytes, shape, value & 0xFFFFFFFF, _stream(stream))
    if code:
        raise RuntimeError(f"zsmr_ceiling_write failed with code {code}")


def set_balance(even_permille: int) -> None:
    """Weight of each even XCD against each odd one in the balanced shapes
    (thousandths, 500..2000)."""
    code = _lib().zsmr_ceiling_set_balance(even_permille)
    if code:
        raise RuntimeError(f"zsmr_ceiling_set_balance failed with code {code}")


def phased_bound(read_bytes: int, write_bytes: int, read_gbps: float, write_gbps: float) -> float:
    """Least time in ms for read_bytes read and write_bytes written at the
    given pure rates (GB/s), with no read/write turnaround."""
    return read_bytes / (read_gbps * 1e6) + write_bytes / (write_gbps * 1e6)


def measure(buf, nbytes: int, reps: int = 5) -> dict:
    """Best pure read and pure write rate (GB/s) over the shapes, on the
    device buffer ``buf`` of at least ``nbytes`` bytes (overwritten), each
    shape timed over ``reps`` launches after one untimed launch."""
    import torch
    nbytes = nbytes // 16 * 16
    sink = torch.zeros(4, dtype=torch.int32, device=buf.device)
    stream = torch.cuda.current_stream()
    out = {"bytes": nbytes, "read": {}, "write": {}}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return nbytes / (e0.elapsed_time(e1) / reps) / 1e6

    for name, shape in WRITE_SHAPES.items():
        out["write"][name] = round(timed(lambda: write(buf, nbytes, shape, 0x3C003C00, stream)), 1)
    for name, shape in READ_SHAPES.items():
        out["read"][name] = round(timed(lambda: read(buf, nbytes, shape, sink, stream)), 1)
    out["read_GBps"] = max(out["read"].values())
    out["write_GBps"] = max(out["write"].values())
    return out
