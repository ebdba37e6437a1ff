"""ctypes binding of ``synth/libzsmr_synth.so`` (GPU fills with the same
definition as ``synth/__init__.py``).  Input preparation only."""
from __future__ import annotations

import ctypes
import os

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libzsmr_synth.so")
_CODES = {"fp16": 1, "bf16": 2}
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m zero_sharded_mixed_reduce_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        lib.zsmr_synth_fill16.restype = i32
        lib.zsmr_synth_fill16.argtypes = [vp, i32, i64, i64, i64, i64, ctypes.c_uint32, i32, i32,
                                          i32, ctypes.c_float, i32, i32, vp]
        lib.zsmr_synth_fill32.restype = i32
        lib.zsmr_synth_fill32.argtypes = [vp, i64, i64, i64, ctypes.c_uint32, i32, i32, i32,
                                          ctypes.c_float, vp]
        _LIB = lib
    return _LIB


# ctypes truncates a Python int that does not fit its C type; refuse instead
_RANGE = {ctypes.c_int32: (-(1 << 31), (1 << 31) - 1), ctypes.c_int64: (-(1 << 63), (1 << 63) - 1),
          ctypes.c_uint32: (0, (1 << 32) - 1)}


def _call(name: str, *args):
    fn = getattr(_lib(), name)
    for i, (x, t) in enumerate(zip(args, fn.argtypes)):
        r = _RANGE.get(t)
        if r is not None and isinstance(x, int) and not r[0] <= x <= r[1]:
            raise ValueError(f"{name}: argument {i} = {x} is outside [{r[0]}, {r[1]}]")
    return fn(*args)


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


def fill16(dst, rows: int, row_stride: int, n: int, p0: int, p_valid: int, seed: int, tag: int,
           rank0: int, step: int, sigma: float, dtype: str, outlier_permyriad: int = 0,
           stream=None) -> None:
    code = _call("zsmr_synth_fill16", _ptr(dst), rows, row_stride, n, p0, p_valid, seed, tag,
                 rank0, step, sigma, _CODES[dtype], outlier_permyriad, _stream(stream))
    if code:
        raise RuntimeError(f"zsmr_synth_fill16 failed with code {code}")


def fill32(dst, n: int, p0: int, p_valid: int, seed: int, tag: int, rank: int, step: int,
           sigma: float, stream=None) -> None:
    code = _call("zsmr_synth_fill32", _ptr(dst), n, p0, p_valid, seed, tag, rank, step, sigma,
                 _stream(stream))
    if code:
        raise RuntimeError(f"zsmr_synth_fill32 failed with code {code}")
