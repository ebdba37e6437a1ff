"""Python binding of libzsmr.so, the ZeRO shard step on one MI355X (gfx950).

Argument marshalling only: every function here has the name of a C entry
point of ``include/zsmr.h`` and passes pointers (``tensor.data_ptr()`` or a
plain int), sizes and a HIP stream (default: torch's current stream) to it.
All arithmetic runs in the library's HIP kernels.  There is no fallback: if
``libzsmr.so`` has not been built, importing the library raises.
"""
from __future__ import annotations

import ctypes
import os
import types
from typing import Optional, Sequence

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libzsmr.so")

ZSMR_OK, ZSMR_ERR_ARG, ZSMR_ERR_INDIVISIBLE, ZSMR_ERR_STATE = 0, 1, 2, 3
ZSMR_ERR_DTYPE, ZSMR_ERR_ALIGN, ZSMR_ERR_HIP = 4, 5, 6
ZSMR_FP16, ZSMR_BF16 = 1, 2
ZSMR_DP, ZSMR_ZERO1, ZSMR_ZERO2, ZSMR_ZERO3 = 0, 1, 2, 3
ZSMR_ZERO3_OWNER = 4           # stage 3 with whole units owned by single ranks (owner broadcast)
DTYPES = {"fp16": ZSMR_FP16, "bf16": ZSMR_BF16}

_i32, _i64, _vp, _f32p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p


class ZsmrError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = f"{where}: {_lib().zsmr_strerror(code).decode()} (code {code})"
        if code == ZSMR_ERR_HIP:
            msg += f": {_lib().zsmr_last_hip_error().decode()}"
        super().__init__(msg)
        self.code = code


class zsmr_adam(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double)]


class zsmr_layout_info(ctypes.Structure):
    _fields_ = [("numel", _i64), ("padded_numel", _i64), ("shard_numel", _i64),
                ("max_unit_numel", _i64), ("world", _i32), ("stage", _i32), ("n_units", _i32),
                ("grad_dtype", _i32), ("param_dtype", _i32), ("pad", _i32)]


class zsmr_bytes(ctypes.Structure):
    _fields_ = [(n, _i64) for n in ("res_p16", "res_grad", "res_master", "res_m", "res_v",
                                    "resident", "gathered", "peak", "unit_grad", "rs_elems",
                                    "ag_elems", "ar_elems", "traffic_elems", "traffic_bytes")]


class zsmr_plan(ctypes.Structure):
    _fields_ = [("kernel", _i32), ("ring_tiles", _i32), ("windowed", _i32), ("store_elems", _i32),
                ("launches", _i32), ("row_batch", _i32), ("head", _i64)]


ZSMR_KERNEL_SCALAR, ZSMR_KERNEL_DIRECT, ZSMR_KERNEL_DEFERRED = 0, 1, 2
KERNEL_NAMES = {0: "scalar", 1: "direct", 2: "deferred"}


class zsmr_counters(ctypes.Structure):
    _fields_ = [(n, _i64) for n in ("rs_elems", "ag_elems", "ar_elems", "traffic_elems",
                                    "traffic_bytes", "stage3_gathers", "stage3_releases",
                                    "live_units", "live_bytes", "peak_live_bytes")]


# name -> (restype, argtypes); the list is the ABI of include/zsmr.h
SIGNATURES = {
    "zsmr_strerror": (ctypes.c_char_p, [_i32]),
    "zsmr_last_hip_error": (ctypes.c_char_p, []),
    "zero_init_shards": (_i32, [ctypes.POINTER(_vp), _i64, _i32, _i32, _i32, _i32, _i32,
                                ctypes.POINTER(_i64), _i32]),
    "zero_destroy": (None, [_vp]),
    "zero_layout_info": (_i32, [_vp, ctypes.POINTER(zsmr_layout_info)]),
    "zero_layout": (_i32, [_vp, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                           ctypes.POINTER(_i64)]),
    "zero_bytes_per_rank": (_i32, [_vp, _i32, _i32, ctypes.POINTER(zsmr_bytes)]),
    "zero_bytes_of_rank": (_i32, [_vp, _i32, _i32, _i32, ctypes.POINTER(zsmr_bytes)]),
    "zero_unit_owner": (_i32, [_vp, _i32, ctypes.POINTER(_i32)]),
    "zero_set_unit_owners": (_i32, [_vp, ctypes.POINTER(_i32), _i32]),
    "zero_counters": (_i32, [_vp, _i32, ctypes.POINTER(zsmr_counters)]),
    "zero_reset_counters": (_i32, [_vp]),
    "zero_init_state": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "zero_reduce_shard": (_i32, [_vp, _i32, _i32, _vp, _i64, _i64, _i32, _vp, _vp]),
    "zero_adam_step": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, ctypes.POINTER(zsmr_adam), _vp]),
    "zero_gather_cast": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "zero_fused_step": (_i32, [_vp, _i32, _i32, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _i32,
                               ctypes.POINTER(zsmr_adam), _vp]),
    "zero_fused_step_range": (_i32, [_vp, _i32, _i32, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp,
                                     _vp, _i32, ctypes.POINTER(zsmr_adam), _vp]),
    "zsmr_fused_step_plan": (_i32, [_vp, _i32, _i32, _vp, _i64, _i64, _vp, _vp, _vp, _vp,
                                    ctypes.POINTER(zsmr_plan)]),
    "zero_gather_copy": (_i32, [_vp, _i32, _vp, _vp, _i64, _vp]),
    "zero_gather_copy_blocks": (_i32, [_vp, _i32, _vp, _vp, _i64, _i32, _i64, _vp]),
    "zero_stage3_set_max_live": (_i32, [_vp, _i32]),
    "zero_stage3_unit_gather": (_i32, [_vp, _i32, ctypes.POINTER(_vp), _vp, _vp]),
    "zero_stage3_unit_release": (_i32, [_vp, _i32]),
    "zero_stage3_unit_state": (_i32, [_vp, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i64),
                                      ctypes.POINTER(_i64)]),
    "zsmr_set_launch_shape": (_i32, [_i32, _i32, _i32, _i32]),
    "zsmr_set_write_window": (_i32, [_i32, _i32, _i32, _i32]),
    "zsmr_set_xcd_balance": (_i32, [_i32]),
}

_LIB = None

# ctypes converts a Python int to a C integer by truncation (2**32 + 4 passed
# as int32_t arrives as 4), so every integer argument is range-checked first.
_INT_RANGE = {ctypes.c_int32: (-(1 << 31), (1 << 31) - 1),
              ctypes.c_int64: (-(1 << 63), (1 << 63) - 1),
              ctypes.c_uint32: (0, (1 << 32) - 1)}


class CheckedFunction:
    """A ctypes function whose integer arguments must fit their C types."""

    def __init__(self, name: str, fn, argtypes):
        self.name, self.fn = name, fn
        self.ints = [(i, *_INT_RANGE[t]) for i, t in enumerate(argtypes) if t in _INT_RANGE]

    def __call__(self, *args):
        for i, lo, hi in self.ints:
            x = args[i] if i < len(args) else None
            if isinstance(x, int) and not lo <= x <= hi:
                raise ValueError(f"{self.name}: argument {i} = {x} is outside [{lo}, {hi}]")
        return self.fn(*args)


def int_array(ctype, values, what: str):
    """A ctypes array of integers, each checked to fit ``ctype`` (ctypes would
    truncate silently: 2**32 + 1 stored in an int32_t array arrives as 1)."""
    lo, hi = _INT_RANGE[ctype]
    vals = [int(x) for x in values]
    for i, x in enumerate(vals):
        if not lo <= x <= hi:
            raise ValueError(f"{what}[{i}] = {x} is outside [{lo}, {hi}]")
    return (ctype * max(len(vals), 1))(*vals)


def checked_library(path: str, signatures: dict):
    """Load a shared library and give it the (restype, argtypes) of each
    named function; returns a namespace of CheckedFunction."""
    lib = ctypes.CDLL(path)
    fns = {}
    for name, (res, args) in signatures.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
        fns[name] = CheckedFunction(name, fn, args)
    return types.SimpleNamespace(**fns)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m zero_sharded_mixed_reduce_amd.build`")
        _LIB = checked_library(LIB_PATH, SIGNATURES)
    return _LIB


def load():
    """Load libzsmr.so (raises ImportError if it has not been built)."""
    return _lib()


def _check(code: int, where: str) -> None:
    if code != ZSMR_OK:
        raise ZsmrError(code, where)


def _ptr(x) -> Optional[int]:
    """Device address of a tensor (or a raw address, passed as it is).  A
    tensor in host memory is refused: a kernel would take its address for a
    device one."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    dev = getattr(x, "device", None)
    if dev is not None and getattr(dev, "type", "cuda") != "cuda":
        raise ValueError(f"a {dev.type} tensor was passed where device memory is required")
    return x.data_ptr()


def _fits(x, elems: int, elem_bytes: int, what: str) -> None:
    """A tensor argument must be contiguous and hold the elems * elem_bytes
    bytes the call touches from its first element: the library sees only the
    address and cannot check.  Raw addresses are the caller's to check."""
    if x is None or isinstance(x, int) or elems <= 0:
        return
    if not x.is_contiguous():
        raise ValueError(f"{what}: the tensor is not contiguous")
    have = x.numel() * x.element_size()
    if have < elems * elem_bytes:
        raise ValueError(f"{what}: {have} bytes, the call touches {elems * elem_bytes}")


def _piece_len(ctx, rank: int, unit: int) -> int:
    """Elements of the (rank, unit) piece, or 0 where the layout refuses the
    pair (the call itself then reports the error)."""
    off, ln, loc = _i64(), _i64(), _i64()
    if _lib().zero_layout(ctx.handle, rank, unit, ctypes.byref(off), ctypes.byref(ln),
                          ctypes.byref(loc)) != ZSMR_OK:
        return 0
    return ln.value


def _rows_fit(ctx, grads, row_stride: int, base: int, end: int, what: str) -> None:
    """The N gradient rows: row r covers [base + r*row_stride, ... + end)."""
    if grads is None or isinstance(grads, int) or end <= 0:
        return
    _fits(grads, int(base) + (ctx.world - 1) * max(int(row_stride), 0) + end, 2, what)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _hp(lr: float, betas=(0.9, 0.999), eps: float = 1e-8) -> zsmr_adam:
    return zsmr_adam(float(lr), float(betas[0]), float(betas[1]), float(eps))


class Ctx:
    """Owner of a ``zsmr_ctx*`` (freed with ``zero_destroy`` on close/GC)."""

    def __init__(self, handle: int):
        self.handle = handle
        self._world = None

    @property
    def world(self) -> int:
        """N, fixed when the context is made (read once, then kept)."""
        if self._world is None:
            self._world = zero_layout_info(self)["world"]
        return self._world

    def close(self):
        if self.handle:
            _lib().zero_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def _as_param(self):
        return self.handle

    def info(self) -> dict:
        return zero_layout_info(self)

    def layout(self, rank: int, unit: int = 0):
        return zero_layout(self, rank, unit)


def zero_init_shards(numel: int, world: int, stage: int, grad_dtype: str = "bf16",
                     param_dtype: Optional[str] = None, pad: bool = False,
                     units: Optional[Sequence[int]] = None) -> Ctx:
    h = _vp()
    arr = None
    n_units = 0
    if units:
        arr = int_array(_i64, units, "units")
        n_units = len(units)
    code = _lib().zero_init_shards(ctypes.byref(h), int(numel), int(world), int(stage),
                                   DTYPES[grad_dtype], DTYPES[param_dtype or grad_dtype],
                                   int(bool(pad)), arr, n_units)
    _check(code, "zero_init_shards")
    return Ctx(h.value)


def zero_destroy(ctx: Ctx) -> None:
    ctx.close()


def zero_layout_info(ctx: Ctx) -> dict:
    out = zsmr_layout_info()
    _check(_lib().zero_layout_info(ctx.handle, ctypes.byref(out)), "zero_layout_info")
    return {n: getattr(out, n) for n, _ in out._fields_}


def zero_layout(ctx: Ctx, rank: int, unit: int = 0):
    off, ln, loc = _i64(), _i64(), _i64()
    _check(_lib().zero_layout(ctx.handle, rank, unit, ctypes.byref(off), ctypes.byref(ln),
                              ctypes.byref(loc)), "zero_layout")
    return off.value, ln.value, loc.value


def zero_bytes_per_rank(ctx: Ctx, gather_bytes: int = 0, max_live: int = 0) -> dict:
    out = zsmr_bytes()
    _check(_lib().zero_bytes_per_rank(ctx.handle, gather_bytes, max_live, ctypes.byref(out)),
           "zero_bytes_per_rank")
    return {n: getattr(out, n) for n, _ in out._fields_}


def zero_bytes_of_rank(ctx: Ctx, rank: int, gather_bytes: int = 0, max_live: int = 0) -> dict:
    out = zsmr_bytes()
    _check(_lib().zero_bytes_of_rank(ctx.handle, rank, gather_bytes, max_live, ctypes.byref(out)),
           "zero_bytes_of_rank")
    return {n: getattr(out, n) for n, _ in out._fields_}


def zero_unit_owner(ctx: Ctx, unit: int) -> int:
    o = _i32()
    _check(_lib().zero_unit_owner(ctx.handle, unit, ctypes.byref(o)), "zero_unit_owner")
    return o.value


def zero_set_unit_owners(ctx: Ctx, owners: Sequence[int]) -> None:
    arr = int_array(_i32, owners, "owners")
    _check(_lib().zero_set_unit_owners(ctx.handle, arr, len(owners)), "zero_set_unit_owners")


def zero_counters(ctx: Ctx, rank: int) -> dict:
    out = zsmr_counters()
    _check(_lib().zero_counters(ctx.handle, rank, ctypes.byref(out)), "zero_counters")
    return {n: getattr(out, n) for n, _ in out._fields_}


def zero_reset_counters(ctx: Ctx) -> None:
    _check(_lib().zero_reset_counters(ctx.handle), "zero_reset_counters")


def zero_init_state(ctx: Ctx, rank: int, unit: int, theta0, master, m, v, p16, stream=None):
    n = _piece_len(ctx, rank, unit)
    for x, what in ((theta0, "theta0"), (master, "master"), (m, "m"), (v, "v")):
        _fits(x, n, 4, what)
    _fits(p16, n, 2, "p16")
    _check(_lib().zero_init_state(ctx.handle, rank, unit, _ptr(theta0), _ptr(master), _ptr(m),
                                  _ptr(v), _ptr(p16), _stream(stream)), "zero_init_state")


def zero_reduce_shard(ctx: Ctx, rank: int, unit: int, grads, row_stride: int, base_elem: int,
                      mean: bool, g_out, stream=None):
    n = _piece_len(ctx, rank, unit)
    _rows_fit(ctx, grads, row_stride, base_elem, n, "grads")
    _fits(g_out, n, 4, "g_out")
    _check(_lib().zero_reduce_shard(ctx.handle, rank, unit, _ptr(grads), int(row_stride),
                                    int(base_elem), int(bool(mean)), _ptr(g_out), _stream(stream)),
           "zero_reduce_shard")


def zero_adam_step(master, m, v, g, n: int, t: int, lr: float, betas=(0.9, 0.999),
                   eps: float = 1e-8, stream=None):
    for x, what in ((master, "master"), (m, "m"), (v, "v"), (g, "g")):
        _fits(x, int(n), 4, what)
    hp = _hp(lr, betas, eps)
    _check(_lib().zero_adam_step(_ptr(master), _ptr(m), _ptr(v), _ptr(g), int(n), int(t),
                                 ctypes.byref(hp), _stream(stream)), "zero_adam_step")


def zero_gather_cast(ctx: Ctx, rank: int, unit: int, master, p16_dst, stream=None):
    n = _piece_len(ctx, rank, unit)
    _fits(master, n, 4, "master")
    _fits(p16_dst, n, 2, "p16_dst")
    _check(_lib().zero_gather_cast(ctx.handle, rank, unit, _ptr(master), _ptr(p16_dst),
                                   _stream(stream)), "zero_gather_cast")


def zero_fused_step(ctx: Ctx, rank: int, unit: int, grads, row_stride: int, base_elem: int,
                    master, m, v, p16_dst, t: int, lr: float, betas=(0.9, 0.999),
                    eps: float = 1e-8, stream=None):
    n = _piece_len(ctx, rank, unit)
    _rows_fit(ctx, grads, row_stride, base_elem, n, "grads")
    for x, what in ((master, "master"), (m, "m"), (v, "v")):
        _fits(x, n, 4, what)
    _fits(p16_dst, n, 2, "p16_dst")
    hp = _hp(lr, betas, eps)
    _check(_lib().zero_fused_step(ctx.handle, rank, unit, _ptr(grads), int(row_stride),
                                  int(base_elem), _ptr(master), _ptr(m), _ptr(v), _ptr(p16_dst),
                                  int(t), ctypes.byref(hp), _stream(stream)), "zero_fused_step")


def zsmr_fused_step_plan(ctx: Ctx, rank: int, unit: int, grads, row_stride: int, base_elem: int,
                         master, m, v, p16_dst) -> dict:
    """Which kernel ``zero_fused_step`` with these arguments runs (nothing is
    launched): kernel ("scalar", "direct" or "deferred"), ring_tiles,
    windowed, store_elems, launches, row_batch, head."""
    out = zsmr_plan()
    _check(_lib().zsmr_fused_step_plan(ctx.handle, rank, unit, _ptr(grads), int(row_stride),
                                       int(base_elem), _ptr(master), _ptr(m), _ptr(v),
                                       _ptr(p16_dst), ctypes.byref(out)), "zsmr_fused_step_plan")
    d = {n: getattr(out, n) for n, _ in out._fields_}
    d["kernel"] = KERNEL_NAMES[d["kernel"]]
    return d


def zero_fused_step_range(ctx: Ctx, rank: int, unit: int, begin: int, count: int, grads,
                          row_stride: int, base_elem: int, master, m, v, p16_dst, t: int,
                          lr: float, betas=(0.9, 0.999), eps: float = 1e-8, stream=None):
    end = int(begin) + int(count) if int(begin) >= 0 and int(count) >= 0 else 0
    _rows_fit(ctx, grads, row_stride, base_elem, end, "grads")
    for x, what in ((master, "master"), (m, "m"), (v, "v")):
        _fits(x, end, 4, what)
    _fits(p16_dst, end, 2, "p16_dst")
    hp = _hp(lr, betas, eps)
    _check(_lib().zero_fused_step_range(ctx.handle, rank, unit, int(begin), int(count), _ptr(grads),
                                        int(row_stride), int(base_elem), _ptr(master), _ptr(m),
                                        _ptr(v), _ptr(p16_dst), int(t), ctypes.byref(hp),
                                        _stream(stream)), "zero_fused_step_range")


def zero_gather_copy(ctx: Ctx, recv_rank: int, src, dst, n: int, stream=None):
    _fits(src, int(n), 2, "src")
    _fits(dst, int(n), 2, "dst")
    _check(_lib().zero_gather_copy(ctx.handle, recv_rank, _ptr(src), _ptr(dst), int(n),
                                   _stream(stream)), "zero_gather_copy")


def zero_gather_copy_blocks(ctx: Ctx, recv_rank: int, src, dst, n: int, count: int, stride: int,
                            stream=None):
    if int(n) > 0 and int(count) > 0:
        span = (int(count) - 1) * max(int(stride), 0) + int(n)
        _fits(src, span, 2, "src")
        _fits(dst, span, 2, "dst")
    _check(_lib().zero_gather_copy_blocks(ctx.handle, recv_rank, _ptr(src), _ptr(dst), int(n),
                                          int(count), int(stride), _stream(stream)),
           "zero_gather_copy_blocks")


def zero_stage3_set_max_live(ctx: Ctx, max_live: int) -> None:
    _check(_lib().zero_stage3_set_max_live(ctx.handle, max_live), "zero_stage3_set_max_live")


def zero_stage3_unit_gather(ctx: Ctx, unit: int, shard_ptrs: Sequence, unit_buf, stream=None):
    info = zero_layout_info(ctx)
    if info["stage"] in (ZSMR_ZERO3, ZSMR_ZERO3_OWNER) and 0 <= unit < info["n_units"]:
        if info["stage"] == ZSMR_ZERO3_OWNER:
            each = _piece_len(ctx, zero_unit_owner(ctx, unit), unit)
            nsrc = 1
        else:
            each = _piece_len(ctx, 0, unit)
            nsrc = info["world"]
        if len(shard_ptrs) < nsrc:
            # the library reads nsrc pointers from the array
            raise ValueError(f"zero_stage3_unit_gather: {len(shard_ptrs)} shard pointers, "
                             f"unit {unit} needs {nsrc}")
        for r, p in enumerate(list(shard_ptrs)[:nsrc]):
            _fits(p, each, 2, f"shard {r}")
        _fits(unit_buf, nsrc * each, 2, "unit_buf")
    arr = (_vp * len(shard_ptrs))(*[_ptr(p) for p in shard_ptrs])
    _check(_lib().zero_stage3_unit_gather(ctx.handle, unit, arr, _ptr(unit_buf), _stream(stream)),
           "zero_stage3_unit_gather")


def zero_stage3_unit_release(ctx: Ctx, unit: int) -> None:
    _check(_lib().zero_stage3_unit_release(ctx.handle, unit), "zero_stage3_unit_release")


def zero_stage3_unit_state(ctx: Ctx, unit: int):
    live, g, r = _i32(), _i64(), _i64()
    _check(_lib().zero_stage3_unit_state(ctx.handle, unit, ctypes.byref(live), ctypes.byref(g),
                                         ctypes.byref(r)), "zero_stage3_unit_state")
    return bool(live.value), g.value, r.value


def zsmr_set_launch_shape(step_bpc: int = 0, copy_bpc: int = 0, defer_tiles: int = 3,
                          defer_min_rows: int = 24) -> None:
    _check(_lib().zsmr_set_launch_shape(int(step_bpc), int(copy_bpc), int(defer_tiles),
                                        int(defer_min_rows)), "zsmr_set_launch_shape")


WRITE_WINDOW_DEFAULT = (72000, 11000, 1000, 4000)     # the library's own defaults


def zsmr_set_write_window(cycle_ns: int = WRITE_WINDOW_DEFAULT[0],
                          write_ns: int = WRITE_WINDOW_DEFAULT[1],
                          margin_ns: int = WRITE_WINDOW_DEFAULT[2],
                          lead_ns: int = WRITE_WINDOW_DEFAULT[3]) -> None:
    _check(_lib().zsmr_set_write_window(int(cycle_ns), int(write_ns), int(margin_ns), int(lead_ns)),
           "zsmr_set_write_window")


XCD_BALANCE_DEFAULT = 1200


def zsmr_set_xcd_balance(even_permille: int = XCD_BALANCE_DEFAULT) -> None:
    _check(_lib().zsmr_set_xcd_balance(int(even_permille)), "zsmr_set_xcd_balance")
