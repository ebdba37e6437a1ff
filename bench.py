"""Benchmark of the ZeRO shard step on one MI355X.

Default workload (share64): one rank's share of a 7.5e9-parameter model on 64
data-parallel ranks -- the fused reduce + Adam + cast over its 117,187,500
owned elements with 64 bf16 gradient contributions, then the receive of the
63 peer slices into the full 7.5e9-element bf16 working copy.  One step is
one pass of the whole path over one batch of synthetic gradients that are
resident in HBM before timing starts.

Prints one JSON line: params/s (owned fp32 elements updated per second),
the roofline of the dominant kernel (algorithmic bytes / average launch time
from HIP events on the launch stream, against 8 TB/s), each part's time
against the least time its reads and writes could take at the pure read and
write rates this device shows in the same run (``phased_bound``), and the
CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload share64|gpt2s|gpt2xl|llama8b]
"""
from __future__ import annotations

import argparse
import ast
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBPS = 8000.0
METRIC = "fused ZeRO shard-step params/sec and achieved HBM GB/s (% of peak), 1 GPU"
# the pure-rate references run on buffers of the share64 receive's size (63
# peer slices of 117,187,500 bf16 elements), rounded down to 16 bytes
REFERENCE_BYTES = 14_765_624_992
TRAFFIC_SOURCES = (os.path.join(ROOT, "zero_sharded_mixed_reduce_amd", "csrc", "zsmr_kernels.hip"),
                   os.path.join(ROOT, "workloads.py"))


def _code_of(path: str) -> str:
    """A source file's code without its comments (and, for Python, its
    docstrings), whitespace normalised: what a comment edit leaves alone."""
    with open(path) as f:
        src = f.read()
    if path.endswith(".py"):
        tree = ast.parse(src)
        for node in ast.walk(tree):
            body = getattr(node, "body", None)
            if (isinstance(body, list) and body and isinstance(body[0], ast.Expr)
                    and isinstance(body[0].value, ast.Constant) and isinstance(body[0].value.value, str)):
                node.body = body[1:] or [ast.Pass()]
        return ast.dump(tree)
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return " ".join(src.split())


def kernel_source_hash() -> str:
    """The measured traffic depends on the kernels and on the workloads'
    buffer layout: hash the code of both sources (comments aside)."""
    h = hashlib.sha256()
    for path in TRAFFIC_SOURCES:
        h.update(_code_of(path).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, field: str = "hbm_bytes_per_launch"):
    """HBM bytes (per launch, or per step for the world workloads) from a
    committed rocprofv3 --pmc summary, if it was taken on the current kernel
    and workload sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_and_workload_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(vals[field]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, window: int = 1 << 19, min_seconds: float = 10.0, threads: int = 0):
    """The oracle, untuned, timed on the host's cores: each of ``threads``
    threads (default: the cores this process may use, at most 16) runs it on
    its own window of the rank's shard (all N contributions, T Adam steps and
    the same window of the 63 peer slices), repeated until ``min_seconds``
    have passed; NumPy releases the interpreter lock inside its array
    operations, so the threads run in parallel.  Inputs are made before the
    clock starts; one gradient set serves every step."""
    import threading

    import numpy as np
    import synth
    from oracle import numerics as nm

    if threads <= 0:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    start = threading.Barrier(threads + 1)
    reps = [0] * threads
    ends = [0.0] * threads
    t0 = [0.0]

    def run(k):
        p = np.arange(k * window, (k + 1) * window, dtype=np.int64)
        rows16 = [synth.grad16(w.seed, r, 1, p, w.grad_sigma, w.dtype) for r in range(w.world)]
        peers = np.stack(rows16[1:])          # 63 slices of 16-bit values to copy
        theta = synth.theta0(w.seed, p)
        wc = np.zeros((w.world, window), np.uint16)
        start.wait()
        while time.perf_counter() - t0[0] < min_seconds:
            master, m, v = theta.copy(), np.zeros(window, np.float32), np.zeros(window, np.float32)
            for t in range(1, w.steps + 1):
                g = nm.reduce_rank_order([nm.widen16(r, w.dtype) for r in rows16])
                c = nm.adam_consts(w.lr, w.betas[0], w.betas[1], w.eps, t)
                master, m, v = nm.adam_update(master, m, v, g, c)
                wc[0] = nm.cast16(master, w.dtype)
                wc[1:] = peers
            reps[k] += 1
        ends[k] = time.perf_counter()

    pool = [threading.Thread(target=run, args=(k,)) for k in range(threads)]
    for th in pool:
        th.start()
    t0[0] = time.perf_counter()
    start.wait()
    t0[0] = time.perf_counter()
    for th in pool:
        th.join()
    elapsed = max(ends) - t0[0]
    params = sum(reps) * w.steps * window
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": params / elapsed, "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": f"{threads} windows of {window} owned elements of rank 0 (of {117_187_500}), "
                      f"all {w.world} bf16 contributions, {w.steps} Adam steps + cast + the same "
                      f"window of the {w.world - 1} peer slices, {sum(reps)} repetitions in all "
                      f"({elapsed:.1f} s); NumPy, one thread per window, on {cpu}"}


def warm(step, warmup: int, min_seconds: float = 1.0) -> None:
    """The W untimed warm-up steps, continued until the GPU has been busy for
    at least ``min_seconds`` (its clocks start from an idle state)."""
    import torch
    t, t0 = 0, time.perf_counter()
    while t < warmup or time.perf_counter() - t0 < min_seconds:
        t += 1
        step(t)
        torch.cuda.synchronize()


def tune_write_window(share, reps: int = 6) -> dict:
    """Pick the fused step's write window for this device.  The best cycle is
    the time the waves' LDS rings take to fill, which follows the device's
    read rate.  Two stages, every candidate timed over a few untimed warm-up
    steps (the window changes only when results are stored): cycles from 66
    to 82 us with the default window, then write window and lead around the
    fastest cycle; the three fastest are timed once more and the fastest of
    those is kept."""
    import torch
    import zero_sharded_mixed_reduce_amd as z
    c0, w0, margin, lead0 = z.WRITE_WINDOW_DEFAULT
    stream = torch.cuda.current_stream()
    tried = []

    def timed(cfg):
        z.zsmr_set_write_window(*cfg)
        share.fused(1000)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            share.fused(1000)
        e1.record(stream)
        torch.cuda.synchronize()
        tried.append((e0.elapsed_time(e1) / reps, cfg))
        return tried[-1]

    best = min(timed((c0 + dc * 1000, w0, margin, lead0)) for dc in (-8, -4, -2, 0, 2, 4, 8))
    c1 = best[1][0]
    for dc in (-2000, 0, 2000):
        for dw in (-2000, -1000, 0):
            for lead in (2000, 3000, 4000):
                cfg = (c1 + dc, w0 + dw, margin, lead)
                if cfg not in [t[1] for t in tried]:
                    timed(cfg)
    n = len(tried)
    # the three fastest again, so that one lucky timing does not decide
    finalists = [cfg for _, cfg in sorted(tried)[:3]]
    del tried[:]
    best = min(timed(cfg) for cfg in finalists)
    z.zsmr_set_write_window(*best[1])
    return {"cycle": best[1][0], "write": best[1][1], "margin": best[1][2], "lead": best[1][3],
            "tuned_over": n}


def tune_xcd_balance(share, reps: int = 3) -> dict:
    """Pick the copies' work split between even and odd XCDs for this device
    (the even XCDs of MI355X move data faster): the receive is timed at a
    few splits, each over a few launches after an untimed one, the two
    fastest again, and the fastest of those is kept."""
    import torch
    import zero_sharded_mixed_reduce_amd as z
    stream = torch.cuda.current_stream()
    tried = []

    def timed(permille):
        z.zsmr_set_xcd_balance(permille)
        share.receive()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            share.receive()
        e1.record(stream)
        torch.cuda.synchronize()
        tried.append((e0.elapsed_time(e1) / reps, permille))
        return tried[-1]

    for permille in (1000, 1100, 1150, 1200, 1250, 1300):
        timed(permille)
    n = len(tried)
    finalists = [p for _, p in sorted(tried)[:2]]
    del tried[:]
    best = min(timed(p) for p in finalists)
    z.zsmr_set_xcd_balance(best[1])
    return {"even_permille": best[1], "tuned_over": n}


def references(z, nbytes: int, reps: int = 5, balance: int = 1200) -> dict:
    """Rates this device gives simple streams of the receive's size, measured
    in the same process on two fresh, equally aligned buffers of ``nbytes``:
    the library's 128-bit copy and the runtime's device-to-device copy (GB/s
    of reads + writes), and the best pure read and pure write rates of the
    reference streams in ``ceiling/`` (their balanced shapes weighted like
    the library's copies, ``balance`` thousandths per even XCD)."""
    import torch
    import ceiling
    ceiling.set_balance(balance)
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ctx = z.zero_init_shards(2, 2, 2, "bf16")
    stream = torch.cuda.current_stream()
    for _ in range(2):
        z.zero_gather_copy(ctx, 0, src, dst, src.numel())
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        z.zero_gather_copy(ctx, 0, src, dst, src.numel())
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # the runtime's own device-to-device copy (hipMemcpyAsync, behind torch's
    # copy_) on the same buffers, for comparison only
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_vendor = e0.elapsed_time(e1) / reps
    pure = ceiling.measure(dst, nbytes, reps)
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_GBps": 2 * nbytes / ms / 1e6, "runtime_copy_GBps": 2 * nbytes / ms_vendor / 1e6,
            "pure": pure}


def phased(parts: dict, rw: dict, pure: dict) -> dict:
    """Each part's time against the least time its reads and writes could take
    at this device's pure read and write rates (``ceiling.phased_bound``)."""
    import ceiling
    out = {"read_GBps": pure["read_GBps"], "write_GBps": pure["write_GBps"],
           "read_shapes_GBps": pure["read"], "write_shapes_GBps": pure["write"],
           "reference_bytes": pure["bytes"]}
    for name, (rb, wb, ms) in rw.items():
        bound = ceiling.phased_bound(rb, wb, pure["read_GBps"], pure["write_GBps"])
        out[name] = {"read_bytes": rb, "write_bytes": wb, "bound_ms": round(bound, 4),
                     "measured_ms": round(ms, 4), "frac": round(bound / ms, 4)}
    return out


def bucketed_overlap(share, args, reps: int = 5) -> dict:
    """Steps that include the simulated backward pass (the gradient fill of
    all 64 rows): sequential (fill everything, then one fused launch) against
    bucketed (each bucket's fill on a second stream, its fused launch as soon
    as it is ready).  Reported beside the headline, which excludes the fill."""
    import torch
    side = torch.cuda.Stream()
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn(1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(2 + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def sequential(t):
        share.gen_grads(t)
        share.step(t)

    seq = timed(sequential)
    fill = timed(share.gen_grads)
    buck = timed(lambda t: share.step_bucketed(t, args.buckets, side))
    share.gen_grads(1)
    torch.cuda.synchronize()
    return {"n_buckets": args.buckets, "backward_fill_ms": round(fill, 4),
            "sequential_ms": round(seq, 4), "bucketed_overlapped_ms": round(buck, 4),
            "hidden_fraction_of_step": round((seq - buck) / (seq - fill), 4) if seq > fill else None}


def untuned_step(share, args) -> dict:
    """The same step at the library's default write window and XCD split
    (what a caller gets without tuning), timed like the headline; the tuned
    settings are restored afterwards."""
    import torch
    import zero_sharded_mixed_reduce_amd as z
    stream = torch.cuda.current_stream()
    z.zsmr_set_write_window()
    z.zsmr_set_xcd_balance()
    t0 = args.warmup + args.steps + 1
    share.step(t0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        share.step(t0 + 1 + i)
    e1.record(stream)
    torch.cuda.synchronize()
    z.zsmr_set_write_window(*args.tuned["window"])
    z.zsmr_set_xcd_balance(args.tuned["balance"])
    return {"ms": round(e0.elapsed_time(e1) / args.steps, 4),
            "write_window_ns": list(z.WRITE_WINDOW_DEFAULT),
            "xcd_even_permille": z.XCD_BALANCE_DEFAULT}


def unfused_step(share, args, reps: int = 10) -> dict:
    """The fused pass's work done by the three unfused calls (reduce to an
    fp32 gradient, Adam, cast), timed with HIP events on the launch stream:
    12 more bytes per element (the gradient written and read back, the
    master read again) and three launches."""
    import torch
    stream = torch.cuda.current_stream()
    g_tmp = torch.empty(share.S, dtype=torch.float32, device=share.master.device)
    import zero_sharded_mixed_reduce_amd as z
    w, S = share.w, share.S

    def step(t):
        z.zero_reduce_shard(share.ctx, share.rank, 0, share.grads, share.row_stride, 0, True, g_tmp)
        z.zero_adam_step(share.master, share.m, share.v, g_tmp, S, t, w.lr, w.betas, w.eps)
        z.zero_gather_cast(share.ctx, share.rank, 0, share.master, share.wc[share.off:])

    t0 = args.warmup + args.steps + 1
    step(t0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        step(t0 + 1 + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    byts = share.S * (2 * share.w.world + 26 + 12)
    del g_tmp
    return {"ms": round(ms, 4), "bytes": byts, "GBps": round(byts / ms / 1e6, 1)}


def bench_share64(args, w):
    import torch
    import workloads as wl
    import zero_sharded_mixed_reduce_amd as z

    z.zsmr_set_launch_shape(args.step_bpc, args.copy_bpc, args.defer_tiles, args.defer_min_rows)
    z.zsmr_set_write_window(args.window_cycle_ns, args.window_write_ns, args.window_margin_ns,
                            args.window_lead_ns)
    share = wl.RankShare(w, rank=0)
    share.gen_grads(1)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    warm(lambda t: share.step(t), args.warmup)
    window = {"cycle": args.window_cycle_ns, "write": args.window_write_ns,
              "margin": args.window_margin_ns, "lead": args.window_lead_ns, "tuned_over": 0}
    if not args.window_explicit:
        window = tune_write_window(share)
    balance = {"even_permille": args.xcd_balance, "tuned_over": 0}
    if args.xcd_balance is None:
        balance = tune_xcd_balance(share)
    else:
        z.zsmr_set_xcd_balance(args.xcd_balance)
    # what the run tuned, restored after the untuned comparison
    args.tuned = None
    if window["tuned_over"] or balance["tuned_over"]:
        args.tuned = {"window": (window["cycle"], window["write"], window["margin"], window["lead"]),
                      "balance": balance["even_permille"]}
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()                    # the timed region starts with an idle device
    t0 = time.perf_counter()
    for i in range(args.steps):
        t = args.warmup + 1 + i
        ev[i][0].record(stream)
        share.fused(t)
        ev[i][1].record(stream)
        share.receive()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fused_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    recv_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    ms_step = wall * 1e3 / args.steps
    untuned = untuned_step(share, args) if args.tuned else None

    S, N = share.S, w.world
    bucketed = bucketed_overlap(share, args) if args.buckets else None
    unfused = unfused_step(share, args) if args.unfused else None
    fused_bytes = S * (2 * N + 26)              # N x 2 B grads, 24 B master/m/v r+w, 2 B cast
    recv_bytes = (share.P - S) * 4              # 2 B read + 2 B written per peer element
    parts = {
        "fused_step": {"ms": round(fused_ms, 4), "bytes": fused_bytes,
                       "GBps": round(fused_bytes / fused_ms / 1e6, 1),
                       "frac": round(fused_bytes / fused_ms / 1e6 / PEAK_HBM_GBPS, 4)},
        "peer_receive": {"ms": round(recv_ms, 4), "bytes": recv_bytes,
                         "GBps": round(recv_bytes / recv_ms / 1e6, 1),
                         "frac": round(recv_bytes / recv_ms / 1e6 / PEAK_HBM_GBPS, 4)},
        "step_GBps": round((fused_bytes + recv_bytes) / ms_step / 1e6, 1),
    }
    if untuned:
        parts["step_at_library_defaults"] = dict(
            untuned, GBps=round((fused_bytes + recv_bytes) / untuned["ms"] / 1e6, 1),
            frac=round((fused_bytes + recv_bytes) / untuned["ms"] / 1e6 / PEAK_HBM_GBPS, 4))
    if bucketed:
        parts["bucketed_with_backward"] = bucketed
    if unfused:
        unfused["fused_over_unfused_time"] = round(fused_ms / unfused["ms"], 4)
        parts["unfused_step"] = unfused
    dom = "fused_step" if fused_ms >= recv_ms else "peer_receive"
    fused_kernel = ("step_deferred_kernel" if args.defer_tiles > 0 and N >= args.defer_min_rows
                    else "step_vec8_kernel")
    kname = {"fused_step": fused_kernel, "peer_receive": "copy16_kernel"}[dom]
    roof = {"bound": "hbm", "achieved": parts[dom]["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": parts[dom]["frac"], "traffic": read_traffic(kname, w.key),
            "kernel": kname, "algorithmic_bytes_per_launch": parts[dom]["bytes"]}
    # the hot path's own kernel, reported beside the dominant one
    roof_fused = {"bound": "hbm", "achieved": parts["fused_step"]["GBps"], "peak": PEAK_HBM_GBPS,
                  "unit": "GB/s", "frac": parts["fused_step"]["frac"],
                  "traffic": read_traffic(fused_kernel, w.key), "kernel": fused_kernel,
                  "algorithmic_bytes_per_launch": fused_bytes}
    half = recv_bytes // 2
    rw = {"fused_step": (S * (2 * N + 12), 14 * S, fused_ms), "peer_receive": (half, half, recv_ms),
          "step": (S * (2 * N + 12) + half, 14 * S + half, ms_step)}
    return S / (ms_step / 1e3), ms_step, roof, roof_fused, parts, rw, {
        "workload": w.name, "numel": w.numel, "world": N, "stage": w.stage, "owned_shard": S,
        "grad_dtype": w.dtype, "working_copy_elems": share.P, "steps_T": w.steps, "lr": w.lr,
        "rank": 0, "step_workgroups_per_cu": args.step_bpc,
        "copy_workgroups_per_cu": args.copy_bpc, "fused_defer_tiles": args.defer_tiles,
        "fused_defer_min_rows": args.defer_min_rows,
        "fused_write_window_ns": window, "copy_xcd_balance": balance}


def time_world(args, w, owner: bool = False, prefetch: bool = False):
    """Simulated-world workloads (all N ranks on the GPU): one step = N fused
    launches (stages 1-2) or the ZeRO-3 unit schedule (stage 3), timed with
    HIP events on the compute stream.  Returns (ms per step, algorithmic
    bytes per step, (read bytes, write bytes) per step)."""
    import torch
    import workloads as wl

    stream = torch.cuda.current_stream()
    if w.stage == 3:
        # each unit size's gradients are made once, so that whole steps --
        # gathers, fused launches and (with prefetch) the overlap of the next
        # gather -- are timed end to end on the compute stream
        world = wl.Stage3World(w, prefetch=prefetch, fixed_grads=True, owner=owner,
                               owners=wl.LLAMA8B_OWNERS if owner and w.key == "llama8b" else None)
    else:
        world = wl.ShardedWorld(w)
        world.gen_grads(1)
    warm(lambda t: world.step(t), args.warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        world.step(args.warmup + 1 + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    del world
    free_device()
    N = w.world
    byts = w.numel * (2 * N + 26) + (8 * w.numel if w.stage == 3 else 0)
    gather = 4 * w.numel if w.stage == 3 else 0      # two gathers: 2 B read + 2 B written each
    return ms_step, byts, (w.numel * (2 * N + 12) + gather, 14 * w.numel + gather)


def free_device():
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def fused_kernel_name(args, rows: int) -> str:
    return "step_deferred_kernel" if args.defer_tiles > 0 and rows >= args.defer_min_rows \
        else "step_vec8_kernel"


def bench_world(args, w):
    import zero_sharded_mixed_reduce_amd as z

    z.zsmr_set_launch_shape(args.step_bpc, args.copy_bpc, args.defer_tiles, args.defer_min_rows)
    z.zsmr_set_write_window(args.window_cycle_ns, args.window_write_ns, args.window_margin_ns,
                            args.window_lead_ns)
    z.zsmr_set_xcd_balance(args.xcd_balance if args.xcd_balance is not None else z.XCD_BALANCE_DEFAULT)
    ms_step, byts, (rb, wb) = time_world(args, w, owner=args.owner, prefetch=args.prefetch)
    N = w.world
    gbps = byts / ms_step / 1e6
    kname = fused_kernel_name(args, N)
    roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "traffic": read_traffic(kname, w.key, "hbm_bytes_per_step"),
            "kernel": kname, "algorithmic_bytes_per_step": byts,
            "note": "whole step (every rank's fused launch" + (", and the unit gathers" if w.stage == 3 else "")
                    + ") timed with HIP events on the compute stream"}
    rw = {"step": (rb, wb, ms_step)}
    return w.numel / (ms_step / 1e3), ms_step, roof, None, {}, rw, {
        "workload": w.name, "numel": w.numel, "world": N, "stage": w.stage, "grad_dtype": w.dtype,
        "steps_T": w.steps, "lr": w.lr, "prefetch": bool(args.prefetch and w.stage == 3),
        "stage3_layout": ("owner_broadcast" if args.owner else "per_unit_split") if w.stage == 3 else None,
        "copy_xcd_balance": {"even_permille": args.xcd_balance or z.XCD_BALANCE_DEFAULT, "tuned_over": 0}}


# The other workloads, timed after the headline in the same run: key ->
# (workload, ZeRO-3 layout owner broadcast, prefetch)
OTHER_CONFIGS = {
    "psi65k_zero2": ("psi65k", False, False),
    "gpt2s_zero2": ("gpt2s", False, False),
    "gpt2xl_zero1": ("gpt2xl", False, False),
    "llama8b_zero3_split": ("llama8b", False, False),
    "llama8b_zero3_owner": ("llama8b", True, False),
}


def other_configs(args, pure) -> dict:
    """Every other workload's whole step, at the library's default launch
    shape and write window (the copies at the XCD split this run chose):
    ms per step, parameters per second, GB/s of algorithmic bytes, its
    fraction of 8 TB/s, and its fraction of the phased bound (the least time
    its reads and writes could take at this run's pure read and write
    rates).  psi65k (65,536 parameters) is latency-bound and reported for
    completeness only."""
    import ceiling
    import workloads as wl
    import zero_sharded_mixed_reduce_amd as z

    z.zsmr_set_launch_shape()
    z.zsmr_set_write_window()
    out = {}
    for name, (key, owner, prefetch) in OTHER_CONFIGS.items():
        w = wl.WORKLOADS[key]
        if key == "psi65k":
            w = wl.Workload(w.key, w.name, w.numel, w.world, 2, w.dtype, w.grad_sigma, w.lr, w.steps)
        ms, byts, (rb, wb) = time_world(args, w, owner=owner, prefetch=prefetch)
        bound = ceiling.phased_bound(rb, wb, pure["read_GBps"], pure["write_GBps"])
        gbps = byts / ms / 1e6
        out[name] = {"workload": w.name, "ms_per_step": round(ms, 4),
                     "params_per_s": round(w.numel / (ms / 1e3), 1),
                     "algorithmic_bytes_per_step": byts, "GBps": round(gbps, 1),
                     "frac_of_8TBps": round(gbps / PEAK_HBM_GBPS, 4),
                     "phased_bound_ms": round(bound, 4), "frac_of_phased_bound": round(bound / ms, 4),
                     "fused_kernel": fused_kernel_name(args, w.world)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="share64")
    ap.add_argument("--step-bpc", type=int, default=0,
                    help="step kernels: 0 = one wave tile per wave, k = k workgroups per CU grid-stride")
    ap.add_argument("--copy-bpc", type=int, default=0,
                    help="burst copies: 0 = one 32 KB burst per wave, k = k workgroups per CU grid-stride")
    ap.add_argument("--defer-tiles", type=int, default=3, help="fused-step tiles kept in LDS per wave (0-5)")
    ap.add_argument("--defer-min-rows", type=int, default=24,
                    help="fewest gradient rows for which the fused step defers its writes")
    ap.add_argument("--window-cycle-ns", type=int, default=None,
                    help="fused step: write-window cycle (0 = no windows)")
    ap.add_argument("--window-write-ns", type=int, default=None, help="fused step: write window")
    ap.add_argument("--window-margin-ns", type=int, default=None,
                    help="fused step: no loads issued this long before a window")
    ap.add_argument("--window-lead-ns", type=int, default=None,
                    help="fused step: loads resume this long before a window ends")
    ap.add_argument("--xcd-balance", type=int, default=None,
                    help="copies: each even XCD's share against an odd one's, in thousandths "
                         "(default: tuned on the device)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="share64: skip timing the other workloads after the headline")
    ap.add_argument("--prefetch", action="store_true",
                    help="ZeRO-3 workload: gather the next unit while the current one is in use")
    ap.add_argument("--owner", action="store_true",
                    help="ZeRO-3 workload: whole units owned by single ranks (owner broadcast)")
    ap.add_argument("--unfused", action="store_true",
                    help="share64: also time the same update by the three unfused calls")
    ap.add_argument("--buckets", type=int, default=0,
                    help="share64: also measure steps with the simulated backward, bucketed")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the N ranks of the ZeRO world are simulated in "
              "that GPU's HBM, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import torch
    import workloads as wl
    import zero_sharded_mixed_reduce_amd as z

    names = ("window_cycle_ns", "window_write_ns", "window_margin_ns", "window_lead_ns")
    args.window_explicit = any(getattr(args, n) is not None for n in names)
    for name, dflt in zip(names, z.WRITE_WINDOW_DEFAULT):
        if getattr(args, name) is None:
            setattr(args, name, dflt)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    w = wl.WORKLOADS[args.workload]
    if args.workload == "share64":
        value, ms, roof, roof_fused, parts, rw, cfg = bench_share64(args, w)
    else:
        value, ms, roof, roof_fused, parts, rw, cfg = bench_world(args, w)
    torch.cuda.synchronize()
    line = {"metric": METRIC, "value": value, "unit": "params/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic", "config": cfg, "roofline": roof}
    if roof_fused is not None:
        line["roofline_fused_step"] = roof_fused
    if parts:
        line["parts"] = parts
    if rw:
        bal = cfg.get("copy_xcd_balance", {}).get("even_permille") or z.XCD_BALANCE_DEFAULT
        ref = references(z, REFERENCE_BYTES, balance=bal)
        if "peer_receive" in parts:
            line["copy_reference_GBps"] = round(ref["copy_GBps"], 1)
            line["runtime_d2d_copy_GBps"] = round(ref["runtime_copy_GBps"], 1)
            parts["peer_receive"]["frac_of_copy_reference"] = round(
                parts["peer_receive"]["GBps"] / ref["copy_GBps"], 4)
        line["phased_bound"] = phased(parts, rw, ref["pure"])
    if args.workload == "share64" and not args.no_configs and rw:
        line["other_configs"] = other_configs(args, ref["pure"])
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
