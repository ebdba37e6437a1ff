"""Build the gfx950 shared libraries in-tree with hipcc.

* ``zero_sharded_mixed_reduce_amd/libzsmr.so`` -- the ZeRO shard step (C ABI in
  ``include/zsmr.h``).
* ``synth/libzsmr_synth.so`` -- the GPU fill kernels of the seeded input
  generator (C ABI in ``include/zsmr_synth.h``).
* ``ceiling/libzsmr_ceiling.so`` -- pure-read and pure-write reference
  streams for the benchmark (C ABI in ``include/zsmr_ceiling.h``).

Every HIP source is compiled for gfx950 only, with floating-point contraction
off (the method's Adam is specified one rounding per operation) and with
packed fp32 instructions disabled.  hipcc cross-compiles without a GPU.

Usage: ``python -m zero_sharded_mixed_reduce_amd.build``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")

LIB = os.path.join(PKG, "libzsmr.so")
SYNTH_LIB = os.path.join(ROOT, "synth", "libzsmr_synth.so")
CEILING_LIB = os.path.join(ROOT, "ceiling", "libzsmr_ceiling.so")


def hipcc() -> str:
    env = os.environ.get("HIPCC")
    if env:
        return env
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP libraries)")


def common_flags(extra=()):
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-I", INCLUDE, "-I", CSRC, *extra]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _build(out, sources, extra=()):
    tmp = out + ".tmp"
    _run([hipcc(), *common_flags(extra), *sources, "-o", tmp])
    os.replace(tmp, out)


def build_lib(extra=()):
    _build(LIB, [os.path.join(CSRC, "zsmr_kernels.hip"), os.path.join(CSRC, "zsmr_api.cpp")], extra)
    return LIB


def build_synth(extra=()):
    _build(SYNTH_LIB, [os.path.join(ROOT, "synth", "synth_fill.hip")], extra)
    return SYNTH_LIB


def build_ceiling(extra=()):
    _build(CEILING_LIB, [os.path.join(ROOT, "ceiling", "ceiling.hip")], extra)
    return CEILING_LIB


def build_all():
    build_lib()
    build_synth()
    build_ceiling()


if __name__ == "__main__":
    build_all()
    sys.exit(0)
