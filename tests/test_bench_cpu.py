"""Host-side parts of bench.py that run without a GPU: the one-GPU refusal,
the CPU baseline's report, and the source hash that gates the counter
figures."""
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_times_the_oracle_on_a_bounded_sample():
    w = types.SimpleNamespace(seed=0, world=4, grad_sigma=1e-3, dtype="bf16", steps=2, lr=1e-4,
                              betas=(0.9, 0.999), eps=1e-8)
    out = bench.cpu_baseline(w, window=512, min_seconds=0.05, threads=2)
    assert out["kind"] == "oracle" and out["unit"] == "params/s" and out["cores"] == 2
    assert out["value"] > 0
    assert "2 windows of 512" in out["sample"]


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    """A counter summary whose recorded hash differs from the current sources
    gives no traffic figure; a matching one gives its bytes."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    path = prof / "k_w_pmc.txt"
    path.write_text("# comment: 1\nhbm_bytes_per_launch: 1234\n"
                    "kernel_and_workload_source_sha256_16: 0000000000000000\n")
    assert bench.read_traffic("k", "w") is None
    path.write_text("hbm_bytes_per_launch: 1234\n"
                    f"kernel_and_workload_source_sha256_16: {bench.kernel_source_hash()}\n")
    assert bench.read_traffic("k", "w") == 1234
    assert bench.read_traffic("missing", "w") is None


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    hip, py = tmp_path / "k.hip", tmp_path / "w.py"
    hip.write_text("// a kernel\n__global__ void k(int* p) { p[0] = 1; }  /* tail */\n")
    py.write_text('"""Doc."""\nX = 1  # comment\n\ndef f():\n    """Doc."""\n    return X\n')
    monkeypatch.setattr(bench, "TRAFFIC_SOURCES", (str(hip), str(py)))
    h0 = bench.kernel_source_hash()
    hip.write_text("// another comment\n__global__ void k(int* p) {\n  p[0] = 1;\n}\n")
    py.write_text('"""Other doc."""\nX = 1\n\ndef f():\n    return X  # other\n')
    assert bench.kernel_source_hash() == h0
    hip.write_text("__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.kernel_source_hash() != h0
    hip.write_text("__global__ void k(int* p) { p[0] = 1; }\n")
    assert bench.kernel_source_hash() == h0
    py.write_text("X = 2\n\ndef f():\n    return X\n")
    assert bench.kernel_source_hash() != h0


def test_phased_bound_report():
    pure = {"read_GBps": 7000.0, "write_GBps": 6000.0, "read": {"bursts": 7000.0},
            "write": {"bursts_nt": 6000.0}, "bytes": 16}
    out = bench.phased({}, {"step": (7_000_000_000, 3_000_000_000, 2.0)}, pure)
    assert out["step"]["bound_ms"] == 1.5 and out["step"]["measured_ms"] == 2.0
    assert out["step"]["frac"] == 0.75
    assert out["read_GBps"] == 7000.0 and out["write_GBps"] == 6000.0
