"""bench.py's output contract on the GPU: one JSON line with the metric, the
whole-step value, the roofline of the dominant kernel (with counter traffic
when the committed summaries match the sources), the phased bound and the
copy references, for the default workload."""
import json
import os
import subprocess
import sys

import pytest

from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_complete_json_line():
    say("[bench] share64, 2 steps")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "phased_bound"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["unit"] == "params/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "one_rank_share_psi7.5e9_n64_zero2_bf16"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert 0 < roof["frac"] <= 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    for part in ("fused_step", "peer_receive", "step"):
        assert 0 < d["phased_bound"][part]["frac"] < 1.2
    assert d["copy_reference_GBps"] > 0 and d["runtime_d2d_copy_GBps"] > 0
    bal = d["config"]["copy_xcd_balance"]                 # tuned on the device
    assert 1000 <= bal["even_permille"] <= 1300 and bal["tuned_over"] == 6
    win = d["config"]["fused_write_window_ns"]
    assert win["tuned_over"] > 0 and win["write"] + win["margin"] < win["cycle"]
    shapes = d["phased_bound"]
    assert "bursts_balanced" in shapes["read_shapes_GBps"]
    assert "bursts_plain_balanced" in shapes["write_shapes_GBps"]
    # the same step at the library's untuned defaults, beside the tuned one
    untuned = d["parts"]["step_at_library_defaults"]
    assert untuned["ms"] > 0 and 0 < untuned["frac"] < 1
    # every other workload, timed in the same run
    oc = d["other_configs"]
    assert set(oc) == {"psi65k_zero2", "gpt2s_zero2", "gpt2xl_zero1", "llama8b_zero3_split",
                       "llama8b_zero3_owner"}
    for name, v in oc.items():
        assert v["ms_per_step"] > 0 and v["params_per_s"] > 0, name
        assert 0 < v["frac_of_8TBps"] < 1 and 0 < v["frac_of_phased_bound"] < 1.2, name
        assert abs(v["GBps"] - v["algorithmic_bytes_per_step"] / v["ms_per_step"] / 1e6) < 1, name
