"""The benchmark's command-line contract: one JSON line with the fields the reporting expects,
N > 1 refused with a message, and the HBM traffic figure taken only from a profile of the same
kernel source and V layout."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_read_only_for_the_same_kernel_and_layout(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    assert bench.read_traffic("c3", "dim") is None                   # no profile
    (prof / "prefill_c3_traffic.json").write_text(json.dumps({"kernel_sha": "abc", "v_layout": "dim",
                                                              "hbm_bytes_per_launch": 123}))
    assert bench.read_traffic("c3", "dim") == 123
    assert bench.read_traffic("c3", "token") is None                 # other V layout
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "def")
    assert bench.read_traffic("c3", "dim") is None                   # other kernel source


@pytest.mark.gpu
def test_bench_prints_one_json_line():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline", "--no-layout-ab"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["value"] > 0 and d["unit"] == "TFLOP/s" and d["dtype"] == "bf16" and d["vs_baseline"] is None
    assert "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert d["speedup_vs_dense"]["kernel"] > 0
    assert d["table_build_bit_masks"]["tables_equal_byte_masks"] is True
    fu = d["fused_union"]   # the fused launches, timed in turn with the separate pair
    assert fu["outputs_equal_separate"] is True
    assert fu["step_ms"] > 0 and fu["separate_step_ms"] > 0 and fu["bit_masks_step_ms"] > 0
    mp = rf["measured_peak"]
    assert mp["achieved_tflops"] > 0 and mp["engine_clock_mhz"] > 0
