"""bench.py's host-side contract (CPU only): the one-GPU guard, the CPU
baseline record and the traffic lookup, without touching a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_record():
    rec = bench.cpu_baseline(budget_s=0.0)     # one (batch, head) pair of the S=4096 prefill
    assert set(rec) == {"value", "unit", "cores", "kind", "sample"}
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert rec["sample"].startswith("1 whole (batch, head) pairs")


def test_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "x_traffic.json").write_text(json.dumps({"kernel_src_sha": bench._sha(str(src)),
                                                     "hbm_bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench._traffic("x", str(src)) == 123
    src.write_text("kernel v2")                  # source changed since the counters were taken
    assert bench._traffic("x", str(src)) is None
    assert bench._traffic("missing", str(src)) is None
