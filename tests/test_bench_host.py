"""Host checks of bench.py's contract (no GPU): the single-GPU refusal, the
workload table and the HBM traffic record's guard."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_headline_workload_and_units():
    assert "fp32_transpose" in bench.WORKLOADS
    for name in ("bf16_gemm", "bf16_gemm_fused", "bf16_gemm_fused_bf16c", "map_batch", "u8_narrow16"):
        assert name in bench.WORKLOADS, name


def test_traffic_bytes_only_while_the_kernel_sources_match(tmp_path, monkeypatch):
    """bench.py reports counter bytes only from a record taken on the kernel
    sources as they are now (same digest); a stale record gives null."""
    rec = {"workloads": {"fp32_transpose": {"bytes_per_launch": 123}}}
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(json.dumps(dict(rec, kernel_sources_sha256=bench.kernel_sources_digest())))
    assert bench.measured_traffic("fp32_transpose") == 123
    assert bench.measured_traffic("no_such_workload") is None
    f.write_text(json.dumps(dict(rec, kernel_sources_sha256="0" * 64)))
    assert bench.measured_traffic("fp32_transpose") is None
    f.write_text("not json")
    assert bench.measured_traffic("fp32_transpose") is None
