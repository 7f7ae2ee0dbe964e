"""Host checks of bench.py's contract (no GPU): the single-GPU refusal, the
workload table and the HBM traffic record's guard."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import pytest  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_headline_workload_and_units():
    assert "fp32_transpose" in bench.WORKLOADS
    for name in ("bf16_gemm", "bf16_gemm_fused", "bf16_gemm_fused_bf16c", "map_batch", "u8_narrow16", "fp32_rows3",
                 "u8_rows48"):
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


def test_conflict_counters_equal_the_models_prediction_for_every_layout():
    """The recorded SQ_LDS_BANK_CONFLICT readings (rocprofv3, one record per
    workload and layout) equal, per tile, what swz_predict_conflicts predicts
    under the built-in gfx950 bank model -- zero for every swizzled and
    direct-fill kernel ("CuTe Swizzle 学习手册", ⑥: verify with a measured
    count that the swizzle removes the conflicts)."""
    import tiled_movement_amd as T

    with open(bench.CONFLICT_FILE) as f:
        rec = json.load(f)
    rows = {"fp32_rows3", "u8_rows48"}
    assert len(rec["workloads"]) == 11 and rows <= set(rec["workloads"])
    for wname, layouts in rec["workloads"].items():
        if wname in rows:  # the flat-row kind: its reads depend on the width, so no per-kind prediction
            assert set(layouts) == {"swizzle", "plain"}, wname
            sw, pl = layouts["swizzle"], layouts["plain"]
            assert sw["conflict_cycles_per_lds_instr"] < 1e-3, wname
            assert sw["SQ_LDS_BANK_CONFLICT"] <= pl["SQ_LDS_BANK_CONFLICT"], wname
            continue
        assert set(layouts) == {"swizzle", "pad", "plain", "direct"}, wname
        for layout, r in layouts.items():
            w, rd = T.swz_predict_conflicts(r["read_kind"], layout)
            assert r["conflict_cycles_per_tile"] == pytest.approx(w + rd, abs=0.5), (wname, layout)
            if layout in ("swizzle", "direct"):
                assert r["SQ_LDS_BANK_CONFLICT"] == 0, (wname, layout)


def test_conflicts_reported_only_while_the_kernel_sources_match(tmp_path, monkeypatch):
    rec = {"workloads": {"fp32_transpose": {"swizzle": {"conflict_cycles_per_tile": 0.0, "conflict_cycles_per_lds_instr": 0.0,
                                                        "SQ_LDS_BANK_CONFLICT": 0, "SQ_LDS_IDX_ACTIVE": 1,
                                                        "SQ_INSTS_LDS": 1}}}}
    f = tmp_path / "lds.json"
    monkeypatch.setattr(bench, "CONFLICT_FILE", str(f))
    f.write_text(json.dumps(dict(rec, kernel_sources_sha256=bench.kernel_sources_digest())))
    assert bench.measured_conflicts("fp32_transpose")["swizzle"]["conflict_cycles_per_tile"] == 0.0
    assert bench.measured_conflicts("bf16_stage") is None
    f.write_text(json.dumps(dict(rec, kernel_sources_sha256="0" * 64)))
    assert bench.measured_conflicts("fp32_transpose") is None


def test_source_digest_follows_code_not_comments():
    """The counter records stay valid across comment edits of the kernel
    sources and go stale on any change of the code."""
    src = "int f(int x) {  // one\n  /* two\n three */ return x ^ 3;\n}\n"
    assert bench.code_text(src) == bench.code_text(src.replace("// one", "// changed").replace("two", "other"))
    assert bench.code_text(src) == "int f(int x) {\n   return x ^ 3;\n}"
    assert bench.code_text(src) != bench.code_text(src.replace("x ^ 3", "x ^ 5"))
