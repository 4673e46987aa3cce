"""CPU checks of bench.py's host logic: the one-GPU guard, the kernel-source hash that gates the
committed HBM-traffic counters, the counters' lookup, the oracle's CPU-baseline leg and the
summary fields of a timed case.  No GPU is touched."""
import json
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def _tree_copy(tmp_path):
    csrc = tmp_path / "fp8_linear_layer_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("gemm.hip", "cast.hip"):
        shutil.copy(os.path.join(ROOT, "fp8_linear_layer_amd", "csrc", f), csrc / f)
    return csrc


def test_kernel_hash_ignores_comments_and_blank_space_but_not_code(tmp_path, monkeypatch):
    base = bench.kernel_hash()
    csrc = _tree_copy(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_hash() == base
    g = csrc / "gemm.hip"
    src = g.read_text()
    g.write_text("// a new comment line\n/* and a block\n   comment */\n\n" + src.replace("\n", "\n\n", 3) + "\n   \n")
    assert bench.kernel_hash() == base, "a comment or blank-space edit changed the hash"
    g.write_text(src + "\nnamespace { int hash_probe; }\n")
    assert bench.kernel_hash() != base, "a code edit left the hash unchanged"


def test_traffic_is_reported_only_for_the_profiled_source(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.json")) as f:
        rec = json.load(f)
    key = "wgrad_full_7168x2112x4096"
    want = rec["kernels"][key]["hbm_bytes_per_launch"]
    assert isinstance(want, int) and want > 0
    monkeypatch.setattr(bench, "kernel_hash", lambda: rec["kernel_source_hash"])
    assert bench.traffic_from_profile(key) == want
    assert bench.traffic_from_profile("no_such_kernel") is None
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.traffic_from_profile(key) is None, "counters of another kernel source were used"


def test_cpu_baseline_runs_the_oracle_on_a_bounded_sample():
    r = bench.cpu_baseline(rows=1, min_seconds=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert r["sample"].startswith("1 of 7168 output rows")


def test_case_summary_fields():
    case = bench.Case(lambda: None, 2.0e12, nbytes=4.0e9, note="n")
    rec = bench._summ(case, [1.0, 2.0, 3.0])
    assert rec["ms"] == 2.0 and rec["rounds"] == 3
    assert rec["tflops"] == pytest.approx(2.0e12 / 2.0 / 1e9, rel=1e-3)
    assert rec["frac_fp8_peak"] == pytest.approx(rec["tflops"] / bench.MFMA_FP8_PEAK_TFLOPS, rel=1e-3)
    assert rec["gbs"] == pytest.approx(4.0e9 / 2.0 / 1e6, rel=1e-3)
    assert rec["note"] == "n"
    assert rec["p10_ms"] <= rec["ms"] <= rec["p90_ms"]
    np.testing.assert_allclose(rec["frac_hbm"], rec["gbs"] / bench.HBM_PEAK_GBS, rtol=1e-3)
