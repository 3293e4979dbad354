"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the percentile summary, and the
rule that a GEMM's HBM traffic is reported only while its counters were taken on the current
kernel sources."""
import os
import shutil
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""


def test_percentiles():
    v = np.arange(1, 101, dtype=np.float64) / 1000.0  # 0.001 .. 0.100 ms
    p = bench.percentiles(v)
    assert p["n"] == 100
    assert p["mean"] == round(float(v.mean()), 4)
    assert p["p10"] == round(float(np.percentile(v, 10)), 4)
    assert p["p50"] == round(float(np.percentile(v, 50)), 4)
    assert p["p90"] == round(float(np.percentile(v, 90)), 4)


def test_traffic_reported_only_for_the_measured_sources(tmp_path, monkeypatch):
    # a copy of the GEMM sources and one counter summary in a scratch tree
    src = os.path.join(ROOT, "w4a4_quantized_dit_amd", "csrc")
    dst = tmp_path / "w4a4_quantized_dit_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in bench.GEMM_SOURCES["attn"]:
        shutil.copy(os.path.join(src, f), dst / f)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    name = bench.workload_config("attn")["name"]
    prof = tmp_path / "profiles" / f"k_gemm_nvfp4_{name}_traffic.md"
    digest = bench.source_digest(bench.GEMM_SOURCES["attn"])
    prof.write_text(f"- kernel source digest: `{digest}`\n- traffic bytes per launch: `5.5e+08`\n")
    assert bench.measured_traffic("attn") == 5.5e8
    # any change to a digested source makes the figure stale
    with open(dst / bench.GEMM_SOURCES["attn"][0], "a") as fh:
        fh.write("\n")
    assert bench.measured_traffic("attn") is None
    # no summary at all
    prof.unlink()
    assert bench.measured_traffic("attn") is None
