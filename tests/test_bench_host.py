"""Host-side logic of bench.py (no GPU): the profile-backed traffic figure,
the clock summary and the multi-GPU refusal."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_recorded_traffic_tracks_the_gemm_code(tmp_path, monkeypatch):
    src = tmp_path / "gemm.hip"
    src.write_text("// kernel v1\nint f() { return 1; }\n")
    sha = bench.code_sha256(str(src))
    prof = tmp_path / "prof.txt"
    prof.write_text("# header: ignored\n"
                    f"code_sha256: {sha}   (at collection time)\n"
                    "traffic_bytes_per_launch: 6.25e+08\n")
    monkeypatch.setattr(bench, "GEMM_SOURCE", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.recorded_traffic() == 6.25e8
    src.write_text("/* reworded */ // kernel v1, same code\nint f()  {\n  return 1; }\n")
    assert bench.recorded_traffic() == 6.25e8      # commentary and layout only
    src.write_text("// kernel v1\nint f() { return 2; }\n")
    assert bench.recorded_traffic() is None         # the code changed since the counters
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.txt"))
    assert bench.recorded_traffic() is None


def test_clock_summary():
    c = bench.ClockSampler()
    c.samples = [(1800.0, 1300.0, 1900.0), (1700.0, None, None), (1750.0, 1400.0, 1800.0)]
    s = c.summary(1300.0)
    assert s["readings"] == 3 and s["sclk_mhz_mean"] == 1750.0
    assert s["sclk_mhz_min"] == 1700.0 and s["sclk_mhz_max"] == 1800.0
    assert s["socket_power_w_mean"] == 1350.0
    assert s["mclk_mhz_mean"] == 1850.0
    peak = bench.PEAK_BF16_TFLOPS * 1750.0 / bench.SPEC_SCLK_MHZ
    assert s["mfma_peak_at_mean_clock"] == round(peak, 1)
    assert s["roofline_frac_at_mean_clock"] == round(1300.0 / peak, 4)
    empty = bench.ClockSampler()
    empty.err = "no SMI"
    assert empty.summary(1.0) == {"source": "amdsmi gpu_metrics", "readings": 0, "error": "no SMI"}


def test_clock_sampler_without_a_card_records_nothing():
    c = bench.ClockSampler()
    with c:
        pass
    s = c.summary(1.0)
    assert s["readings"] == 0 or s["sclk_mhz_mean"] > 0


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
