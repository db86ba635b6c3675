"""Host-side checks of bench.py (no GPU): the one-GPU guard, the roofline
arithmetic, and the rule that a committed HBM counter reading is reported only
while the kernel's sources are the ones it was taken on."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a run that did not happen


def test_roofline_fraction_is_achieved_over_peak():
    r = bench.roofline("hbm", 7044.848, bench.HBM_PEAK_GBS, "GB/s", 4483487597)
    assert r == {"bound": "hbm", "achieved": 7044.848, "peak": 8000.0, "unit": "GB/s",
                 "frac": 0.8806, "traffic": 4483487597}
    assert bench.roofline("mfma", 1200.0, bench.BF16_PEAK_TFLOPS, "TFLOP/s")["frac"] == 0.48


def test_spread_takes_min_and_90th_percentile():
    s = bench.spread([5.0, 1.0, 3.0, 2.0, 4.0, 6.0, 7.0, 8.0, 9.0, 10.0])
    assert s == {"ms_min": 1.0, "ms_p90": 10.0}


def test_kernel_source_digest_is_stable_and_distinct():
    a = bench.kernel_source_digest("fwd_varlen_kernel")
    assert a == bench.kernel_source_digest("fwd_varlen_kernel")
    assert a != bench.kernel_source_digest("fwd_dense_kernel")
    assert len(a) == 16 and int(a, 16) >= 0


def _counters(tmp_path, digest):
    path = tmp_path / "hbm_counters.json"
    path.write_text(json.dumps({"kernels": {"fwd_varlen_kernel": {"w": {
        "source_digest": digest, "hbm_bytes_per_dispatch": 123456}}}}))
    return str(path)


def test_traffic_reported_only_for_the_measured_sources(tmp_path, monkeypatch):
    current = bench.kernel_source_digest("fwd_varlen_kernel")
    monkeypatch.setattr(bench, "COUNTERS_FILE", _counters(tmp_path, current))
    assert bench.load_traffic("fwd_varlen_kernel", "w") == 123456
    assert bench.load_traffic("fwd_varlen_kernel", "other workload") is None
    monkeypatch.setattr(bench, "COUNTERS_FILE", _counters(tmp_path, "0" * 16))
    assert bench.load_traffic("fwd_varlen_kernel", "w") is None  # sources changed since
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic("fwd_varlen_kernel", "w") is None


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCES))
def test_committed_counter_files_name_existing_sources(kernel):
    for name in bench.KERNEL_SOURCES[kernel]:
        assert os.path.isfile(os.path.join(ROOT, "maxsim_scoring_amd", name)), name
