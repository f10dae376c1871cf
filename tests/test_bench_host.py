"""Host-side logic of bench.py: the one-GPU guard and the traffic records
read from counter summaries (no GPU needed)."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_text("kernel source v1\n")
    (tmp_path / "k.h").write_text("header\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _record(root, launch, workload, nbytes):
    digest = hashlib.sha256((root / "k.hip").read_bytes() + (root / "k.h").read_bytes()).hexdigest()
    return (f"traffic-record: launch={launch} workload={workload} kernel=k sources=k.hip+k.h "
            f"sha256={digest} bytes={nbytes}\n")


def test_traffic_record_found_for_its_launch_and_workload(fake_root):
    (fake_root / "profiles" / "k_w_counters.md").write_text(
        "# counters\n\n" + _record(fake_root, "gemm", "w", 123456) + _record(fake_root, "reduce", "w", 77))
    assert bench.recorded_traffic("gemm", "w") == 123456.0
    assert bench.recorded_traffic("reduce", "w") == 77.0
    assert bench.recorded_traffic("gemm", "other") is None
    assert bench.recorded_traffic("fused", "w") is None


def test_traffic_record_dropped_once_the_kernel_changes(fake_root):
    (fake_root / "profiles" / "k_w_counters.md").write_text(_record(fake_root, "gemm", "w", 5))
    assert bench.recorded_traffic("gemm", "w") == 5.0
    (fake_root / "k.hip").write_text("kernel source v2\n")
    assert bench.recorded_traffic("gemm", "w") is None


def test_traffic_record_with_missing_source_is_ignored(fake_root):
    (fake_root / "profiles" / "k_w_counters.md").write_text(_record(fake_root, "gemm", "w", 5))
    os.remove(fake_root / "k.h")
    assert bench.recorded_traffic("gemm", "w") is None


def test_rate_hbm_prefers_the_cache_cold_figure():
    """For an HBM-bound launch whose data would fit in the Infinity Cache the
    figure is the one measured over rotating buffer copies; the same-buffer
    (warm) rate is kept apart. Without a cold figure the back-to-back one is
    reported as is."""
    import bench

    r = bench.rate("hbm", 8e9, 2.0, cold_ms=4.0)
    assert r["achieved"] == 2000.0 and r["frac"] == 0.25 and r["avg_ms"] == 4.0
    assert r["warm_achieved"] == 4000.0 and r["warm_avg_ms"] == 2.0
    assert r["cache"] == "rotating copies"
    w = bench.rate("hbm", 8e9, 2.0)
    assert w["achieved"] == 4000.0 and "warm_achieved" not in w
    assert w["cache"] == "footprint over 512 MiB"
    g = bench.rate("mfma", 2.5166e15, 1000.0)
    assert g["achieved"] == 2516.6 and g["frac"] == 1.0
