"""Host-side pieces of bench.py: the one-GPU guard, traffic ageing, row fields."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    # the guard runs before anything imports torch or touches a device
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_measured_traffic_is_null_once_the_kernel_source_changes(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    good = bench.source_hash("k_alltoall")
    f.write_text(json.dumps({"k_alltoall:w": {"bytes_per_launch": 123, "source_hash": good},
                             "k_alltoall:stale": {"bytes_per_launch": 456, "source_hash": "0" * 16}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("k_alltoall", "w") == 123
    assert bench.measured_traffic("k_alltoall", "stale") is None
    assert bench.measured_traffic("k_alltoall", "missing") is None


def test_source_hash_covers_the_kernel_file_and_the_device_header():
    # one hash per kernel source; kernels built from one file share it
    assert bench.source_hash("k_dispatch") == bench.source_hash("k_dispatch_dedup")
    assert bench.source_hash("k_dispatch") != bench.source_hash("k_alltoall")


def test_row_entry_reports_both_timings():
    t = bench.Times([2.0, 1.0, 3.0])
    t.b2b_ms = 0.5
    d = bench.row_entry("x", 8_000_000_000, t, "k_put", "none")
    assert d["median_ms"] == 2.0 and d["min_ms"] == 1.0
    assert d["GBps"] == pytest.approx(4000.0)
    assert d["frac_of_peak"] == pytest.approx(0.5)
    assert d["back_to_back_ms"] == 0.5
    assert d["back_to_back_GBps"] == pytest.approx(16000.0)
    plain = bench.row_entry("y", 1000, [1.0], "k_put", "none")
    assert "back_to_back_ms" not in plain
