"""CPU checks of the benchmark's contract: one GPU only, and HBM traffic read
from a counter summary only while that summary was taken on the current
kernel source."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_read_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / "k_decode_w_pmc.md"
    path.write_text("- kernel_source_sha = %s\n- traffic_bytes_per_launch = 123456\n" % bench.kernel_source_hash())
    assert bench.read_traffic("w") == 123456.0
    path.write_text("- kernel_source_sha = 0000000000000000\n- traffic_bytes_per_launch = 123456\n")
    assert bench.read_traffic("w") is None
    assert bench.read_traffic("absent") is None
