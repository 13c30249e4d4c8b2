"""The benchmark's host-side contract, on the CPU: more than one GPU is refused with a
message and a non-zero status, and the HBM traffic of the GEMM is taken from the committed
counter summary only while the GEMM source and the launch shape match it."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""                   # no JSON line


def test_counter_traffic_follows_source_and_shape(tmp_path, monkeypatch):
    shape = (19989, 10752, 5376)
    fake = tmp_path / "summary.md"
    fake.write_text("gemm_source_sha256_16: 0000000000000000\nlaunch_shape_m_n_kpad: 19989 10752 5376\n"
                    "hbm_bytes_per_launch_calibrated: 1.0e+09\n")
    monkeypatch.setattr(bench, "PMC_PROFILE", str(fake))
    assert bench.counter_traffic(shape) is None                     # the GEMM source changed
    fake.write_text(fake.read_text().replace("0000000000000000", bench.gemm_source_hash()))
    assert bench.counter_traffic(shape) == 1.0e9
    assert bench.counter_traffic((19989, 5376, 5376)) is None       # another launch shape
    monkeypatch.setattr(bench, "PMC_PROFILE", str(tmp_path / "missing.md"))
    assert bench.counter_traffic(shape) is None
