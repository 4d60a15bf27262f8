"""Host-side pieces of bench.py (no GPU): the one-GPU guard, the
source-hash gate on the counter-measured traffic, and the CPU-oracle
baseline on a tiny shape."""
import hashlib
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_only_for_the_profiled_source(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "profile.txt"
    prof.write_text(f"header line\nsource_sha256: {digest}\nfetch_bytes: 10\n"
                    f"write_bytes: 5\ntraffic_bytes: 15\n")
    assert bench.measured_traffic(str(prof), str(src)) == 15
    src.write_text("// kernel v2\n")  # the kernel changed since the counters were taken
    assert bench.measured_traffic(str(prof), str(src)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.txt"), str(src)) is None


def test_cpu_baseline_tiny_shape():
    rng = np.random.default_rng(0)
    M, N, K = 512, 1024, 256
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    out = bench.cpu_baseline(a, w, 0, -6, M, N, K, 0.5)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert out["quantize_W_GB/s"] > 0 and out["quantize_W_GB/s_1core"] > 0
    assert "sample" in out
