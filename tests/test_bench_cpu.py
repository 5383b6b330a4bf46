"""bench.py's host-side contract, without a GPU: the measured HBM traffic is
reported only for the kernel source, tile and launch grouping it was
measured on; the kernel name follows the persistent kernel's launch rule;
more than one GPU is refused with a message."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_measured_traffic_is_tied_to_source_tile_and_group(monkeypatch):
    name = "80666x28672x5376 per-row+bias"
    t = bench.MEASURED_TRAFFIC[name]
    monkeypatch.setattr(bench, "kernel_sha256", lambda: t["source_sha256"])
    assert bench.measured_traffic(name, t["tile"], t["group_m"]) == t["fetch_bytes"] + t["write_bytes"]
    assert bench.measured_traffic(name, t["tile"] - 1, t["group_m"]) is None
    assert bench.measured_traffic(name, t["tile"], t["group_m"] + 1) is None
    assert bench.measured_traffic("4096x4096x4096 tensorwise", t["tile"], t["group_m"]) is None
    monkeypatch.setattr(bench, "kernel_sha256", lambda: "0" * 64)
    assert bench.measured_traffic(name, t["tile"], t["group_m"]) is None


def test_measured_traffic_is_above_the_algorithmic_bytes():
    """What the counters saw can only exceed what the GEMM must move."""
    t = bench.MEASURED_TRAFFIC["80666x28672x5376 per-row+bias"]
    m, n, k = 80666, 28672, 5376
    alg = m * k + n * k + 4.0 * (m + n) + 2.0 * n + 2.0 * m * n
    assert t["write_bytes"] >= 2.0 * m * n
    assert t["fetch_bytes"] + t["write_bytes"] > alg


def test_kernel_name_rule():
    base = {"m": 80666, "n": 28672, "k": 5376, "bm": 256, "bn": 256, "tile": 13}
    assert bench.gemm_kernel_name(base) == "gemm_persist_kernel"
    assert bench.gemm_kernel_name(dict(base, k=5384)) == "gemm_dma_kernel"        # k % 128 != 0
    assert bench.gemm_kernel_name(dict(base, m=4096, n=4096)) == "gemm_dma_kernel"  # 256 tiles
    assert bench.gemm_kernel_name(dict(base, tile=12)) == "gemm_dma_kernel"


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
