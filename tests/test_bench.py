"""Host-side checks of the benchmark's bookkeeping (no GPU)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_flop_count_matches_the_stated_workload_totals():
    """4MKN + 6Mr(K+N) per linear: 143.9 GFLOP for a 4096 x 4096 linear at
    M = 2048, r = 64, and 1.719 TFLOP for the seven LLaMA-7B linears; 8.966
    TFLOP for the seven 33B linears at M = 4096."""
    assert bench.linear_flops(2048, 4096, 4096, 64) / 1e9 == pytest.approx(143.9, abs=0.05)
    wl = workloads.WORKLOADS["llama7b"]
    tot = sum(bench.linear_flops(2048, l.N, l.K, wl.r) for l in wl.linears)
    assert tot / 1e12 == pytest.approx(1.719, abs=5e-4)
    wl = workloads.WORKLOADS["llama33b_recompute"]
    tot = sum(bench.linear_flops(4096, l.N, l.K, wl.r) for l in wl.linears)
    assert tot / 1e12 == pytest.approx(8.966, abs=5e-4)


def test_more_than_one_gpu_is_refused():
    import subprocess
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert p.returncode == 2 and "one GPU" in p.stderr
