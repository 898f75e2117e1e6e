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


def _counter_csv(folder, counter, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "pmc_counter_collection.csv"), "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, value in rows:
            f.write(f'"{name}",{counter},{value}\n')


def test_traffic_record_scales_counters_by_the_calibration_copy(tmp_path):
    """FETCH_SIZE reads half of a 1 GiB copy's bytes here (scale 2), WRITE_SIZE
    all of them (scale 1); a GEMM reading 1000 KiB and writing 300 KiB per
    dispatch (mean of two) then moved 2.0e6 + 0.3e6 KiB-scaled bytes, and the
    record carries the hash of the kernel's own sources."""
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel>(int)"
    fwd = "void qnf4::k_fwd_gemm<0>(unsigned short const*, long)"
    _counter_csv(fetch, "FETCH_SIZE", [(neg, 524288.0), (fwd, 900.0), (fwd, 1100.0)])
    _counter_csv(write, "WRITE_SIZE", [(neg, 1048576.0), (fwd, 300.0), (fwd, 300.0)])
    out = bench.write_traffic(fetch, write, 1024, "test", path=str(tmp_path / "t.json"))
    rec = out["k_fwd_gemm"]
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["bytes_per_launch"] == pytest.approx(1000 * 1024 * 2 + 300 * 1024)
    assert rec["src_hash"] == bench.kernel_source_hash("k_fwd_gemm")
    assert bench.kernel_source_hash("k_fwd_gemm") != bench.kernel_source_hash("k_dx_gemm")


def test_traffic_record_leaves_the_counter_files_alone(tmp_path):
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel>(int)"
    dx = "void qnf4::k_dx_gemm<0>(unsigned short const*, long)"
    _counter_csv(fetch, "FETCH_SIZE", [(neg, 524288.0), (dx, 10.0)])
    _counter_csv(write, "WRITE_SIZE", [(neg, 1048576.0), (dx, 5.0)])
    before = open(os.path.join(write, "pmc_counter_collection.csv")).read()
    bench.write_traffic(fetch, write, 1024, "test", path=str(tmp_path / "t.json"))
    assert open(os.path.join(write, "pmc_counter_collection.csv")).read() == before
    assert set(bench.json.load(open(tmp_path / "t.json"))) == {"k_dx_gemm"}


def test_decode_filters_parse_and_reject_what_the_sweep_lacks():
    assert bench._int_list("1,16") == [1, 16]
    assert bench._shape_list("22016x8192") == ["22016x8192"]
    for bad in ("0", "17", "", "1,32"):
        with pytest.raises(bench.argparse.ArgumentTypeError):
            bench._int_list(bad)
    for bad in ("4096x4096", "8192x8192,1x1", ""):
        with pytest.raises(bench.argparse.ArgumentTypeError):
            bench._shape_list(bad)


def test_decode_filters_need_decode_only():
    import subprocess
    p = subprocess.run([sys.executable, bench.__file__, "--decode-m", "1"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode != 0 and "--decode-only" in p.stderr
