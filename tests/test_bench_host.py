"""bench.py's host logic on the CPU: the one-GPU contract, the FLOP counts
the metric divides by, the check that ties recorded counters to the kernel
sources they were taken on, and the clock reader's parsing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "ONE GPU" in r.stderr
    assert r.stdout == ""


def test_flops_of_the_swiglu_shard_step():
    # nine products of 2 N H F/T FLOPs each: FC1 gate|up (2), FC2, dH, dB,
    # dA|dA_up (2), dX over [dG|dU] (2)
    w = wl.WORKLOADS["c4_bf16_swiglu_fwdbwd"]
    f = bench.role_flops(w)
    per = 2.0 * 4096 * 8192 * 3584
    assert f == {"FC1": 2 * per, "FC2": per, "dH": per, "dB": per, "dA": 2 * per,
                 "dX": 2 * per}
    assert abs(bench.gemm_flops(w) / 1e9 - 2164.7) < 0.1


def test_flops_of_the_gelu_shards():
    c2 = wl.WORKLOADS["c2_bf16_gelu_fwd"]
    assert abs(bench.gemm_flops(c2) / 1e9 - 274.9) < 0.1      # forward only
    c3 = wl.WORKLOADS["c3_bf16_gelu_fwdbwd"]
    assert abs(bench.gemm_flops(c3) / 1e9 - 824.6) < 0.1


def test_recorded_counters_must_match_the_sources(tmp_path):
    good = tmp_path / "good.txt"
    good.write_text("# comment: not a field\nhbm_bytes_FC1: 123\n"
                    f"kernel_source_hash: {bench.kernel_source_hash()}\n")
    assert bench.recorded_fields(str(good))["hbm_bytes_FC1"] == "123"
    stale = tmp_path / "stale.txt"
    stale.write_text("hbm_bytes_FC1: 123\nkernel_source_hash: 0000000000000000\n")
    assert bench.recorded_fields(str(stale)) is None
    assert bench.recorded_fields(str(tmp_path / "missing.txt")) is None


def test_clock_reader_takes_the_current_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1763Mhz *\n2: 2400Mhz\n")
    cs = bench.ClockSampler.__new__(bench.ClockSampler)
    cs.sysfs = str(f)
    assert cs._read_sysfs() == 1763.0
    f.write_text("S: 128Mhz *\n0: 500Mhz\n")
    assert cs._read_sysfs() == 128.0
    # implausible medians (an idle reading) are reported as None
    assert bench.ClockSampler._median_ghz([128.0] * 10) is None
    assert bench.ClockSampler._median_ghz([1800.0] * 10) == pytest.approx(1.8)
    assert bench.ClockSampler._median_ghz([1800.0] * 3) is None   # too few samples
