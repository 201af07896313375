"""Host logic of bench.py that needs no GPU: the shader-clock sampler's
parsing, the side kernels' algorithmic byte counts and the argument guards."""
import os
import subprocess
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_sclk_sampler_reads_the_current_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 96Mhz\n0: 500Mhz\n1: 1645Mhz *\n2: 2400Mhz\n")
    s = bench.SclkSampler(0.005)
    s.path = str(f)
    with s:
        time.sleep(0.05)
    out = s.summary()
    assert out["mean_mhz"] == 1645.0 and out["min_mhz"] == 1645.0 and out["samples"] >= 2


def test_sclk_sampler_without_a_readout_reports_nothing(tmp_path):
    s = bench.SclkSampler(0.005)
    s.path = None
    with s:
        time.sleep(0.01)
    assert s.summary() is None
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")          # no level marked current
    s = bench.SclkSampler(0.005)
    s.path = str(f)
    with s:
        time.sleep(0.02)
    assert s.summary() is None


def test_side_kernel_bytes_count_each_array_once():
    T, H, V = 1000, 1536, 151936
    n_vt = 594                                      # ceil(151936 / 256)
    assert bench.side_kernel_bytes("k_rmsnorm_fwd", T, H, V, 1) == T * H * (2 + 2)
    assert bench.side_kernel_bytes("k_rmsnorm_bwd", T, H, V, 1) == T * H * (2 + 4 + 4)
    # read: M, S per tile, z_target, mu (fp32) and the float64 scale;
    # written: logprob, lse, coef, the row factor (fp32) and a shift per tile
    assert bench.side_kernel_bytes("k_lse_combine", T, H, V, 1) == T * (
        (4 + 4) * n_vt + 4 + 4 + 8 + 4 * 4 + 4 * n_vt)
    assert bench.side_kernel_bytes("k_transpose_w", T, H, V, 1) == 2 * (2 * V * H)
    assert bench.side_kernel_bytes("k_kl", T, H, V, 2) == 2 * 8 * T
    assert bench.side_kernel_bytes("k_lmhead_fwd", T, H, V, 1) is None


@pytest.mark.parametrize("args", [["--steps", "0"], ["--warmup", "-1"], ["--cpu-tokens", "0"]])
def test_bench_rejects_bad_counts(args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True)
    assert p.returncode == 2 and "must be at least" in p.stderr


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert p.returncode == 2 and "one GPU" in p.stdout
