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


def test_sclk_sampler_reads_board_power_in_watts(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1645Mhz *\n")
    p = tmp_path / "power1_average"
    p.write_text("1400000000\n")                  # microwatts
    s = bench.SclkSampler(0.005)
    s.path, s.power_path, s.cap_w = str(f), str(p), 1400.0
    with s:
        time.sleep(0.05)
    out = s.summary()
    assert out["board_power"]["mean_w"] == 1400.0 and out["board_power"]["cap_w"] == 1400.0
    assert bench.SclkSampler._read_w(str(tmp_path / "absent")) is None


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


def _counter_csv(path, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(w.fieldnames, r)))


def test_summarize_counters_scales_by_the_copy_and_maps_kernels(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE arrive in KiB per dispatch and are divided by
    what the calibration copy reads; the DRAM request counters are divided by
    the copy's requests per byte.  The persistent forward's dispatches are
    the forward's, and k_dw adds the row scaling to the token contraction."""
    C = bench.CALIBRATION_BYTES
    kib = 1024.0
    copy = "__amd_rocclr_copyBuffer"
    fwd = "void rz::k_lmhead_fwd_p<true>(unsigned short const*, ...)"
    fetch = [(1, copy, "FETCH_SIZE", 0.5 * C / kib),
             (2, fwd, "FETCH_SIZE", 0.5 * 3e9 / kib), (3, fwd, "FETCH_SIZE", 0.5 * 5e9 / kib),
             (4, "rz::k_dhidden(...)", "FETCH_SIZE", 0.5 * 2e9 / kib),
             (5, "rz::k_scale_rows_t(...)", "FETCH_SIZE", 0.5 * 1e9 / kib),
             (6, "rz::k_dw_tr(...)", "FETCH_SIZE", 0.5 * 7e9 / kib)]
    write = [(1, copy, "WRITE_SIZE", C / kib), (2, fwd, "WRITE_SIZE", 1e9 / kib),
             (3, fwd, "WRITE_SIZE", 1e9 / kib), (4, "rz::k_dhidden(...)", "WRITE_SIZE", 2e9 / kib),
             (5, "rz::k_scale_rows_t(...)", "WRITE_SIZE", 0.0),
             (6, "rz::k_dw_tr(...)", "WRITE_SIZE", 4e9 / kib)]
    dram = [(1, copy, "TCC_EA0_RDREQ_DRAM_sum", C / 128), (1, copy, "TCC_EA0_WRREQ_DRAM_sum", C / 64),
            (2, fwd, "TCC_EA0_RDREQ_DRAM_sum", 6e9 / 128), (2, fwd, "TCC_EA0_WRREQ_DRAM_sum", 2e9 / 64),
            (3, fwd, "TCC_EA0_RDREQ_DRAM_sum", 2e9 / 128), (3, fwd, "TCC_EA0_WRREQ_DRAM_sum", 0.0)]
    paths = [str(tmp_path / n) for n in ("f.csv", "w.csv", "d.csv")]
    for p, rows in zip(paths, (fetch, write, dram)):
        _counter_csv(p, rows)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    bench.summarize_counters(*paths)
    import json
    f = json.load(open(tmp_path / "profiles" / "traffic_k_lmhead_fwd.json"))
    assert f["launches"] == 2
    assert abs(f["fetch_bytes_per_launch"] - 4e9) < 1e3
    assert abs(f["write_bytes_per_launch"] - 1e9) < 1e3
    assert abs(f["dram_read_bytes_per_launch"] - 4e9) < 1e3
    assert abs(f["dram_write_bytes_per_launch"] - 1e9) < 1e3
    assert f["source_sha"] == bench.source_sha()
    d = json.load(open(tmp_path / "profiles" / "traffic_k_dhidden.json"))
    assert abs(d["bytes_per_launch"] - 4e9) < 1e3 and "dram_read_bytes_per_launch" not in d
    w = json.load(open(tmp_path / "profiles" / "traffic_k_dw.json"))
    assert abs(w["fetch_bytes_per_launch"] - 8e9) < 1e3
    assert abs(w["write_bytes_per_launch"] - 4e9) < 1e3


@pytest.mark.parametrize("args", [["--decode", "--stored"], ["--decode", "--grads"],
                                  ["--probe", "--shards", "2"]])
def test_bench_rejects_two_modes(args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True)
    assert p.returncode == 2 and "each time their own pass" in p.stderr
