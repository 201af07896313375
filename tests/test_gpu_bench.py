"""The benchmark's one JSON line, on the Tiny workload: every field the
results are read from is present and consistent."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line(gpu):
    say("bench.py --config tiny --steps 3 --warmup 1 --cpu-tokens 64")
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny",
                        "--steps", "3", "--warmup", "1", "--cpu-tokens", "64"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, p.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline", "kernels", "side_kernels"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    T = d["config"]["T"]
    assert abs(d["value"] - T / (d["ms_per_step"] / 1000.0)) <= 1e-6 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-9
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["cpu_model"] and cb["affinity_cores"] >= 1
    for k, v in d["side_kernels"].items():
        assert v["achieved_GBps"] > 0 and v["ms_per_step"] > 0, k


def _one_line(args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny",
                        "--no-cpu-baseline", *args], capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, p.stdout
    return json.loads(lines[0])


def test_bench_decode_line(gpu):
    say("bench.py --config tiny --decode --steps 3 --warmup 1")
    d = _one_line(["--decode", "--steps", "3", "--warmup", "1"])
    assert d["unit"] == "us" and d["higher_is_better"] is False
    assert d["value"] == d["per_T"]["1"]["us_per_call"] > 0
    assert set(d["per_T"]) == {"1", "8", "64", "128", "256"}   # the Tiny workload: 345 rows
    assert all(v["bits_equal_full_batch"] for v in d["per_T"].values())
    r = d["roofline"]
    assert r["bound"] == "hbm" and abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-9


def test_bench_stored_line(gpu):
    say("bench.py --config tiny --stored --steps 3 --warmup 1")
    d = _one_line(["--stored", "--steps", "3", "--warmup", "1"])
    assert d["bits_equal_rz_learner_step"] is True
    T = d["config"]["T"]
    assert abs(d["value"] - T / (d["ms_per_step"] / 1000.0)) <= 1e-6 * d["value"]
    assert d["config"]["stored_logits_bytes"] > 0
