"""Learner-head benchmark: one step = one rz_learner_step call (log-probs,
IS loss, D3, gradient to the hidden states) over one synthetic batch resident
in HBM.

    python bench.py [--steps K] [--warmup W] [--config qwen15b]

Prints ONE JSON line.  `value` is learner tokens per second on one GPU;
`roofline` covers the kernel with the largest share of the step, timed live
with HIP events that the library records on the stream each kernel is
launched on; `cpu_baseline` times the float64 oracle on a bounded sample of
the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [
    os.path.join(ROOT, "invariant_logprob_is_amd", "csrc", f)
    for f in ("rz_kernels.hip", "rz_gemm.h", "rz_gemm_tr.h", "rz_internal.h", "rz_util.h")
]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha() -> str:
    """Hash of the kernel sources' code: comments and blank lines are left
    out, so a documentation edit does not invalidate measured counters."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        lines = [ln.rstrip() for ln in src.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on different kernel sources."""
    p = os.path.join(PROFILES, f"traffic_{kernel}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_sha") != source_sha():
        return None
    return d.get("bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo (or the platform)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(b, n_tokens: int):
    """The oracle as it stands, on the first `n_tokens` rows of the batch
    (whole responses are not needed: rows are independent in the head), with
    the BLAS thread pools set to every core this process may run on."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        threadpool_info, limiter = None, None
    try:
        threads = cores
        if threadpool_info is not None:
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        n = min(n_tokens, b.T)
        rows = slice(0, n)
        mu_noise = b.lag_noise[rows].astype(np.float64)
        t0 = time.perf_counter()
        lp, lse = oracle.logprob(b.x[rows], b.gamma, b.eps, b.W, b.target[rows])
        mu = lp + mu_noise
        ro = np.array([0, n], np.int64)
        go = np.array([0, 1], np.int64)
        L = oracle.is_loss(lp, mu, ro, go, b.reward[:1])
        oracle.d3(lp, mu)
        oracle.backward(b.x[rows], b.gamma, b.eps, b.W, b.target[rows], lse, L["coef"])
        dt = time.perf_counter() - t0
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "affinity_cores": cores,
            "sample": f"first {n} rows of the workload: RMSNorm, LM head, log-softmax, IS loss, "
                      f"D3 and backward to the hidden states in float64 numpy ({dt:.1f} s)"}


def side_kernel_bytes(name: str, T: int, H: int, V: int, launches: int):
    """Algorithmic HBM bytes per step of the head's memory- or latency-bound
    kernels (what each must read and write at least once), or None for a
    kernel not listed.  n_vt = ceil(V / 256) vocabulary tiles."""
    n_vt = -(-V // 256)
    per = {
        # x read, hhat written (bf16)
        "k_rmsnorm_fwd": 4 * H * T,
        # x read, dhidden read and written in place (fp32)
        "k_rmsnorm_bwd": 10 * H * T,
        # per token: the n_vt tile partials (M, S) and z_target, mu and the
        # float64 token scale read; logprob, lse, coef, the row factor and
        # the n_vt shifts written
        "k_lse_combine": (12 * n_vt + 32) * T,
        # W read, W^T written (bf16)
        "k_transpose_w": 4 * V * H,
        # the float64 token scale written
        "k_token_scale": 8 * T,
        # logprob and mu read, per launch (the loss; D3 and the KL estimators)
        "k_is_loss": 8 * T,
        "k_kl": 8 * T * max(launches, 1),
    }
    return per.get(name)


CALIBRATION_BYTES = 1 << 28   # plain device-to-device copy run once per benchmark
NOMINAL_SCLK_MHZ = 2400.0     # the shader clock the published MFMA peak assumes


class SclkSampler:
    """Reads the GPU's current shader clock (the starred line of the amdgpu
    driver's pp_dpm_sclk in sysfs), and its board power where the driver's
    hwmon files give it, every 50 ms on a side thread while the timed steps
    run.  Reports nothing when the clock file is absent, or when there is
    more than one GPU and the one in use cannot be told apart."""

    def __init__(self, interval_s: float = 0.05):
        import glob
        import threading
        files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = files[0] if len(files) == 1 else None
        self.power_path = self.cap_w = None
        if self.path:
            hw = os.path.join(os.path.dirname(self.path), "hwmon", "hwmon*")
            for name in ("power1_average", "power1_input"):
                cand = sorted(glob.glob(os.path.join(hw, name)))
                if cand:
                    self.power_path = cand[0]
                    break
            cap = sorted(glob.glob(os.path.join(hw, "power1_cap")))
            if cap:
                self.cap_w = self._read_w(cap[0])
        self.interval = interval_s
        self.samples = []
        self.power = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read_w(path):
        """A hwmon power file (microwatts) in watts, or None."""
        try:
            with open(path) as f:
                return float(f.read().strip()) / 1e6
        except (OSError, ValueError):
            return None

    def _read(self):
        import re
        try:
            with open(self.path) as f:
                for line in f:
                    m = re.search(r"(\d+)\s*Mhz\s*\*", line, re.I)
                    if m:
                        return float(m.group(1))
        except OSError:
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            if self.power_path:
                w = self._read_w(self.power_path)
                if w is not None:
                    self.power.append(w)
            self._stop.wait(self.interval)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        v = np.asarray(self.samples)
        out = {"mean_mhz": float(v.mean()), "min_mhz": float(v.min()), "max_mhz": float(v.max()),
               "samples": int(v.size), "source": self.path}
        if self.power:
            w = np.asarray(self.power)
            out["board_power"] = {"mean_w": float(w.mean()), "max_w": float(w.max()),
                                  "cap_w": self.cap_w, "samples": int(w.size),
                                  "source": self.power_path}
        return out


def summarize_counters(fetch_csv: str, write_csv: str, dram_csv: str = None):
    """Per-launch memory traffic of the head's kernels from rocprofv3 counter
    collection (FETCH_SIZE and WRITE_SIZE are in KiB per dispatch), scaled by
    what the same counters read for the calibration copy of known size.
    With dram_csv, a third pass of TCC_EA0_RDREQ_DRAM_sum and
    TCC_EA0_WRREQ_DRAM_sum (the L2's read and write requests to local memory,
    counted in requests) is turned into bytes with the same copy's
    requests per byte."""
    import csv
    import collections

    def per_kernel(path, counter, unit=1024.0):
        acc = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("rz::", "").strip()
            acc[(name, r["Dispatch_Id"])].append(float(r["Counter_Value"]))
        out = collections.defaultdict(list)
        for (name, _), v in acc.items():
            out[name].append(sum(v) * unit)
        return out

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy = "__amd_rocclr_copyBuffer"
    cf = max(fetch.get(copy, [0.0])) / CALIBRATION_BYTES
    cw = max(write.get(copy, [0.0])) / CALIBRATION_BYTES
    dram = None
    if dram_csv:
        drd = per_kernel(dram_csv, "TCC_EA0_RDREQ_DRAM_sum", 1.0)
        dwr = per_kernel(dram_csv, "TCC_EA0_WRREQ_DRAM_sum", 1.0)
        dram = (drd, dwr, max(drd.get(copy, [0.0])) / CALIBRATION_BYTES,
                max(dwr.get(copy, [0.0])) / CALIBRATION_BYTES)
    os.makedirs(PROFILES, exist_ok=True)
    sha = source_sha()
    # the learner step launches the storing forward variant (persistent, or
    # one workgroup per tile); k_dw (--grads) is the row scaling plus the
    # token contraction, one of each per chunk
    fwd = "k_lmhead_fwd_p<true>" if "k_lmhead_fwd_p<true>" in fetch else "k_lmhead_fwd<true>"
    for k, disps in (("k_lmhead_fwd", (fwd,)), ("k_dhidden", ("k_dhidden",)),
                     ("k_dw", ("k_scale_rows_t", "k_dw_tr"))):
        if any(d not in fetch or d not in write for d in disps):
            continue
        disp = disps[-1]
        f = sum(float(np.mean(fetch[d])) for d in disps) / (cf or 1.0)
        w = sum(float(np.mean(write[d])) for d in disps) / (cw or 1.0)
        d = {"kernel": k, "source_sha": sha, "bytes_per_launch": f + w,
             "fetch_bytes_per_launch": f, "write_bytes_per_launch": w,
             "launches": len(fetch[disp]), "calibration": {
                 "copy_bytes": CALIBRATION_BYTES, "fetch_factor": cf, "write_factor": cw},
             "source": "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of bench.py, KiB per dispatch, "
                       "divided by the factor the same counter reads for a copy of copy_bytes"}
        if dram is not None and all(x in dram[0] and x in dram[1] for x in disps):
            drd, dwr, crd, cwr = dram
            d["dram_read_bytes_per_launch"] = sum(float(np.mean(drd[x])) for x in disps) / (crd or 1.0)
            d["dram_write_bytes_per_launch"] = sum(float(np.mean(dwr[x])) for x in disps) / (cwr or 1.0)
            d["calibration"]["dram_read_requests_per_byte"] = crd
            d["calibration"]["dram_write_requests_per_byte"] = cwr
            d["dram_source"] = ("rocprofv3 --pmc TCC_EA0_RDREQ_DRAM_sum TCC_EA0_WRREQ_DRAM_sum: the L2's "
                                "requests to local memory (the MALL serves some of them; no counter "
                                "on this part separates MALL hits from HBM), divided by the requests "
                                "per byte of the same copy")
        with open(os.path.join(PROFILES, f"traffic_{k}.json"), "w") as fh:
            json.dump(d, fh, indent=1)
        print(f"{k}: {f / 1e9:.3f} GB fetched + {w / 1e9:.3f} GB written per launch "
              f"(factors {cf:.3f}, {cw:.3f})"
              + (f"; local-memory requests {d['dram_read_bytes_per_launch'] / 1e9:.3f} GB read, "
                 f"{d['dram_write_bytes_per_launch'] / 1e9:.3f} GB written"
                 if "dram_read_bytes_per_launch" in d else ""))


def probe(args, b, rz, x, g, W, tgt, lp, ws, stream):
    """The decomposition probe on the same workload: the rollout's weights are
    an older version of the head (every gamma and W element moved by
    N(0, 1e-3)), mu is recorded at those weights in another batching
    (8191-row calls), and rz_decompose splits log pi - log mu per token.
    Then the KL estimators are tracked over 16 synthetic updates."""
    import torch
    import workloads
    from invariant_logprob_is_amd.tracking import UpdateTracker

    dev = x.device
    _, g_old, W_old = workloads.older_version(1, b.x[:1], b.gamma, b.W, 1e-3, 0.0, 1e-3)
    go = torch.from_numpy(g_old.view(np.int16)).view(torch.bfloat16).to(dev)
    Wo = torch.from_numpy(np.ascontiguousarray(W_old).view(np.int16)).view(torch.bfloat16).to(dev)
    T, H, V = b.T, b.H, b.V
    mu = torch.empty(T, dtype=torch.float32, device=dev)
    for a in range(0, T, 8191):
        c = min(T, a + 8191)
        mu[a:c] = rz.logprob(x[a:c], go, Wo, tgt[a:c], b.eps, workspace=ws)[0]
    torch.cuda.synchronize()

    def call():
        return rz.decompose(x, g, W, x, go, Wo, tgt, mu, b.eps, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    rz.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prof = rz.profile_read()
    rz.profile_enable(False)
    ms = 1000.0 * wall / args.steps
    summ = out["summary"].cpu().numpy()
    log(f"probe {ms:.2f} ms/call; max|lag|={summ[0]:.3e} mean lag={summ[1]:.3e} "
        f"max|mismatch|={summ[2]:.3e} tokens with mismatch={int(summ[3])}")
    for k, (tot, n) in sorted(prof.items(), key=lambda kv: -kv[1][0]):
        log(f"  {k:16s} {tot / args.steps:9.3f} ms/call  {n // args.steps:4d} launches/call")
    tot, n = prof["k_lmhead_fwd"]
    achieved = 2 * 2.0 * T * H * V * args.steps / (tot / 1000.0)

    # KL tracking over synthetic updates: mu_u = logprob + sigma_u * (a seeded
    # permutation of the workload's N(0, 1) lag noise), sigma_u ~ lognormal
    # around 0.05, one update with a tenfold spike
    rng = np.random.default_rng(20260)
    base = b.lag_noise / np.float32(b.lag_noise.std())
    sig = 0.05 * np.exp(rng.normal(0, 0.2, 16))
    sig[11] *= 10.0
    tr = UpdateTracker()
    for u in range(16):
        noise = torch.from_numpy((base[rng.permutation(T)] * np.float32(sig[u])).astype(np.float32))
        tr.add(rz.kl(lp, (lp + noise.to(dev)).contiguous(), workspace=ws))
    track = tr.summary()
    log(f"kl tracking over 16 updates: D3 median {track['k3']['median']:.3e}, "
        f"peak/median {track['k3']['peak_over_median']:.2f}")
    print(json.dumps({
        "metric": "decomposition probe tokens/sec (two forward passes + per-token lag/mismatch split), 1 GPU",
        "value": T / (ms / 1000.0), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{b.name}: T={T} tokens, H={H}, V={V}; rollout weights moved by N(0, 1e-3)",
                   "T": T, "H": H, "V": V},
        "summary": {"max_abs_lag": float(summ[0]), "mean_lag": float(summ[1]),
                    "max_abs_mismatch": float(summ[2]), "tokens_with_mismatch": int(summ[3])},
        "kl_tracking": track,
        "roofline": {"kernel": "k_lmhead_fwd", "bound": "mfma", "achieved": achieved / 1e12,
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_FLOPS, "traffic": None},
    }), flush=True)


def executed_flops(T: int, H: int, V: int, grads: bool) -> float:
    """MFMA flops the step's kernels execute, from their tile grids: the
    stored e replaces a second forward, so the only work beyond the
    algorithmic count is the padding of the edge tiles (256-row tiles of
    tokens per 32768-token chunk, of V and of H; V padded to 64 along K)."""
    def up(a, b):
        return -(-a // b) * b
    chunks = [min(32768, T - c) for c in range(0, T, 32768)]
    Vt, Ht, Vk = up(V, 256), up(H, 256), up(V, 64)
    f = 0.0
    for tc in chunks:
        tp = up(tc, 256)
        f += 2.0 * Vt * tp * H          # forward: vocab x token tiles, K = H
        f += 2.0 * tp * Ht * Vk         # hidden-state contraction, K = V padded to 64
        if grads:
            f += 2.0 * Vt * Ht * tp     # dW: vocab x hidden tiles, K = tokens
    return f


def shards(args, b, rz, x, g, W, tgt, lp, lse, ws):
    """The log-probabilities of the workload through `args.shards` equal
    shares of the vocabulary splits (rz_logprob_shard on each share's rows of
    W, one share after another on this GPU) and the merge (rz_logprob_merge).
    Each share's time is what one device of a vocabulary-parallel head would
    spend on it; the merged bits are checked against rz_logprob's."""
    import torch

    dev = x.device
    T, H, V = b.T, b.H, b.V
    d = args.shards
    k = rz.VOCAB_SPLITS // d
    plan = [(r * k, (r + 1) * k) for r in range(d)]
    rows = [(rz.vocab_split_begin(V, s0), rz.vocab_split_begin(V, s1)) for s0, s1 in plan]
    parts = torch.empty((rz.VOCAB_SPLITS, T, 3), dtype=torch.float64, device=dev)
    mlp = torch.empty(T, dtype=torch.float32, device=dev)
    mlse = torch.empty(T, dtype=torch.float32, device=dev)

    def call(ev=None):
        for r, ((s0, s1), (a, c)) in enumerate(zip(plan, rows)):
            if ev:
                ev[r][0].record()
            rz.logprob_shard(x, g, W[a:c], tgt, V, s0, s1, b.eps, workspace=ws,
                             out=parts[s0:s1])
            if ev:
                ev[r][1].record()
        if ev:
            ev[d][0].record()
        rz.logprob_merge(parts, tgt, V, out=mlp, lse_out=mlse)
        if ev:
            ev[d][1].record()

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    same = bool(torch.equal(mlp.view(torch.int32), lp.view(torch.int32)) and
                torch.equal(mlse.view(torch.int32), lse.view(torch.int32)))
    per = np.zeros(d + 1)
    rz.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(d + 1)]
        call(ev)
        torch.cuda.synchronize()
        per += [a.elapsed_time(c) for a, c in ev]
    wall = time.perf_counter() - t0
    prof = rz.profile_read()
    rz.profile_enable(False)
    per /= args.steps
    ms = 1000.0 * wall / args.steps
    log(f"{d} shares: {ms:.2f} ms per pass; shares {np.round(per[:d], 2).tolist()} ms, "
        f"merge {per[d]:.3f} ms; bits equal to rz_logprob: {same}")
    if not same:
        raise SystemExit("sharded logprob differs from rz_logprob")
    tot, n = prof["k_lmhead_fwd"]
    achieved = 2.0 * T * H * V * args.steps / (tot / 1000.0)
    print(json.dumps({
        "metric": "vocab-split logprob tokens/sec (all shares in turn + merge), 1 GPU",
        "value": T / (ms / 1000.0), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{b.name}: T={T} tokens, H={H}, V={V}; vocabulary in {d} shares "
                               f"of {k} splits", "T": T, "H": H, "V": V, "shares": d},
        "share_ms": per[:d].tolist(), "merge_ms": float(per[d]), "bits_equal_rz_logprob": same,
        "roofline": {"kernel": "k_lmhead_fwd", "bound": "mfma", "achieved": achieved / 1e12,
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_FLOPS, "traffic": None},
    }), flush=True)


def decode(args, b, rz, x, g, W, tgt, lp_full, ws):
    """rz_logprob on small batches, the decode-style call: the first T rows
    of the workload for T = 1 .. 2048, each call timed with HIP events on the
    launch stream (median over the calls).  Every size runs the same 256 x
    256 tiles as the learner step -- the price of batch invariance at small
    T -- so the bits of each row must equal the full batch's; below 256 rows
    a call costs about the same whatever T."""
    import torch

    dev = x.device
    H, V = b.H, b.V
    reps = max(args.steps, 20)
    per = {}
    for T in (n for n in (1, 8, 64, 128, 256, 2048) if n <= b.T):
        lp = torch.empty(T, dtype=torch.float32, device=dev)
        lse = torch.empty(T, dtype=torch.float32, device=dev)
        xs, ts = x[:T], tgt[:T]
        for _ in range(args.warmup + 1):
            rz.logprob(xs, g, W, ts, b.eps, workspace=ws, out=lp, lse_out=lse)
        torch.cuda.synchronize()
        same = bool(torch.equal(lp.view(torch.int32), lp_full[:T].view(torch.int32)))
        if not same:
            raise SystemExit(f"decode-style call at T={T} differs from the full batch")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, c in ev:
            a.record()
            rz.logprob(xs, g, W, ts, b.eps, workspace=ws, out=lp, lse_out=lse)
            c.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(c) for a, c in ev])) * 1000.0
        w_gbps = 2.0 * V * H / (us * 1e-6) / 1e9
        per[str(T)] = {"us_per_call": us, "tokens_per_s": T / (us * 1e-6),
                       "w_read_GBps": w_gbps, "bits_equal_full_batch": same}
        log(f"decode T={T}: {us:.1f} us per call, {T / (us * 1e-6):.0f} tokens/s, "
            f"W read at {w_gbps:.0f} GB/s; bits equal the full batch's: {same}")
    t1 = per["1"]
    print(json.dumps({
        "metric": "decode-style rz_logprob latency (one row), 1 GPU",
        "value": t1["us_per_call"], "unit": "us", "n_gpus": 1, "steps": reps,
        "warmup": args.warmup, "ms_per_step": t1["us_per_call"] / 1000.0,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{b.name}: the first T rows, H={H}, V={V}", "H": H, "V": V},
        "per_T": per,
        "roofline": {"kernel": "rz_logprob call", "bound": "hbm",
                     "achieved": t1["w_read_GBps"], "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                     "frac": t1["w_read_GBps"] * 1e9 / PEAK_HBM_BYTES, "traffic": None},
    }), flush=True)


def stored(args, b, rz, x, g, W, tgt, mu, ro, go, reward, ws, outs):
    """The learner head through the separate entry points with stored logits:
    rz_logprob_store, rz_is_loss, rz_backward_stored.  The whole batch's
    logits stay in HBM between the forward and the backward (about 2 bytes
    per logit); the bits are checked against rz_learner_step's."""
    import torch

    dev = x.device
    T, H, V = b.T, b.H, b.V
    need = rz.logits_bytes(T, H, V)
    free, _ = torch.cuda.mem_get_info(dev)
    if need + (1 << 30) > free:
        raise SystemExit(f"stored logits need {need / 2**30:.1f} GiB, {free / 2**30:.1f} GiB free")
    buf = torch.empty(need, dtype=torch.uint8, device=dev)
    lp = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    dh = torch.empty(T, H, dtype=torch.float32, device=dev)
    log(f"stored logits {need / 2**30:.1f} GiB")
    res = {}

    def call():
        rz.logprob_store(x, g, W, tgt, b.eps, logits=buf, workspace=ws, out=lp, lse_out=lse)
        res["loss"], res["coef"], _ = rz.is_loss(lp, mu, ro, go, reward, workspace=ws,
                                                 want_advantage=False)
        rz.backward_stored(x, g, W, tgt, lse, res["coef"], buf, b.eps, workspace=ws, out=dh)

    rz.learner_step(x, g, W, tgt, mu, ro, go, reward, b.eps, workspace=ws, out=outs)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    same = all(torch.equal(a.view(torch.int32), c.view(torch.int32))
               for a, c in ((lp, outs["logprob"]), (res["coef"], outs["coef"]),
                            (dh, outs["dhidden"])))
    same = same and bool(torch.equal(res["loss"], outs["loss"]))
    rz.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prof = rz.profile_read()
    rz.profile_enable(False)
    ms = 1000.0 * wall / args.steps
    log(f"stored-logits pass {ms:.2f} ms; bits equal to rz_learner_step: {same}")
    for k, (tot, n) in sorted(prof.items(), key=lambda kv: -kv[1][0]):
        log(f"  {k:16s} {tot / args.steps:9.3f} ms/pass  {n // args.steps:4d} launches/pass")
    if not same:
        raise SystemExit("stored-logits pass differs from rz_learner_step")
    kernels = {}
    for k in ("k_lmhead_fwd", "k_dhidden"):
        tot, n = prof[k]
        achieved = 2.0 * T * H * V * args.steps / (tot / 1000.0)
        kernels[k] = {"ms_per_step": tot / args.steps, "achieved_tflops": achieved / 1e12,
                      "frac": achieved / PEAK_BF16_FLOPS}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    tps = T / (ms / 1000.0)
    print(json.dumps({
        "metric": "stored-logits learner tokens/sec (rz_logprob_store + rz_is_loss + "
                  "rz_backward_stored) and % bf16 MFMA peak, 1 GPU",
        "value": tps, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{b.name}: T={T} tokens, H={H}, V={V}, {b.R} responses in "
                               f"{b.G} groups; logits stored between the calls",
                   "T": T, "H": H, "V": V, "R": b.R, "G": b.G, "stored_logits_bytes": need},
        "mfma_frac_algorithmic": tps * 4.0 * H * V / PEAK_BF16_FLOPS,
        "bits_equal_rz_learner_step": same, "kernels": kernels,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": kernels[dom]["achieved_tflops"],
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": kernels[dom]["frac"], "traffic": None},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="qwen15b",
                    choices=["qwen15b", "qwen4b_lag64", "a3b30_head", "tiny"])
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--grads", action="store_true",
                    help="also compute the weight gradients dW, dgamma in the timed step "
                         "(6*H*V algorithmic flops per token instead of 4*H*V)")
    ap.add_argument("--probe", action="store_true",
                    help="time the log-ratio decomposition probe (rz_decompose) and track the KL "
                         "estimators over synthetic updates instead of the learner step")
    ap.add_argument("--shards", type=int, choices=[1, 2, 4, 8],
                    help="time the log-probabilities through this many equal shares of the "
                         "vocabulary splits and their merge instead of the learner step")
    ap.add_argument("--decode", action="store_true",
                    help="time the decode-style rz_logprob call on the first 1 .. 2048 rows "
                         "instead of the learner step")
    ap.add_argument("--stored", action="store_true",
                    help="time the separate entry points with the whole batch's logits stored "
                         "between forward and backward (rz_logprob_store, rz_is_loss, "
                         "rz_backward_stored) instead of the learner step")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="turn rocprofv3 --pmc runs of this script (FETCH_SIZE, WRITE_SIZE and "
                         "optionally TCC_EA0_RDREQ_DRAM_sum + TCC_EA0_WRREQ_DRAM_sum) into "
                         "profiles/traffic_<kernel>.json and exit")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.cpu_tokens < 1:
        ap.error("--steps and --cpu-tokens must be at least 1, --warmup at least 0")
    modes = (args.probe, args.shards, args.stored, args.decode)
    if sum(map(bool, modes)) > 1 or (args.grads and any(modes)):
        ap.error("--probe, --shards, --stored and --decode each time their own pass, "
                 "without --grads")
    if args.summarize_counters:
        if len(args.summarize_counters) not in (2, 3):
            ap.error("--summarize-counters takes FETCH_CSV WRITE_CSV [DRAM_CSV]")
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the learner head is measured on one GPU; --gpus above 1 is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import invariant_logprob_is_amd as rz
    import workloads

    rz.lib()
    dev = torch.device("cuda", 0)
    t_gen = time.perf_counter()
    b = workloads.CONFIGS[args.config]()
    log(f"generated {args.config}: T={b.T} H={b.H} V={b.V} R={b.R} G={b.G} "
        f"in {time.perf_counter() - t_gen:.1f}s")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x, g, W = bf16(b.x), bf16(b.gamma), bf16(b.W)
    tgt = torch.from_numpy(b.target).to(dev)
    ro = torch.from_numpy(b.resp_offsets).to(dev)
    go = torch.from_numpy(b.group_offsets).to(dev)
    reward = torch.from_numpy(b.reward).to(dev)
    rz.validate_offsets(b.resp_offsets, b.group_offsets, b.T)
    ws_need = (rz.workspace_bytes_grads if args.grads else rz.workspace_bytes)(b.T, b.H, b.V)
    ws = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    lp = torch.empty(b.T, dtype=torch.float32, device=dev)
    lse = torch.empty(b.T, dtype=torch.float32, device=dev)
    dh = torch.empty(b.T, b.H, dtype=torch.float32, device=dev)
    log(f"workspace {ws.numel() / 2**30:.2f} GiB")

    # Rollout log-probabilities: the learner log-probability plus lag noise
    # (a setup step, outside the timed region).
    rz.logprob(x, g, W, tgt, b.eps, workspace=ws, out=lp, lse_out=lse)
    mu = (lp + torch.from_numpy(b.lag_noise).to(dev)).contiguous()
    outs = {"logprob": lp, "lse": lse, "dhidden": dh,
            "coef": torch.empty(b.T, dtype=torch.float32, device=dev),
            "loss": torch.empty(1, dtype=torch.float64, device=dev),
            "d3": torch.empty(1, dtype=torch.float64, device=dev)}
    if args.grads:
        outs["dW"] = torch.empty(b.V, b.H, dtype=torch.float32, device=dev)
        outs["dgamma"] = torch.empty(b.H, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    # a plain copy of known size: the reference for the HBM byte counters
    cal = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
    torch.empty_like(cal).copy_(cal)
    del cal
    torch.cuda.synchronize()
    if args.probe:
        probe(args, b, rz, x, g, W, tgt, lp, ws, stream)
        return
    if args.shards:
        shards(args, b, rz, x, g, W, tgt, lp, lse, ws)
        return
    if args.stored:
        stored(args, b, rz, x, g, W, tgt, mu, ro, go, reward, ws, outs)
        return
    if args.decode:
        decode(args, b, rz, x, g, W, tgt, lp, ws)
        return

    def step():
        rz.learner_step(x, g, W, tgt, mu, ro, go, reward, b.eps, workspace=ws, out=outs,
                        weight_grads=args.grads)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup}")

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    rz.profile_enable(True)
    torch.cuda.synchronize()
    with SclkSampler() as sclk:
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(args.steps):
            step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    prof = rz.profile_read()
    rz.profile_enable(False)
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms_step = 1000.0 * wall / args.steps
    log(f"step {ms_step:.2f} ms wall, events median {float(np.median(step_ms)):.2f} ms; "
        f"loss={outs['loss'].item():.6e} d3={outs['d3'].item():.6e}")
    for k, (tot, n) in sorted(prof.items(), key=lambda kv: -kv[1][0]):
        log(f"  {k:16s} {tot / args.steps:9.3f} ms/step  {n // args.steps:4d} launches/step")

    T, H, V = b.T, b.H, b.V
    tokens_per_s = T / (ms_step / 1000.0)
    alg_flops_token = (6.0 if args.grads else 4.0) * H * V
    exec_flops_token = executed_flops(T, H, V, args.grads) / T
    gemm_flops_step = 2.0 * T * H * V      # algorithmic flops of each GEMM kernel per step
    kernels = {}
    for k in ("k_lmhead_fwd", "k_dhidden") + (("k_dw",) if args.grads else ()):
        tot, n = prof.get(k, (float("nan"), 0))
        achieved = gemm_flops_step * args.steps / (tot / 1000.0)
        kernels[k] = {"ms_per_step": tot / args.steps, "launches_per_step": n // args.steps,
                      "achieved_tflops": achieved / 1e12, "frac": achieved / PEAK_BF16_FLOPS}
    side = {}
    for k, (tot, n) in prof.items():
        nb = side_kernel_bytes(k, T, H, V, n // args.steps)
        if nb is None or tot <= 0:
            continue
        gbs = nb * args.steps / (tot / 1000.0) / 1e9
        side[k] = {"ms_per_step": tot / args.steps, "launches_per_step": n // args.steps,
                   "algorithmic_bytes_per_step": nb, "achieved_GBps": gbs,
                   "frac_of_hbm_peak": gbs * 1e9 / PEAK_HBM_BYTES}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    roofline = {
        "kernel": dom, "bound": "mfma", "achieved": kernels[dom]["achieved_tflops"],
        "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s", "frac": kernels[dom]["frac"],
        "traffic": measured_traffic(dom),
    }
    metric = "learner tokens/sec (fwd+bwd logprob+IS loss) and % bf16 MFMA peak, 1 GPU"
    if args.grads:
        metric = ("learner tokens/sec (fwd+bwd logprob+IS loss, with LM-head dW and RMSNorm "
                  "dgamma) and % bf16 MFMA peak, 1 GPU")
    out = {
        "metric": metric,
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{b.name}: T={T} tokens, H={H}, V={V}, {b.R} responses in {b.G} groups",
                   "T": T, "H": H, "V": V, "R": b.R, "G": b.G},
        "mfma_frac_algorithmic": tokens_per_s * alg_flops_token / PEAK_BF16_FLOPS,
        "executed_flops_per_token": exec_flops_token,
        "mfma_frac_executed": tokens_per_s * exec_flops_token / PEAK_BF16_FLOPS,
        "kernels": kernels,
        "side_kernels": side,
        "roofline": roofline,
    }
    clock = sclk.summary()
    if clock is not None:
        # the same algorithmic rate against the peak at the clock the chip held
        clock["mfma_frac_algorithmic_at_this_clock"] = (
            out["mfma_frac_algorithmic"] * NOMINAL_SCLK_MHZ / clock["mean_mhz"])
        bp = clock.get("board_power")
        if bp:
            # the board's energy per step at its mean power, and tokens per joule
            bp["joules_per_step"] = bp["mean_w"] * ms_step / 1000.0
            bp["tokens_per_joule"] = T / bp["joules_per_step"]
        out["sclk_during_timed_steps"] = clock
    if not args.no_cpu_baseline:
        log(f"cpu baseline on {args.cpu_tokens} tokens ...")
        cb = cpu_baseline(b, args.cpu_tokens)
        # the oracle's rate applied to the whole batch, and the GPU's rate over it
        cb["full_batch_s_extrapolated"] = T / cb["value"]
        cb["gpu_over_cpu"] = tokens_per_s / cb["value"]
        out["cpu_baseline"] = cb
        log(f"cpu baseline {cb['value']:.1f} tokens/s; full batch ~{cb['full_batch_s_extrapolated']:.0f} s; "
            f"GPU/CPU {cb['gpu_over_cpu']:.0f}x")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
