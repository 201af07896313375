"""The diagnostics next to the learner head, through the C ABI:

- rz_kl: the three KL estimators (k3 = D3), against the oracle on the same
  inputs, and bit for bit against rz_d3 and the learner step's kl output;
- rz_decompose: the log-ratio decomposition of log pi_new - log mu into the
  weight lag and the kernel mismatch, against the oracle, with the pages'
  claim checked token by token (mismatch exactly 0 when mu came from this
  library at the rollout's weights, in other batchings), and shown to detect
  a mismatch when mu came from a different computation.

Tolerances: the estimators are float64 reductions of the same float32
inputs as the oracle's, so they agree to ~1e-12 relative (k1 against the
scale of |delta|, since it cancels); lag is a difference of two
log-probabilities, each within 5e-4 of the oracle, so it is held to 1e-3."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16, f32, host, i32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rz():
    import invariant_logprob_is_amd as m
    m.lib()
    return m


def _check_kl(got, lp, mu):
    k1, k2, k3 = oracle.kl_estimators(lp.astype(np.float64), mu.astype(np.float64))
    scale = float(np.mean(np.abs(lp.astype(np.float64) - mu)))
    assert abs(got[0] - k1) <= 1e-12 * scale + 1e-300
    assert got[1] == pytest.approx(k2, rel=1e-12)
    assert got[2] == pytest.approx(k3, rel=1e-12)


@pytest.mark.parametrize("T", [1, 300, 16384, 16385, 100003])
def test_kl_matches_oracle_and_d3_bits(rz, gpu, T):
    say(f"kl T={T}")
    rng = np.random.default_rng(T)
    lp = (-rng.exponential(2.0, T)).astype(np.float32)
    mu = (lp + rng.normal(0, 0.05, T)).astype(np.float32)
    lpd, mud = f32(lp, gpu), f32(mu, gpu)
    got = host(rz.kl(lpd, mud))
    _check_kl(got, lp, mu)
    d3 = host(rz.d3(lpd, mud))
    assert d3[0] == got[2]                    # same kernels: the same float64 bits
    # on-policy: every estimator exactly 0
    z = host(rz.kl(lpd, lpd))
    assert np.all(z == 0.0)


def test_step_kl_output_is_rz_kl(rz, gpu):
    b = workloads.tiny()
    x, g, W, t = bf16(b.x, gpu), bf16(b.gamma, gpu), bf16(b.W, gpu), i32(b.target, gpu)
    olp, _ = oracle.logprob(b.x, b.gamma, b.eps, b.W, b.target)
    mu = f32((olp + b.lag_noise).astype(np.float32), gpu)
    out = rz.learner_step(x, g, W, t, mu, b.resp_offsets, b.group_offsets, b.reward, b.eps)
    kl = rz.kl(out["logprob"], mu)
    np.testing.assert_array_equal(host(out["kl"]).view(np.uint64), host(kl).view(np.uint64))
    assert host(out["kl"])[2] == host(out["d3"])[0]
    _check_kl(host(kl), host(out["logprob"]), host(mu))


def _version_pair(seed, T, H, V, w_sigma, x_sigma=0.0, g_sigma=0.0):
    rng = np.random.default_rng(seed)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    g = workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    W = workloads.f32_to_bf16_bits((0.05 * rng.standard_normal((V, H))).astype(np.float32))
    t = rng.integers(0, V, T).astype(np.int32)
    xo, go, Wo = workloads.older_version(seed, x, g, W, w_sigma, x_sigma, g_sigma)
    return (x, g, W), (xo, go, Wo), t


@pytest.mark.parametrize("T,H,V", [(300, 128, 1024), (513, 192, 2500)])
def test_decompose_zero_mismatch_when_mu_is_ours(rz, gpu, T, H, V):
    say(f"decompose T={T} H={H} V={V}")
    (x, g, W), (xo, go, Wo), t = _version_pair(T + V, T, H, V, 2e-3, 1e-2, 1e-3)
    dn = [bf16(a, gpu) for a in (x, g, W)]
    do = [bf16(a, gpu) for a in (xo, go, Wo)]
    td = i32(t, gpu)
    # mu as a rollout engine would record it: decode-style calls (one row at
    # a time for the first rows, then uneven prefill-like chunks), at the
    # rollout's weights
    mu = torch.empty(T, dtype=torch.float32, device=gpu)
    edges = list(range(0, 17)) + list(range(17, T, 97)) + [T]
    for a, c in zip(edges[:-1], edges[1:]):
        lp, _ = rz.logprob(do[0][a:c], do[1], do[2], td[a:c])
        mu[a:c] = lp
    out = rz.decompose(dn[0], dn[1], dn[2], do[0], do[1], do[2], td, mu)
    lag, mis, summ = host(out["lag"]), host(out["mismatch"]), host(out["summary"])
    assert np.all(mis == 0.0) and summ[2] == 0.0 and summ[3] == 0.0
    # lag against the oracle's two log-probabilities
    lp_new, _ = oracle.logprob(x, g, 1e-6, W, t)
    lp_old, _ = oracle.logprob(xo, go, 1e-6, Wo, t)
    olag, _ = oracle.decompose(lp_new, lp_old, host(mu))
    err = np.abs(lag - olag).max()
    say(f"  max|lag|={np.abs(olag).max():.3e} max|dlag|={err:.2e}")
    assert err <= 1e-3
    assert np.abs(olag).max() > 1e-2           # the versions really differ
    assert summ[0] == pytest.approx(np.abs(lag.astype(np.float64)).max(), rel=1e-6)
    assert summ[1] == pytest.approx(lag.astype(np.float64).mean(), rel=1e-5, abs=1e-9)


def test_decompose_same_version_has_zero_lag(rz, gpu):
    (x, g, W), _, t = _version_pair(7, 200, 128, 777, 0.0)
    d = [bf16(a, gpu) for a in (x, g, W)]
    td = i32(t, gpu)
    mu, _ = rz.logprob(d[0], d[1], d[2], td)
    out = rz.decompose(d[0], d[1], d[2], d[0], d[1], d[2], td, mu)
    assert np.all(host(out["lag"]) == 0.0) and np.all(host(out["mismatch"]) == 0.0)
    assert np.all(host(out["summary"]) == 0.0)


def test_decompose_detects_a_different_computation(rz, gpu):
    # mu from another implementation of the same math (the float64 oracle,
    # rounded to float32): a kernel mismatch the probe must see, bounded by
    # the parity tolerance
    (x, g, W), (xo, go, Wo), t = _version_pair(11, 300, 128, 1024, 2e-3)
    lp_old, _ = oracle.logprob(xo, go, 1e-6, Wo, t)
    mu = f32(lp_old.astype(np.float32), gpu)
    d = [bf16(a, gpu) for a in (x, g, W, xo, go, Wo)]
    out = rz.decompose(*d, i32(t, gpu), mu)
    mis, summ = host(out["mismatch"]), host(out["summary"])
    say(f"  tokens with mismatch: {int(summ[3])}/300, max {summ[2]:.2e}")
    assert summ[3] > 0 and summ[3] == np.count_nonzero(mis)
    assert 0 < summ[2] <= 5e-4
