"""rz_learner_step (the fused learner head) against the oracle, and against
the separate entry points it must agree with bit for bit (log-probabilities,
lse, coef, loss, D3)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16, bits32, f32, host, i32, rel_fro, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rz():
    import invariant_logprob_is_amd as m
    m.lib()
    return m


def _ragged(seed, T, n_groups, per_group):
    rng = np.random.default_rng(seed)
    R = n_groups * per_group
    cuts = np.sort(rng.choice(np.arange(1, T), R - 1, replace=False))
    ro = np.concatenate([[0], cuts, [T]]).astype(np.int64)
    go = np.arange(0, R + 1, per_group, dtype=np.int64)
    reward = (rng.random(R) < 0.5).astype(np.float32)
    return ro, go, reward


def test_tiny_step_matches_oracle(rz, gpu):
    b = workloads.tiny()
    olp, olse = oracle.logprob(b.x, b.gamma, b.eps, b.W, b.target)
    mu = (olp + b.lag_noise).astype(np.float32)
    ref = oracle.is_loss(olp, mu.astype(np.float64), b.resp_offsets, b.group_offsets, b.reward)
    ref_d3 = oracle.d3(olp, mu.astype(np.float64))
    ref_dh = oracle.backward(b.x, b.gamma, b.eps, b.W, b.target, olse, ref["coef"])
    out = rz.learner_step(bf16(b.x, gpu), bf16(b.gamma, gpu), bf16(b.W, gpu), i32(b.target, gpu),
                          f32(mu, gpu), b.resp_offsets, b.group_offsets, b.reward, b.eps)
    dlp = np.abs(host(out["logprob"]) - olp).max()
    rl = abs(host(out["loss"])[0] / ref["loss"] - 1)
    rd = abs(host(out["d3"])[0] / ref_d3 - 1)
    e = rel_fro(host(out["dhidden"]), ref_dh)
    say(f"  step tiny: dlogprob={dlp:.2e} loss rel={rl:.2e} d3 rel={rd:.2e} dhidden rel_fro={e:.2e}")
    assert dlp <= 5e-4 and rl <= 1e-3 and rd <= 1e-3 and e <= 1e-3
    np.testing.assert_allclose(host(out["coef"]), ref["coef"], rtol=1e-4)


@pytest.mark.parametrize("T,H,V", [(300, 128, 1000), (70001, 128, 1024), (40000, 192, 513)])
def test_step_agrees_with_separate_entry_points(rz, gpu, T, H, V):
    """Same bits as rz_logprob / rz_is_loss / rz_d3 / rz_backward (given the
    step's own lse and coef).  T > 32768 crosses chunk boundaries."""
    say(f"step vs separate T={T} H={H} V={V}")
    rng = np.random.default_rng(T + H)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    g = workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    W = workloads.f32_to_bf16_bits((0.05 * rng.standard_normal((V, H))).astype(np.float32))
    t = rng.integers(0, V, T).astype(np.int32)
    ro, go, reward = _ragged(T, T, 4, 4)
    mu = (-math.log(V) + rng.normal(0, 0.3, T)).astype(np.float32)
    xd, gd, Wd, td, mud = bf16(x, gpu), bf16(g, gpu), bf16(W, gpu), i32(t, gpu), f32(mu, gpu)
    out = rz.learner_step(xd, gd, Wd, td, mud, ro, go, reward)
    lp, lse = rz.logprob(xd, gd, Wd, td)
    loss, coef, _ = rz.is_loss(lp, mud, ro, go, reward)
    d3 = rz.d3(lp, mud)
    np.testing.assert_array_equal(bits32(out["logprob"]), bits32(lp))
    np.testing.assert_array_equal(bits32(out["lse"]), bits32(lse))
    np.testing.assert_array_equal(bits32(out["coef"]), bits32(coef))
    assert host(out["loss"])[0] == host(loss)[0]
    assert host(out["d3"])[0] == host(d3)[0]
    dh = rz.backward(xd, gd, Wd, td, lse, coef)
    np.testing.assert_array_equal(bits32(out["dhidden"]), bits32(dh))
    # sampled rows against the oracle
    rows = np.unique(np.concatenate([[0, T - 1, min(T - 1, 32767), min(T - 1, 32768)],
                                     rng.choice(T, 40, replace=False)]))
    olp, olse = oracle.logprob(x[rows], g, 1e-6, W, t[rows])
    assert np.abs(host(out["logprob"])[rows] - olp).max() <= 5e-4
    ocoef = oracle.is_coef_rows(olp, mu[rows].astype(np.float64), rows, ro, go, reward)
    odh = oracle.backward(x[rows], g, 1e-6, W, t[rows], olse, ocoef)
    e2 = rel_fro(host(out["dhidden"])[rows], odh)
    say(f"  dhidden vs oracle rows rel_fro={e2:.2e}")
    assert e2 <= 1e-3


def test_step_is_deterministic(rz, gpu):
    b = workloads.tiny()
    args = (bf16(b.x, gpu), bf16(b.gamma, gpu), bf16(b.W, gpu), i32(b.target, gpu),
            f32(b.lag_noise - 7.0, gpu), b.resp_offsets, b.group_offsets, b.reward)
    runs = []
    for _ in range(3):
        o = rz.learner_step(*args)
        runs.append([host(o[k]).tobytes() for k in ("logprob", "lse", "coef", "loss", "d3", "dhidden")])
    assert runs[0] == runs[1] == runs[2]
