"""Pins of the float64 oracle against things other than itself: closed forms,
hand-derived golden cases, library routines (torch / scipy), brute force and
finite differences.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log, "exp": math.exp, "expm1": math.expm1}))


def _rand_bits(rng, shape, std=1.0, mean=0.0):
    return workloads.f32_to_bf16_bits((rng.standard_normal(shape) * std + mean).astype(np.float32))


# ---------------------------------------------------------------- bf16_round

def test_bf16_round_ties_to_even_and_single_rounding():
    # bf16 spacing at 1 is 2**-7.
    cases = {
        1.0 + 2.0 ** -8: 1.0,                      # tie -> even (mantissa 0)
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,      # tie -> even (mantissa 2)
        1.0 + 2.0 ** -8 + 2.0 ** -30: 1.0 + 2.0 ** -7,  # just above the tie: a float32
                                                   # intermediate would round to the tie first
        -(1.0 + 2.0 ** -8 + 2.0 ** -30): -(1.0 + 2.0 ** -7),
        1.0 + 2.0 ** -8 - 2.0 ** -40: 1.0,
        3.0: 3.0, -0.0: 0.0, 0.0: 0.0,
    }
    for y, want in cases.items():
        assert oracle.bf16_round(np.array([y]))[0] == want, y


def test_bf16_round_matches_bit_rounding_of_float32():
    # For float32-representable inputs a single rounding from float64 equals
    # the integer bit trick on float32 storage (an independent implementation).
    rng = np.random.default_rng(11)
    a = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    want = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(a)).astype(np.float64)
    got = oracle.bf16_round(a.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_round_brackets_and_is_nearest():
    rng = np.random.default_rng(12)
    y = rng.standard_normal(100000) * 10.0
    r = oracle.bf16_round(y)
    # r is a bf16 value: it survives a float32 round trip with zero low bits
    bits = r.astype(np.float32).view(np.uint32)
    assert np.all(bits & np.uint32(0xFFFF) == 0)
    # nearest: |y - r| <= half the spacing at |r|
    _, e = np.frexp(r)
    half = np.ldexp(1.0, e - 9)
    assert np.all(np.abs(y - r) <= half * (1 + 1e-12))


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(1)
    x = _rand_bits(rng, (37, 96))
    g = _rand_bits(rng, (96,), 0.1, 1.0)
    eps = 1e-6
    y, r = oracle.rmsnorm(x, g, eps, round_output=False)
    xt = torch.from_numpy(oracle.bf16_decode(x))
    gt = torch.from_numpy(oracle.bf16_decode(g))
    want = torch.nn.functional.rms_norm(xt, (96,), weight=gt, eps=float(np.float32(eps))).numpy()
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-15)
    hh, _ = oracle.rmsnorm(x, g, eps)
    np.testing.assert_array_equal(hh, oracle.bf16_round(want))


def test_rmsnorm_constant_row_closed_form_and_scale():
    H = 64
    c = 0.75
    x = workloads.f32_to_bf16_bits(np.full((1, H), c, np.float32))
    g = workloads.f32_to_bf16_bits(np.linspace(0.5, 1.5, H).astype(np.float32))
    eps = 1e-6
    y, r = oracle.rmsnorm(x, g, eps, round_output=False)
    e = float(np.float32(eps))
    assert r[0] == pytest.approx(1.0 / math.sqrt(c * c + e), rel=1e-15)
    np.testing.assert_allclose(y[0], oracle.bf16_decode(g) * c / math.sqrt(c * c + e), rtol=1e-15)
    # scale invariance up to eps (outlier rows): x16 is exact in bf16
    rng = np.random.default_rng(3)
    xr = rng.standard_normal((4, H)).astype(np.float32)
    x1 = workloads.f32_to_bf16_bits(xr)
    x16 = workloads.f32_to_bf16_bits(oracle.bf16_decode(x1).astype(np.float32) * 16)
    y1, _ = oracle.rmsnorm(x1, g, eps, round_output=False)
    y16, _ = oracle.rmsnorm(x16, g, eps, round_output=False)
    np.testing.assert_allclose(y16, y1, rtol=2e-6)


def test_rmsnorm_h1_is_sign():
    x = workloads.f32_to_bf16_bits(np.array([[3.0], [-2.0]], np.float32))
    g = workloads.f32_to_bf16_bits(np.array([1.0], np.float32))
    y, _ = oracle.rmsnorm(x, g, 0.0, round_output=False)
    np.testing.assert_allclose(y[:, 0], [1.0, -1.0], rtol=1e-15)


# ---------------------------------------------------------------- logprob

def _small_case(seed, T=23, H=64, V=97):
    rng = np.random.default_rng(seed)
    x = _rand_bits(rng, (T, H))
    g = _rand_bits(rng, (H,), 0.1, 1.0)
    W = _rand_bits(rng, (V, H), 0.3)
    tgt = rng.integers(0, V, T).astype(np.int32)
    return x, g, W, tgt


def test_logprob_matches_torch_log_softmax_brute_force():
    x, g, W, tgt = _small_case(5)
    lp, lse = oracle.logprob(x, g, 1e-6, W, tgt, row_chunk=7)
    hh, _ = oracle.rmsnorm(x, g, 1e-6)
    z = torch.from_numpy(hh) @ torch.from_numpy(oracle.bf16_decode(W)).T
    want = torch.log_softmax(z, dim=1)[torch.arange(len(tgt)), torch.from_numpy(tgt.astype(np.int64))]
    np.testing.assert_allclose(lp, want.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=1).numpy(), rtol=0, atol=1e-12)
    assert np.all(lp <= 0)


def test_logprob_w_zero_is_uniform_and_v1_is_zero():
    x, g, W, tgt = _small_case(6, V=1000)
    Wz = np.zeros_like(W)
    lp, lse = oracle.logprob(x, g, 1e-6, Wz, tgt)
    np.testing.assert_array_equal(lp, np.full(len(tgt), -math.log(1000)))
    np.testing.assert_array_equal(lse, np.full(len(tgt), math.log(1000)))
    lp1, _ = oracle.logprob(x, g, 1e-6, W[:1], np.zeros(len(tgt), np.int32))
    np.testing.assert_array_equal(lp1, np.zeros(len(tgt)))


def test_logprob_normalises_over_all_targets():
    x, g, W, _ = _small_case(7, T=1, V=211)
    xs = np.repeat(x, 211, axis=0)
    lp, lse = oracle.logprob(xs, g, 1e-6, W, np.arange(211, dtype=np.int32))
    assert np.sum(np.exp(lp)) == pytest.approx(1.0, abs=1e-13)
    assert np.all(lse == lse[0])


def test_logprob_identical_w_rows_uniform():
    x, g, W, tgt = _small_case(8, V=50)
    Wsame = np.repeat(W[:1], 50, axis=0)
    lp, _ = oracle.logprob(x, g, 1e-6, Wsame, tgt)
    np.testing.assert_allclose(lp, -math.log(50), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- IS loss / D3

def _load_cases():
    with open(os.path.join(GOLDEN, "is_loss_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_is_loss_golden_closed_forms(case):
    lp = np.array([_ev(e) for e in case["logp"]])
    mu = np.array([_ev(e) for e in case["mu"]])
    out = oracle.is_loss(lp, mu, case["resp_offsets"], case["group_offsets"], np.array(case["reward"], np.float32))
    ex = case["expect"]
    assert out["loss"] == pytest.approx(_ev(ex["loss"]), rel=1e-14, abs=1e-15)
    np.testing.assert_allclose(out["coef"], [_ev(e) for e in ex["coef"]], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(out["advantage"], [_ev(e) for e in ex["advantage"]], rtol=1e-14, atol=1e-15)
    assert oracle.d3(lp, mu) == pytest.approx(_ev(ex["d3"]), rel=1e-14)


def test_is_loss_on_policy_is_zero_and_advantages_sum_to_zero():
    b = workloads.tiny()
    rng = np.random.default_rng(0)
    lp = -rng.uniform(0, 10, b.T)
    out = oracle.is_loss(lp, lp.copy(), b.resp_offsets, b.group_offsets, b.reward)
    np.testing.assert_array_equal(out["w"], np.ones(b.T))
    assert out["loss"] == 0.0
    assert oracle.d3(lp, lp.copy()) == 0.0
    go = b.group_offsets
    for gidx in range(b.G):
        assert np.sum(out["advantage"][go[gidx]:go[gidx + 1]]) == 0.0
    R = b.R
    L = np.diff(b.resp_offsets)
    want = np.repeat(-out["advantage"] / (R * L), L)
    np.testing.assert_allclose(out["coef"], want, rtol=1e-15)


def test_is_loss_constant_rewards_give_zero_coef():
    lp = np.log(np.array([0.1, 0.2, 0.3, 0.4]))
    mu = lp - 0.3
    out = oracle.is_loss(lp, mu, [0, 2, 4], [0, 2], np.array([0.7, 0.7], np.float32))
    assert np.all(out["coef"] == 0.0)
    assert out["loss"] == 0.0


def test_is_loss_coef_is_finite_difference_gradient():
    b = workloads.tiny()
    rng = np.random.default_rng(1)
    lp = -rng.uniform(0.5, 8, b.T)
    mu = lp + rng.normal(0, 0.3, b.T)
    out = oracle.is_loss(lp, mu, b.resp_offsets, b.group_offsets, b.reward)
    h = 1e-6
    for t in rng.choice(b.T, 25, replace=False):
        lpp = lp.copy(); lpp[t] += h
        lpm = lp.copy(); lpm[t] -= h
        fd = (oracle.is_loss(lpp, mu, b.resp_offsets, b.group_offsets, b.reward)["loss"]
              - oracle.is_loss(lpm, mu, b.resp_offsets, b.group_offsets, b.reward)["loss"]) / (2 * h)
        assert fd == pytest.approx(out["coef"][t], rel=1e-6, abs=1e-12)


def test_is_coef_rows_agrees_with_is_loss_on_every_row():
    b = workloads.tiny()
    rng = np.random.default_rng(3)
    lp = -rng.uniform(0.5, 8, b.T)
    mu = lp + rng.normal(0, 0.2, b.T)
    full = oracle.is_loss(lp, mu, b.resp_offsets, b.group_offsets, b.reward)["coef"]
    rows = np.array([0, 1, 7, b.T // 2, b.T - 1])
    got = oracle.is_coef_rows(lp[rows], mu[rows], rows, b.resp_offsets, b.group_offsets, b.reward)
    np.testing.assert_array_equal(got, full[rows])


def test_d3_constant_delta_and_nonnegative():
    lp = np.full(10, -2.0)
    for c in (math.log(2.0), -0.7, 1e-5, 3.0):
        assert oracle.d3(lp + c, lp) == pytest.approx(math.exp(c) - 1 - c, rel=1e-13)
    rng = np.random.default_rng(2)
    assert oracle.d3(rng.normal(0, 1, 1000), rng.normal(0, 1, 1000)) >= 0


def test_d3_equals_kl_by_enumeration():
    # Tokens drawn from mu with exact multiplicities: the token mean of
    # w - 1 - log w with w = pi/mu equals KL(mu || pi) because E_mu[w] = 1.
    from scipy.stats import entropy
    V = 6
    counts = np.array([1, 2, 3, 4, 5, 9])
    mu = counts / counts.sum()
    pi = np.array([0.3, 0.1, 0.2, 0.05, 0.15, 0.2])
    tok = np.repeat(np.arange(V), counts)
    got = oracle.d3(np.log(pi[tok]), np.log(mu[tok]))
    assert got == pytest.approx(entropy(mu, pi), rel=1e-13)


def test_d3_small_lag_noise_is_half_variance():
    rng = np.random.default_rng(4)
    sigma = 0.01
    d = rng.normal(0, sigma, 2_000_000)
    assert oracle.d3(d, np.zeros_like(d)) == pytest.approx(sigma ** 2 / 2, rel=0.01)


def test_kl_estimators_constant_delta():
    lp = np.full(7, -3.0)
    for c in (math.log(2.0), -0.4, 2.5):
        k1, k2, k3 = oracle.kl_estimators(lp + c, lp)
        assert k1 == pytest.approx(-c, rel=1e-14)
        assert k2 == pytest.approx(c * c / 2, rel=1e-14)
        assert k3 == pytest.approx(math.exp(c) - 1 - c, rel=1e-13)
    assert oracle.kl_estimators(lp, lp) == (0.0, 0.0, 0.0)


def test_kl_estimators_k1_k3_equal_kl_by_enumeration():
    # tokens drawn from mu with exact multiplicities: E_mu[-log(pi/mu)] and
    # E_mu[pi/mu - 1 - log(pi/mu)] both equal KL(mu || pi); k2 does not
    from scipy.stats import entropy
    counts = np.array([3, 1, 4, 1, 5, 9, 2, 6])
    mu = counts / counts.sum()
    pi = np.array([0.05, 0.2, 0.1, 0.15, 0.1, 0.2, 0.1, 0.1])
    tok = np.repeat(np.arange(len(counts)), counts)
    k1, k2, k3 = oracle.kl_estimators(np.log(pi[tok]), np.log(mu[tok]))
    kl = entropy(mu, pi)
    assert k1 == pytest.approx(kl, rel=1e-13)
    assert k3 == pytest.approx(kl, rel=1e-13)
    assert abs(k2 - kl) > 1e-3 * kl


def test_kl_estimators_small_noise_limit():
    rng = np.random.default_rng(5)
    sigma = 0.02
    d = rng.normal(0, sigma, 1_000_000)
    k1, k2, k3 = oracle.kl_estimators(d, np.zeros_like(d))
    assert abs(k1) < 5 * sigma / 1000
    assert k2 == pytest.approx(sigma ** 2 / 2, rel=0.01)
    assert k3 == pytest.approx(sigma ** 2 / 2, rel=0.01)


def test_peak_median_hand_values():
    assert oracle.peak_median([1.0, 2.0, 3.0, 10.0]) == (2.5, 10.0, 4.0)
    assert oracle.peak_median([3.0, 1.0, 2.0]) == (2.0, 3.0, 1.5)
    assert oracle.peak_median([0.5]) == (0.5, 0.5, 1.0)


def test_decompose_identity_and_degenerate_cases():
    rng = np.random.default_rng(6)
    a, b, m = rng.normal(-3, 1, (3, 50))
    lag, mis = oracle.decompose(a, b, m)
    np.testing.assert_allclose(lag + mis, a - m, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(lag, a - b)
    # same weights: no lag; rollout recorded the learner's own values: no mismatch
    lag0, _ = oracle.decompose(b, b, m)
    assert np.all(lag0 == 0.0)
    _, mis0 = oracle.decompose(a, b, b)
    assert np.all(mis0 == 0.0)


# ---------------------------------------------------------------- backward

def _chain_loss(xv, gv, eps, Wv, tgt, mu, ro, go, reward):
    hh, _ = oracle.rmsnorm(xv, gv, eps, round_output=False)
    z = oracle.logits(hh, Wv)
    lp, _ = oracle.log_softmax_gather(z, tgt)
    return oracle.is_loss(lp, mu, ro, go, reward)["loss"]


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(9)
    T, H, V = 6, 16, 29
    xv = rng.standard_normal((T, H))
    gv = 1 + 0.1 * rng.standard_normal(H)
    Wv = 0.3 * rng.standard_normal((V, H))
    tgt = rng.integers(0, V, T).astype(np.int32)
    ro = np.array([0, 2, 3, 6]); go = np.array([0, 3])
    reward = np.array([1.0, 0.0, 0.5], np.float32)
    mu = -np.log(V) + 0.3 * rng.standard_normal(T)
    eps = 1e-6
    hh, _ = oracle.rmsnorm(xv, gv, eps, round_output=False)
    lp, lse = oracle.log_softmax_gather(oracle.logits(hh, Wv), tgt)
    coef = oracle.is_loss(lp, mu, ro, go, reward)["coef"]
    dx = oracle.backward(xv, gv, eps, Wv, tgt, lse, coef, round_hhat=False)
    h = 1e-6
    fd = np.zeros_like(xv)
    for t in range(T):
        for k in range(H):
            xp = xv.copy(); xp[t, k] += h
            xm = xv.copy(); xm[t, k] -= h
            fd[t, k] = (_chain_loss(xp, gv, eps, Wv, tgt, mu, ro, go, reward)
                        - _chain_loss(xm, gv, eps, Wv, tgt, mu, ro, go, reward)) / (2 * h)
    np.testing.assert_allclose(dx, fd, rtol=1e-6, atol=1e-9 * np.abs(fd).max())


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(10)
    T, H, V = 9, 32, 41
    xv = rng.standard_normal((T, H))
    gv = 1 + 0.1 * rng.standard_normal(H)
    Wv = 0.2 * rng.standard_normal((V, H))
    tgt = rng.integers(0, V, T)
    ro = np.array([0, 4, 9]); go = np.array([0, 2])
    reward = np.array([1.0, 0.0], np.float32)
    mu = -np.log(V) + 0.2 * rng.standard_normal(T)
    eps = 1e-6
    xt = torch.tensor(xv, requires_grad=True)
    y = torch.nn.functional.rms_norm(xt, (H,), weight=torch.tensor(gv), eps=float(np.float32(eps)))
    logp = torch.log_softmax(y @ torch.tensor(Wv).T, dim=1)[torch.arange(T), torch.tensor(tgt)]
    w = torch.exp(logp - torch.tensor(mu))
    A = torch.tensor([0.5, -0.5], dtype=torch.float64)
    loss = -(A[0] * w[0:4].mean() + A[1] * w[4:9].mean()) / 2
    loss.backward()
    hh, _ = oracle.rmsnorm(xv, gv, eps, round_output=False)
    lp, lse = oracle.log_softmax_gather(oracle.logits(hh, Wv), tgt)
    L = oracle.is_loss(lp, mu, ro, go, reward)
    assert L["loss"] == pytest.approx(loss.item(), rel=1e-12)
    dx = oracle.backward(xv, gv, eps, Wv, tgt, lse, L["coef"], round_hhat=False)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_weight_grads_match_finite_differences():
    rng = np.random.default_rng(12)
    T, H, V = 7, 12, 23
    xv = rng.standard_normal((T, H))
    gv = 1 + 0.1 * rng.standard_normal(H)
    Wv = 0.3 * rng.standard_normal((V, H))
    tgt = rng.integers(0, V, T).astype(np.int32)
    tgt[3] = tgt[1]                     # two tokens share a target row
    ro = np.array([0, 3, 4, 7]); go = np.array([0, 3])
    reward = np.array([1.0, 0.0, 0.25], np.float32)
    mu = -np.log(V) + 0.3 * rng.standard_normal(T)
    eps = 1e-6
    hh, _ = oracle.rmsnorm(xv, gv, eps, round_output=False)
    lp, lse = oracle.log_softmax_gather(oracle.logits(hh, Wv), tgt)
    coef = oracle.is_loss(lp, mu, ro, go, reward)["coef"]
    dW, dg = oracle.weight_grads(xv, gv, eps, Wv, tgt, lse, coef, round_hhat=False)
    h = 1e-6
    fdW = np.zeros_like(Wv)
    for v in range(V):
        for k in range(H):
            Wp = Wv.copy(); Wp[v, k] += h
            Wm = Wv.copy(); Wm[v, k] -= h
            fdW[v, k] = (_chain_loss(xv, gv, eps, Wp, tgt, mu, ro, go, reward)
                         - _chain_loss(xv, gv, eps, Wm, tgt, mu, ro, go, reward)) / (2 * h)
    fdg = np.zeros_like(gv)
    for k in range(H):
        gp = gv.copy(); gp[k] += h
        gm = gv.copy(); gm[k] -= h
        fdg[k] = (_chain_loss(xv, gp, eps, Wv, tgt, mu, ro, go, reward)
                  - _chain_loss(xv, gm, eps, Wv, tgt, mu, ro, go, reward)) / (2 * h)
    np.testing.assert_allclose(dW, fdW, rtol=1e-6, atol=1e-9 * np.abs(fdW).max())
    np.testing.assert_allclose(dg, fdg, rtol=1e-6, atol=1e-9 * np.abs(fdg).max())


def test_weight_grads_match_torch_autograd_and_invariants():
    rng = np.random.default_rng(13)
    T, H, V = 10, 16, 37
    xv = rng.standard_normal((T, H))
    gv = 1 + 0.1 * rng.standard_normal(H)
    Wv = 0.2 * rng.standard_normal((V, H))
    tgt = rng.integers(0, V, T)
    mu = -np.log(V) + 0.2 * rng.standard_normal(T)
    eps = 1e-6
    Wt = torch.tensor(Wv, requires_grad=True)
    gt = torch.tensor(gv, requires_grad=True)
    y = torch.nn.functional.rms_norm(torch.tensor(xv), (H,), weight=gt, eps=float(np.float32(eps)))
    logp = torch.log_softmax(y @ Wt.T, dim=1)[torch.arange(T), torch.tensor(tgt)]
    w = torch.exp(logp - torch.tensor(mu))
    A = torch.tensor([0.5, -0.5], dtype=torch.float64)
    loss = -(A[0] * w[0:6].mean() + A[1] * w[6:10].mean()) / 2
    loss.backward()
    ro = np.array([0, 6, 10]); go = np.array([0, 2])
    reward = np.array([1.0, 0.0], np.float32)
    hh, _ = oracle.rmsnorm(xv, gv, eps, round_output=False)
    lp, lse = oracle.log_softmax_gather(oracle.logits(hh, Wv), tgt)
    coef = oracle.is_loss(lp, mu, ro, go, reward)["coef"]
    dW, dg = oracle.weight_grads(xv, gv, eps, Wv, tgt, lse, coef, round_hhat=False)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-10, atol=1e-15)
    # every column of dW sums to 0 (each dlogits row sums to 0)
    assert np.abs(dW.sum(axis=0)).max() <= 1e-14 * np.abs(dW).max() * V
    # zero coef: zero gradients
    z = oracle.weight_grads(xv, gv, eps, Wv, tgt, lse, np.zeros(T), round_hhat=False)
    assert not np.any(z[0]) and not np.any(z[1])


def test_backward_invariants():
    x, g, W, tgt = _small_case(13, T=11, H=32, V=40)
    eps = 1e-6
    lp, lse = oracle.logprob(x, g, eps, W, tgt)
    coef = np.linspace(-1, 1, 11)
    # W = 0 -> zero gradient; coef = 0 rows -> zero rows
    d0 = oracle.backward(x, g, eps, np.zeros_like(W), tgt, np.full(11, math.log(40)), coef)
    assert np.all(d0 == 0.0)
    c2 = coef.copy(); c2[3] = 0.0
    d = oracle.backward(x, g, eps, W, tgt, lse, c2)
    assert np.all(d[3] == 0.0)
    # each dlogits row sums to zero
    hh, _ = oracle.rmsnorm(x, g, eps)
    gz = oracle.logit_grad(oracle.logits(hh, oracle.bf16_decode(W)), lse, tgt, coef)
    np.testing.assert_allclose(gz.sum(axis=1), 0.0, atol=1e-15)
    # RMSNorm is scale invariant for eps -> 0, so x . dx -> 0
    dxe = oracle.rmsnorm_backward(x, g, 0.0, np.random.default_rng(0).standard_normal((11, 32)))
    xv = oracle.bf16_decode(x)
    np.testing.assert_allclose(np.sum(xv * dxe, axis=1), 0.0, atol=1e-12)


def test_learner_step_wires_the_pinned_stages():
    """learner_step is the composition of stages pinned one by one above
    (rmsnorm, logprob, is_loss, d3, backward): every output must equal the
    stage it comes from, bit for bit, and the on-policy case must reduce to
    its closed forms (D3 = 0, w = 1)."""
    b = workloads.tiny()
    lp, lse = oracle.logprob(b.x, b.gamma, b.eps, b.W, b.target)
    mu = lp + b.lag_noise.astype(np.float64)
    out = oracle.learner_step(b.x, b.gamma, b.eps, b.W, b.target, mu, b.resp_offsets,
                              b.group_offsets, b.reward)
    np.testing.assert_array_equal(out["logprob"], lp)
    np.testing.assert_array_equal(out["lse"], lse)
    L = oracle.is_loss(lp, mu, b.resp_offsets, b.group_offsets, b.reward)
    for k in ("coef", "advantage", "w"):
        np.testing.assert_array_equal(out[k], L[k])
    assert out["loss"] == L["loss"]
    assert out["d3"] == oracle.d3(lp, mu)
    np.testing.assert_array_equal(
        out["dhidden"], oracle.backward(b.x, b.gamma, b.eps, b.W, b.target, lse, L["coef"]))
    assert out["d3"] == pytest.approx(0.01 ** 2 / 2, rel=0.3)
    on = oracle.learner_step(b.x, b.gamma, b.eps, b.W, b.target, lp, b.resp_offsets,
                             b.group_offsets, b.reward)
    assert on["d3"] == 0.0
    np.testing.assert_array_equal(on["w"], 1.0)