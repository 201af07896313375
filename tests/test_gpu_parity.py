"""Parity of the HIP path (through the C ABI) with the float64 oracle, plus
closed forms, edge shapes, determinism and small-scale batch invariance.

Tolerances: |d logprob| <= 5e-4; relative error <= 1e-3 on loss and D3;
relative Frobenius error <= 1e-3 on dhidden.  Invariance and determinism are
bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16, bits32, f32, host, i32, rel_fro, say

pytestmark = pytest.mark.gpu

LP_TOL = 5e-4
LOSS_RTOL = 1e-3
DH_RTOL = 1e-3


@pytest.fixture(scope="module")
def rz():
    import invariant_logprob_is_amd as m
    m.lib()  # fail loudly if the library is missing
    return m


@pytest.fixture(scope="module")
def tiny():
    return workloads.tiny()


def _dev_head(b, dev):
    return bf16(b.x, dev), bf16(b.gamma, dev), bf16(b.W, dev), i32(b.target, dev)


def _rand_case(seed, T, H, V, wstd=0.02):
    rng = np.random.default_rng(seed)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    g = workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    W = workloads.f32_to_bf16_bits((wstd * rng.standard_normal((V, H))).astype(np.float32))
    t = rng.integers(0, V, T).astype(np.int32)
    return x, g, W, t


# ----------------------------------------------------------------- forward

def test_tiny_logprob_matches_oracle(rz, gpu, tiny):
    say(f"tiny logprob T={tiny.T} H={tiny.H} V={tiny.V}")
    x, g, W, t = _dev_head(tiny, gpu)
    lp, lse = rz.logprob(x, g, W, t, tiny.eps)
    torch.cuda.synchronize()
    olp, olse = oracle.logprob(tiny.x, tiny.gamma, tiny.eps, tiny.W, tiny.target)
    d = np.abs(host(lp) - olp)
    say(f"  max|dlogprob|={d.max():.3e} max|dlse|={np.abs(host(lse) - olse).max():.3e}")
    assert d.max() <= LP_TOL
    assert np.abs(host(lse) - olse).max() <= LP_TOL
    # the fp32 accumulation should be far inside the contract
    assert d.max() <= 2e-5


# The contraction over the vocabulary runs Vp / 64 stages (Vp = V rounded up
# to 64), with separate prologue and tail paths for 1, 2 and 3 stages: V = 64,
# 128 and 129 / 192 take them.  A batch of one token tile (T <= 256) runs the
# forward with the deep W ring, skipping the token blocks with no row (T < 256:
# 128 leaves two waves' blocks empty) or not (T = 256).
@pytest.mark.parametrize("T,H,V", [(1, 64, 65), (255, 128, 1000), (257, 192, 513),
                                   (600, 64, 300), (513, 320, 256), (40, 1536, 2048),
                                   (3, 128, 64), (33, 64, 128), (300, 128, 129),
                                   (77, 256, 192), (256, 128, 1000), (128, 192, 3000)])
def test_edge_shapes_logprob_and_backward(rz, gpu, T, H, V):
    say(f"edge shape T={T} H={H} V={V}")
    xb, gb, Wb, tb = _rand_case(T * 7 + H + V, T, H, V, wstd=0.05)
    x, g, W, t = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu)
    lp, lse = rz.logprob(x, g, W, t)
    olp, olse = oracle.logprob(xb, gb, 1e-6, Wb, tb)
    assert np.abs(host(lp) - olp).max() <= LP_TOL
    assert np.abs(host(lse) - olse).max() <= LP_TOL
    coef = np.random.default_rng(T).normal(0, 1e-2, T).astype(np.float32)
    dh = rz.backward(x, g, W, t, lse, f32(coef, gpu))
    odh = oracle.backward(xb, gb, 1e-6, Wb, tb, olse, coef.astype(np.float64))
    e = rel_fro(host(dh), odh)
    say(f"  max|dlogprob|={np.abs(host(lp) - olp).max():.3e} dhidden rel_fro={e:.3e}")
    assert e <= DH_RTOL


@pytest.mark.parametrize("wstd", [0.5, 8.0])
def test_backward_wide_logit_range(rz, gpu, wstd):
    """Logits spread over hundreds of nats: the per-tile references of the
    stored e differ by up to the flush limit of the exponent shift, and whole
    tiles drop below it.  At wstd = 8 (logits up to ~475) the rows are nearly
    one-hot, dhidden ~ coef (W[target] - W[argmax]): the dominant probability
    is one of the entries made exact, so the bound stays 1e-3."""
    T, H, V = 300, 128, 3000
    say(f"wide logits wstd={wstd}")
    xb, gb, Wb, tb = _rand_case(11 + int(wstd * 10), T, H, V, wstd=wstd)
    x, g, W, t = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu)
    lp, lse = rz.logprob(x, g, W, t)
    olp, olse = oracle.logprob(xb, gb, 1e-6, Wb, tb)
    # logits are large here: the tolerance is on the float32 result
    assert np.abs(host(lse) - olse).max() <= LP_TOL + 4e-7 * np.abs(olse).max()
    assert np.abs(host(lp) - olp).max() <= LP_TOL + 4e-7 * np.abs(olse).max()
    coef = np.random.default_rng(T).normal(0, 1e-2, T).astype(np.float32)
    dh = rz.backward(x, g, W, t, lse, f32(coef, gpu))
    odh = oracle.backward(xb, gb, 1e-6, Wb, tb, olse, coef.astype(np.float64))
    e = rel_fro(host(dh), odh)
    say(f"  logit range {olse.min():.1f}..{olse.max():.1f} dhidden rel_fro={e:.3e}")
    assert e <= DH_RTOL


def test_w_zero_gives_exactly_uniform(rz, gpu):
    T, H, V = 300, 128, 1000
    xb, gb, _, tb = _rand_case(3, T, H, V)
    W = torch.zeros(V, H, dtype=torch.bfloat16, device=gpu)
    lp, lse = rz.logprob(bf16(xb, gpu), bf16(gb, gpu), W, i32(tb, gpu))
    want = np.float32(-math.log(V))
    np.testing.assert_array_equal(host(lp), np.full(T, want, np.float32))
    np.testing.assert_array_equal(host(lse), np.full(T, -want, np.float32))
    # and the gradient through W = 0 is exactly zero
    dh = rz.backward(bf16(xb, gpu), bf16(gb, gpu), W, i32(tb, gpu), lse,
                     torch.ones(T, dtype=torch.float32, device=gpu))
    assert torch.count_nonzero(dh).item() == 0


def test_single_vocab_entry_gives_zero(rz, gpu):
    # log 1 = 0.  The lone term is 2^(z log2 e - m) 2^m with the integer
    # reference m, evaluated in float32, so lse matches z to float rounding;
    # lse is never taken below the max logit, so logprob stays <= 0.
    T, H = 77, 64
    xb, gb, Wb, _ = _rand_case(4, T, H, 1)
    lp, _ = rz.logprob(bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu),
                       torch.zeros(T, dtype=torch.int32, device=gpu))
    a = host(lp)
    assert np.all(a <= 0) and np.all(a >= -1e-6)


def test_row_normalises_over_every_target(rz, gpu):
    # one row evaluated with each of the V targets: the V copies must share
    # their lse bits (they sit at different batch positions) and sum to 1.
    H, V = 256, 1500
    xb, gb, Wb, _ = _rand_case(5, 1, H, V, wstd=0.1)
    xs = np.repeat(xb, V, axis=0)
    lp, lse = rz.logprob(bf16(xs, gpu), bf16(gb, gpu), bf16(Wb, gpu),
                         i32(np.arange(V), gpu))
    L = bits32(lse)
    assert np.all(L == L[0])
    assert abs(float(np.sum(np.exp(host(lp).astype(np.float64)))) - 1.0) <= 1e-5
    assert np.all(host(lp) <= 0)


def test_out_of_range_target_is_nan_only_there(rz, gpu):
    T, H, V = 64, 128, 512
    xb, gb, Wb, tb = _rand_case(6, T, H, V)
    tb2 = tb.copy()
    tb2[5] = V
    tb2[9] = -1
    lp, _ = rz.logprob(bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb2, gpu))
    lp0, _ = rz.logprob(bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu))
    a, b = host(lp), host(lp0)
    assert np.isnan(a[5]) and np.isnan(a[9])
    keep = np.ones(T, bool); keep[[5, 9]] = False
    np.testing.assert_array_equal(a[keep].view(np.uint32), b[keep].view(np.uint32))


# ----------------------------------------------------------------- loss / D3

def test_tiny_end_to_end_loss_d3_coef(rz, gpu, tiny):
    olp, olse = oracle.logprob(tiny.x, tiny.gamma, tiny.eps, tiny.W, tiny.target)
    mu = (olp + tiny.lag_noise).astype(np.float32)    # rollout logprob = oracle logprob + noise
    ref = oracle.is_loss(olp, mu.astype(np.float64), tiny.resp_offsets, tiny.group_offsets, tiny.reward)
    ref_d3 = oracle.d3(olp, mu.astype(np.float64))
    x, g, W, t = _dev_head(tiny, gpu)
    lp, lse = rz.logprob(x, g, W, t)
    mud = f32(mu, gpu)
    loss, coef, adv = rz.is_loss(lp, mud, tiny.resp_offsets, tiny.group_offsets, tiny.reward)
    d3 = rz.d3(lp, mud)
    gl, gd = host(loss)[0], host(d3)[0]
    kappa = np.sum(np.abs(ref["advantage"] * np.add.reduceat(ref["w"], tiny.resp_offsets[:-1])
                          / np.diff(tiny.resp_offsets))) / tiny.R / abs(ref["loss"])
    say(f"  loss gpu={gl:.9e} oracle={ref['loss']:.9e} rel={abs(gl / ref['loss'] - 1):.2e} kappa={kappa:.1f}")
    say(f"  d3   gpu={gd:.9e} oracle={ref_d3:.9e} rel={abs(gd / ref_d3 - 1):.2e}")
    assert abs(gl - ref["loss"]) <= LOSS_RTOL * abs(ref["loss"])
    assert abs(gd - ref_d3) <= LOSS_RTOL * abs(ref_d3)
    np.testing.assert_allclose(host(coef), ref["coef"], rtol=1e-4, atol=0)
    np.testing.assert_allclose(host(adv), ref["advantage"], rtol=1e-7, atol=1e-7)
    # backward end to end
    dh = rz.backward(x, g, W, t, lse, coef)
    odh = oracle.backward(tiny.x, tiny.gamma, tiny.eps, tiny.W, tiny.target, olse, ref["coef"])
    e = rel_fro(host(dh), odh)
    say(f"  dhidden rel_fro={e:.3e}")
    assert e <= DH_RTOL


def _seeded_lp_mu(T, seed, sigma=0.05, tails=0.0):
    # synthetic log-probabilities that come from neither implementation
    rng = np.random.default_rng(seed)
    lp = (-np.abs(rng.normal(11.0, 2.0, T))).astype(np.float32)
    mu = (lp + rng.normal(0, sigma, T)).astype(np.float32)
    if tails:
        k = rng.choice(T, int(tails * T), replace=False)
        mu[k] += rng.choice([-3.0, 3.0], len(k)).astype(np.float32)
    return lp, mu


@pytest.mark.parametrize("cfg", ["tiny", "qwen15b", "qwen4b_lag64", "a3b30_head"])
def test_is_loss_and_d3_stage_on_seeded_inputs(rz, gpu, cfg):
    b = workloads.CONFIGS[cfg](with_W=False, with_x=False) if cfg != "tiny" else workloads.tiny()
    say(f"is_loss stage {cfg}: T={b.T} R={b.R} G={b.G}")
    lp, mu = _seeded_lp_mu(b.T, 100 + b.R, sigma=0.2 if "4b" in cfg else 0.05,
                           tails=0.01 if "4b" in cfg else 0.0)
    ref = oracle.is_loss(lp.astype(np.float64), mu.astype(np.float64), b.resp_offsets,
                         b.group_offsets, b.reward)
    ref_d3 = oracle.d3(lp.astype(np.float64), mu.astype(np.float64))
    lpd, mud = f32(lp, gpu), f32(mu, gpu)
    loss, coef, adv = rz.is_loss(lpd, mud, b.resp_offsets, b.group_offsets, b.reward)
    d3 = rz.d3(lpd, mud)
    gl, gd = host(loss)[0], host(d3)[0]
    say(f"  loss rel={abs(gl / ref['loss'] - 1):.2e} d3 rel={abs(gd / ref_d3 - 1):.2e}")
    assert abs(gl - ref["loss"]) <= 1e-9 * abs(ref["loss"])   # same inputs: fp64 both sides
    assert abs(gd - ref_d3) <= 1e-9 * abs(ref_d3)
    np.testing.assert_allclose(host(coef), ref["coef"], rtol=2e-7, atol=0)
    np.testing.assert_allclose(host(adv), ref["advantage"], rtol=1e-7, atol=1e-7)


def test_on_policy_closed_forms(rz, gpu, tiny):
    # mu = logprob exactly: w = 1, D3 = 0, loss = 0, coef = -A/(R L)
    x, g, W, t = _dev_head(tiny, gpu)
    lp, _ = rz.logprob(x, g, W, t)
    loss, coef, adv = rz.is_loss(lp, lp.clone(), tiny.resp_offsets, tiny.group_offsets, tiny.reward)
    assert host(rz.d3(lp, lp.clone()))[0] == 0.0
    assert host(loss)[0] == 0.0
    A = oracle.advantages(tiny.reward, tiny.group_offsets)
    L = np.diff(tiny.resp_offsets)
    np.testing.assert_array_equal(host(coef), np.repeat(-A / (tiny.R * L), L).astype(np.float32))
    # constant shift delta = ln 2: D3 = 1 - ln 2
    d3 = host(rz.d3(lp, lp - math.log(2.0)))[0]
    assert d3 == pytest.approx(1 - math.log(2), rel=1e-6)


def _malformed_offsets(tiny, gpu, kind):
    ro = torch.tensor(tiny.resp_offsets, device=gpu)
    go = torch.tensor(tiny.group_offsets, device=gpu)
    if kind == "empty_response":
        ro[3] = ro[2]
    elif kind == "overlap":
        ro[3] = ro[1]                               # responses overlap, offsets not increasing
    elif kind == "short_end":
        ro[-1] = ro[-1] - 1                         # does not end at T
    else:
        go[1] = go[0]                               # an empty group
    return ro, go


@pytest.mark.parametrize("kind", ["empty_response", "overlap", "short_end", "empty_group"])
def test_malformed_device_offsets_give_nan(rz, gpu, tiny, kind):
    """Offsets that live on the device are checked there: a malformed
    structure gives NaN for the loss, every coef and every advantage
    (rz_is_loss), and for the loss, coef and every dhidden row
    (rz_learner_step)."""
    ro, go = _malformed_offsets(tiny, gpu, kind)
    lp = torch.full((tiny.T,), -3.0, device=gpu)
    loss, coef, adv = rz.is_loss(lp, lp + 0.1, ro, go, tiny.reward)
    assert np.isnan(host(loss)[0])
    assert np.all(np.isnan(host(coef))) and np.all(np.isnan(host(adv)))
    x, g, W, t = _dev_head(tiny, gpu)
    out = rz.learner_step(x, g, W, t, lp + 0.1, ro, go, tiny.reward)
    assert np.isnan(host(out["loss"])[0])
    assert np.all(np.isnan(host(out["coef"])))
    assert np.all(np.isnan(host(out["dhidden"])))
    # the log-probabilities do not depend on the structure
    lp0, _ = rz.logprob(x, g, W, t)
    np.testing.assert_array_equal(bits32(out["logprob"]), bits32(lp0))


# ----------------------------------------------------------------- determinism / invariance

def test_run_to_run_bitwise_determinism(rz, gpu, tiny):
    x, g, W, t = _dev_head(tiny, gpu)
    mu = f32(tiny.lag_noise - 7.0, gpu)
    outs = []
    for _ in range(3):
        lp, lse = rz.logprob(x, g, W, t)
        loss, coef, _ = rz.is_loss(lp, mu, tiny.resp_offsets, tiny.group_offsets, tiny.reward)
        d3 = rz.d3(lp, mu)
        dh = rz.backward(x, g, W, t, lse, coef)
        outs.append([host(v).tobytes() for v in (lp, lse, loss, coef, d3, dh)])
    assert outs[0] == outs[1] == outs[2]


def test_small_batch_invariance(rz, gpu):
    H, V = 128, 1000
    xb, gb, Wb, tb = _rand_case(9, 40, H, V)
    fx, ft = workloads.rows_only(9, 5, 3000, H, V)
    g, W = bf16(gb, gpu), bf16(Wb, gpu)
    ref_lp, ref_lse = rz.logprob(bf16(xb, gpu), g, W, i32(tb, gpu))
    ref = (bits32(ref_lp), bits32(ref_lse))
    rng = np.random.default_rng(0)
    for B in (1, 2, 7, 255, 256, 257, 1000, 3000):
        for k in range(0, 40, max(1, min(B, 40))):
            ids = np.arange(k, min(40, k + B))
            pos = np.sort(rng.choice(B, len(ids), replace=False))
            bx = fx[:B].copy(); bt = ft[:B].copy()
            bx[pos] = xb[ids]; bt[pos] = tb[ids]
            lp, lse = rz.logprob(bf16(bx, gpu), g, W, i32(bt, gpu))
            np.testing.assert_array_equal(bits32(lp)[pos], ref[0][ids])
            np.testing.assert_array_equal(bits32(lse)[pos], ref[1][ids])
