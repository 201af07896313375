"""The learner step's weight gradients (dW of the LM head, dgamma of the
RMSNorm) through the C ABI, against the float64 oracle.

Tolerance: relative Frobenius error <= 1e-3 on dW and relative error
<= 1e-3 on dgamma, the bound stated for dhidden (the same products, with
coef p rounded once to bf16 for the MFMA contraction, the one-hot term and
each token's dominant probabilities exact).  Determinism is bit-exact, and
the other outputs of the step must not change when the gradients are
requested."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16, bits32, f32, host, i32, rel_fro, say

pytestmark = pytest.mark.gpu

DW_RTOL = 1e-3


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


def _case(seed, T, H, V, same_target=False, wstd=0.05, zipf=False):
    rng = np.random.default_rng(seed)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    g = workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    W = workloads.f32_to_bf16_bits((wstd * rng.standard_normal((V, H))).astype(np.float32))
    t = rng.integers(0, V, T).astype(np.int32)
    if same_target:
        t[:] = V // 3
    if zipf:
        t = workloads.zipf_targets(seed, T, V)
    mu = (-math.log(V) + rng.normal(0, 0.3, T)).astype(np.float32)
    return x, g, W, t, mu


def _oracle_grads(x, g, W, t, mu, ro, go, reward):
    olp, olse = oracle.logprob(x, g, 1e-6, W, t)
    coef = oracle.is_loss(olp, mu.astype(np.float64), ro, go, reward)["coef"]
    return oracle.weight_grads(x, g, 1e-6, W, t, olse, coef)


@pytest.mark.parametrize("T,H,V,same,zstd", [(300, 128, 1024, False, None), (257, 192, 513, False, None),
                                             (1, 64, 65, False, None), (40000, 128, 1000, False, None),
                                             (600, 64, 300, True, None),
                                             # the largest hidden size: 64 hidden tiles, the
                                             # grouped tile raster of the token contraction
                                             (200, 16384, 700, False, 0.8),
                                             # peaked rows: the dominant probabilities
                                             # are among the entries made exact
                                             (300, 128, 3000, False, 5.7),
                                             (200, 16384, 700, False, 6.4)])
def test_weight_grads_match_oracle(rz, gpu, T, H, V, same, zstd):
    say(f"weight grads T={T} H={H} V={V} same_target={same} logit std={zstd}")
    wstd = 0.05 if zstd is None else zstd / math.sqrt(H)
    x, g, W, t, mu = _case(T + H + V, T, H, V, same, wstd)
    ro, go, reward = _ragged(T, T, 1, 1) if T == 1 else _ragged(T, T, 2, 2) if T < 8 else \
        _ragged(T, T, 4, 4)
    d = [bf16(a, gpu) for a in (x, g, W)]
    out = rz.learner_step(d[0], d[1], d[2], i32(t, gpu), f32(mu, gpu), ro, go, reward,
                          weight_grads=True)
    odW, odg = _oracle_grads(x, g, W, t, mu, ro, go, reward)
    if not np.any(odW):
        # one response alone in its group: A = 0, so every gradient is 0
        assert not np.any(host(out["dW"])) and not np.any(host(out["dgamma"]))
        return
    e_w = rel_fro(host(out["dW"]), odW)
    e_g = float(np.linalg.norm(host(out["dgamma"]) - odg) / np.linalg.norm(odg))
    say(f"  dW rel_fro={e_w:.2e} dgamma rel={e_g:.2e}")
    assert e_w <= DW_RTOL and e_g <= DW_RTOL


def test_weight_grads_zipfian_targets(rz, gpu):
    """Targets with Zipfian frequencies and one token id holding 30% of every
    chunk (as end-of-text or newline tokens do): the one-hot terms pile into
    buckets of up to ~10,000 tokens, summed in token order."""
    T, H, V = 40000, 128, 1000
    x, g, W, t, mu = _case(91, T, H, V, zipf=True)
    top = np.bincount(t[:32768], minlength=V).max()
    say(f"zipfian targets: the largest bucket of the first chunk holds {top} of 32768 tokens")
    assert top >= 0.25 * 32768
    ro, go, reward = _ragged(91, T, 4, 4)
    d = [bf16(a, gpu) for a in (x, g, W)]
    out = rz.learner_step(d[0], d[1], d[2], i32(t, gpu), f32(mu, gpu), ro, go, reward,
                          weight_grads=True)
    odW, odg = _oracle_grads(x, g, W, t, mu, ro, go, reward)
    e_w = rel_fro(host(out["dW"]), odW)
    e_g = float(np.linalg.norm(host(out["dgamma"]) - odg) / np.linalg.norm(odg))
    say(f"  dW rel_fro={e_w:.2e} dgamma rel={e_g:.2e}")
    assert e_w <= DW_RTOL and e_g <= DW_RTOL
    again = rz.learner_step(d[0], d[1], d[2], i32(t, gpu), f32(mu, gpu), ro, go, reward,
                            weight_grads=True)
    np.testing.assert_array_equal(bits32(again["dW"]), bits32(out["dW"]))


def test_weight_grads_leave_other_outputs_unchanged_and_are_deterministic(rz, gpu):
    T, H, V = 33000, 128, 777                      # two chunks, ragged last one
    x, g, W, t, mu = _case(5, T, H, V)
    ro, go, reward = _ragged(5, T, 4, 4)
    d = [bf16(a, gpu) for a in (x, g, W)]
    args = (d[0], d[1], d[2], i32(t, gpu), f32(mu, gpu), ro, go, reward)
    plain = rz.learner_step(*args)
    runs = [rz.learner_step(*args, weight_grads=True) for _ in range(2)]
    for k in ("logprob", "lse", "coef", "dhidden"):
        np.testing.assert_array_equal(bits32(runs[0][k]), bits32(plain[k]))
    for k in ("loss", "d3"):
        assert host(runs[0][k])[0] == host(plain[k])[0]
    for k in ("dW", "dgamma"):
        np.testing.assert_array_equal(bits32(runs[0][k]), bits32(runs[1][k]))


def test_weight_grads_zero_coef_gives_zero(rz, gpu):
    # all rewards equal in every group: A = 0, coef = 0, every gradient 0
    T, H, V = 400, 64, 300
    x, g, W, t, mu = _case(9, T, H, V)
    ro, go, _ = _ragged(9, T, 4, 4)
    reward = np.ones(16, np.float32)
    d = [bf16(a, gpu) for a in (x, g, W)]
    out = rz.learner_step(d[0], d[1], d[2], i32(t, gpu), f32(mu, gpu), ro, go, reward,
                          weight_grads=True)
    assert torch.count_nonzero(out["dW"]).item() == 0
    assert torch.count_nonzero(out["dgamma"]).item() == 0
