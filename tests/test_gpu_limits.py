"""The largest shapes the ABI accepts, on the GPU, against the oracle on the
rows and columns it can afford: H = 16384 (the largest hidden size) and
V = 4,000,000 (the largest vocabulary, whose padded 256-row tiles still keep
every buffer offset below 2^31 bytes).  Tolerances as in test_gpu_parity."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16, f32, host, i32, rel_fro, say

pytestmark = pytest.mark.gpu

LP_TOL = 5e-4
DH_RTOL = 1e-3


@pytest.fixture(scope="module")
def rz():
    import invariant_logprob_is_amd as m
    m.lib()
    return m


def _case(seed, T, H, V, wstd):
    rng = np.random.default_rng(seed)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    g = workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    W = np.empty((V, H), np.uint16)
    for a in range(0, V, 262144):                 # bounded host memory
        b = min(V, a + 262144)
        W[a:b] = workloads.f32_to_bf16_bits((wstd * rng.standard_normal((b - a, H)))
                                            .astype(np.float32))
    t = rng.integers(0, V, T).astype(np.int32)
    return x, g, W, t


# 300 rows run the persistent forward; 40 rows the few-row forward, whose
# 4-stage ring then cycles through 256 stages
@pytest.mark.parametrize("T", [300, 40])
def test_largest_hidden_size(rz, gpu, T):
    H, V = 16384, 1024
    say(f"limits H={H} T={T}")
    x, g, W, t = _case(1, T, H, V, 0.01)
    d = [bf16(a, gpu) for a in (x, g, W)]
    lp, lse = rz.logprob(d[0], d[1], d[2], i32(t, gpu))
    olp, olse = oracle.logprob(x, g, 1e-6, W, t)
    assert np.abs(host(lp) - olp).max() <= LP_TOL
    coef = np.random.default_rng(2).normal(0, 1e-2, T).astype(np.float32)
    dh = rz.backward(d[0], d[1], d[2], i32(t, gpu), lse, f32(coef, gpu))
    e = rel_fro(host(dh), oracle.backward(x, g, 1e-6, W, t, olse, coef.astype(np.float64)))
    say(f"  max|dlogprob|={np.abs(host(lp) - olp).max():.2e} dhidden rel_fro={e:.2e}")
    assert e <= DH_RTOL


def test_largest_vocabulary(rz, gpu):
    T, H, V = 16, 64, 4_000_000
    say(f"limits V={V}")
    x, g, W, t = _case(3, T, H, V, 0.05)
    t[:4] = [0, V - 1, V - 256, V // 2]           # targets in the first, last and a ragged tile
    d = [bf16(a, gpu) for a in (x, g, W)]
    lp, lse = rz.logprob(d[0], d[1], d[2], i32(t, gpu))
    olp, olse = oracle.logprob(x, g, 1e-6, W, t, row_chunk=8)
    assert np.abs(host(lp) - olp).max() <= LP_TOL
    assert np.abs(host(lse) - olse).max() <= LP_TOL
    coef = np.random.default_rng(4).normal(0, 1e-2, T).astype(np.float32)
    dh = rz.backward(d[0], d[1], d[2], i32(t, gpu), lse, f32(coef, gpu))
    e = rel_fro(host(dh), oracle.backward(x, g, 1e-6, W, t, olse, coef.astype(np.float64),
                                          row_chunk=8))
    say(f"  max|dlogprob|={np.abs(host(lp) - olp).max():.2e} dhidden rel_fro={e:.2e}")
    assert e <= DH_RTOL


def test_largest_vocabulary_weight_grads(rz, gpu):
    # the learner step with dW and dgamma at V = 4,000,000: 15625 vocabulary
    # tiles in the token contraction and a one-hot bucketing over 4M rows
    T, H, V = 16, 64, 4_000_000
    say(f"limits weight grads V={V}")
    x, g, W, t = _case(5, T, H, V, 0.05)
    t[:4] = [0, V - 1, V - 256, V // 2]
    t[4] = t[5] = 1234567                           # two tokens on one target row
    ro = np.array([0, 4, 8, 12, 16], np.int64)
    go = np.array([0, 2, 4], np.int64)
    reward = np.array([1.0, 0.0, 0.0, 1.0], np.float32)
    say("  oracle logprob")
    olp, olse = oracle.logprob(x, g, 1e-6, W, t, row_chunk=8)
    mu = (olp + np.random.default_rng(6).normal(0, 0.05, T)).astype(np.float32)
    d = [bf16(a, gpu) for a in (x, g, W)]
    out = rz.learner_step(d[0], d[1], d[2], i32(t, gpu), f32(mu, gpu), ro, go, reward,
                          weight_grads=True)
    say("  oracle weight grads")
    coef = oracle.is_loss(olp, mu.astype(np.float64), ro, go, reward)["coef"]
    odW, odg = oracle.weight_grads(x, g, 1e-6, W, t, olse, coef)
    e_w = rel_fro(host(out["dW"]), odW)
    e_g = float(np.linalg.norm(host(out["dgamma"]) - odg) / np.linalg.norm(odg))
    say(f"  dW rel_fro={e_w:.2e} dgamma rel={e_g:.2e}")
    assert e_w <= DH_RTOL and e_g <= DH_RTOL
