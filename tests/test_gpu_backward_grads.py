"""rz_backward_grads: the gradient of sum_t coef_t logprob_t with respect to
the hidden states, the LM-head weight and the RMSNorm weight for any
per-token coef, and the differentiable logprob_fn built on it.

With the learner step's lse and coef the three gradients must equal the
step's bits (the same kernels in the same order); with stored logits they
must equal the recomputing call's; for a random coef they are held to the
oracle at the weight-gradient bound (relative Frobenius <= 1e-3 on dhidden
and dW, relative <= 1e-3 on dgamma)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16, bits32, f32, host, i32, rel_fro, say

pytestmark = pytest.mark.gpu

RTOL = 1e-3


@pytest.fixture(scope="module")
def rz():
    import invariant_logprob_is_amd as m
    m.lib()
    return m


def _case(seed, T, H, V, wstd=0.05):
    rng = np.random.default_rng(seed)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    g = workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    W = workloads.f32_to_bf16_bits((wstd * rng.standard_normal((V, H))).astype(np.float32))
    t = rng.integers(0, V, T).astype(np.int32)
    return x, g, W, t


def _same(a, b):
    return np.array_equal(bits32(a), bits32(b))


def test_step_coef_gives_the_step_bits(rz, gpu):
    T, H, V, R, G = 40000, 128, 1000, 16, 4           # two chunks, the second ragged
    say(f"backward_grads vs learner_step T={T} H={H} V={V}")
    xb, gb, Wb, tb = _case(21, T, H, V)
    rng = np.random.default_rng(22)
    cuts = np.sort(rng.choice(np.arange(1, T), R - 1, replace=False))
    ro = np.concatenate([[0], cuts, [T]]).astype(np.int64)
    go = np.arange(0, R + 1, R // G, dtype=np.int64)
    reward = (rng.random(R) < 0.5).astype(np.float32)
    mu = (-math.log(V) + rng.normal(0, 0.3, T)).astype(np.float32)
    x, g, W, t = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu)
    out = rz.learner_step(x, g, W, t, f32(mu, gpu), torch.from_numpy(ro).to(gpu),
                          torch.from_numpy(go).to(gpu), f32(reward, gpu), weight_grads=True)
    o = rz.backward_grads(x, g, W, t, out["lse"], out["coef"])
    torch.cuda.synchronize()
    assert _same(o["dhidden"], out["dhidden"])
    assert _same(o["dW"], out["dW"])
    assert _same(o["dgamma"], out["dgamma"])


@pytest.mark.parametrize("T,H,V", [(300, 128, 3000), (1, 64, 65), (100, 192, 513)])
def test_random_coef_matches_the_oracle(rz, gpu, T, H, V):
    say(f"backward_grads vs oracle T={T} H={H} V={V}")
    xb, gb, Wb, tb = _case(T + V, T, H, V)
    coef = np.random.default_rng(T).normal(0, 1e-2, T).astype(np.float32)
    x, g, W, t = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu)
    lp, lse = rz.logprob(x, g, W, t)
    o = rz.backward_grads(x, g, W, t, lse, f32(coef, gpu))
    olp, olse = oracle.logprob(xb, gb, 1e-6, Wb, tb)
    c64 = coef.astype(np.float64)
    odh = oracle.backward(xb, gb, 1e-6, Wb, tb, olse, c64)
    odW, odg = oracle.weight_grads(xb, gb, 1e-6, Wb, tb, olse, c64)
    e_dh = rel_fro(host(o["dhidden"]), odh)
    e_dw = rel_fro(host(o["dW"]), odW)
    e_dg = rel_fro(host(o["dgamma"]), odg)
    say(f"  dhidden {e_dh:.2e} dW {e_dw:.2e} dgamma {e_dg:.2e}")
    assert e_dh <= RTOL and e_dw <= RTOL and e_dg <= RTOL
    # dhidden is rz_backward's, bit for bit
    assert _same(o["dhidden"], rz.backward(x, g, W, t, lse, f32(coef, gpu)))


def test_stored_logits_give_the_recomputed_bits(rz, gpu):
    T, H, V = 40000, 64, 1000
    say(f"backward_grads from stored logits T={T} H={H} V={V}")
    xb, gb, Wb, tb = _case(31, T, H, V)
    coef = np.random.default_rng(32).normal(0, 1e-4, T).astype(np.float32)
    x, g, W, t, c = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu), f32(coef, gpu)
    lp, lse, logits = rz.logprob_store(x, g, W, t)
    a = rz.backward_grads(x, g, W, t, lse, c)
    b = rz.backward_grads(x, g, W, t, lse, c, logits=logits)
    torch.cuda.synchronize()
    for k in ("dhidden", "dW", "dgamma"):
        assert _same(a[k], b[k]), k


def test_logprob_fn_autograd(rz, gpu):
    T, H, V = 300, 128, 1000
    say(f"logprob_fn autograd T={T} H={H} V={V}")
    xb, gb, Wb, tb = _case(41, T, H, V)
    c = f32(np.random.default_rng(42).normal(0, 1e-2, T).astype(np.float32), gpu)
    t = i32(tb, gpu)
    x, g, W = (bf16(a, gpu).requires_grad_(True) for a in (xb, gb, Wb))
    lp = rz.logprob_fn(x, g, W, t)
    ref_lp, ref_lse = rz.logprob(x.detach(), g.detach(), W.detach(), t)
    assert _same(lp.detach(), ref_lp)
    (lp * c).sum().backward()
    o = rz.backward_grads(x.detach(), g.detach(), W.detach(), t, ref_lse, c)
    torch.cuda.synchronize()
    for grad, k in ((x.grad, "dhidden"), (g.grad, "dgamma"), (W.grad, "dW")):
        assert grad.dtype == torch.bfloat16, k
        assert torch.equal(grad, o[k].to(torch.bfloat16)), k
    # only the hidden states: the plain backward
    x2 = bf16(xb, gpu).requires_grad_(True)
    (rz.logprob_fn(x2, g.detach(), W.detach(), t) * c).sum().backward()
    dh = rz.backward(x2.detach(), g.detach(), W.detach(), t, ref_lse, c)
    assert torch.equal(x2.grad, dh.to(torch.bfloat16))
