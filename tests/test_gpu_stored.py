"""The stored-logits pair: rz_logprob_store keeps the forward's logits (as the
exponentials the backward contracts) and rz_backward_stored reads them back
instead of recomputing the LM-head GEMM.

The pair runs the same kernels in the same order per row as rz_logprob and
rz_backward, so the results must be the same bits; at a small shape dhidden
is also held to the oracle (relative Frobenius error <= 1e-3)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16, bits32, f32, host, i32, rel_fro, say

pytestmark = pytest.mark.gpu

DH_RTOL = 1e-3


@pytest.fixture(scope="module")
def rz():
    import invariant_logprob_is_amd as m
    m.lib()
    return m


def _rand_case(seed, T, H, V, wstd=0.05):
    rng = np.random.default_rng(seed)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    g = workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    W = workloads.f32_to_bf16_bits((wstd * rng.standard_normal((V, H))).astype(np.float32))
    t = rng.integers(0, V, T).astype(np.int32)
    coef = rng.normal(0, 1e-2, T).astype(np.float32)
    return x, g, W, t, coef


def _same_bits(a, b):
    return np.array_equal(bits32(a), bits32(b))


# one row; one full token tile; several vocabulary tiles with a ragged tail;
# two chunks of 32,768 rows with a ragged second chunk; the 1.5B-shaped head
# over two chunks
@pytest.mark.parametrize("T,H,V", [(1, 64, 65), (256, 128, 1000), (300, 128, 1024),
                                   (513, 320, 257), (40000, 64, 1000), (33000, 1536, 151936)])
def test_stored_pair_gives_the_recomputed_bits(rz, gpu, T, H, V):
    say(f"stored logits T={T} H={H} V={V} ({rz.logits_bytes(T, H, V) / 2**30:.2f} GiB)")
    xb, gb, Wb, tb, cb = _rand_case(T + H + V, T, H, V, wstd=0.05 if H < 1536 else 0.02)
    x, g, W, t, coef = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu), f32(cb, gpu)
    lp, lse = rz.logprob(x, g, W, t)
    dh = rz.backward(x, g, W, t, lse, coef)
    slp, slse, logits = rz.logprob_store(x, g, W, t)
    sdh = rz.backward_stored(x, g, W, t, slse, coef, logits)
    torch.cuda.synchronize()
    assert _same_bits(slp, lp)
    assert _same_bits(slse, lse)
    assert _same_bits(sdh, dh)
    assert np.isfinite(host(sdh)).all()
    del logits


def test_stored_pair_out_of_range_targets(rz, gpu):
    """Out-of-range targets give NaN in exactly those rows, in the same bits
    as the recomputing pair."""
    T, H, V = 300, 128, 1000
    say(f"stored logits with out-of-range targets T={T} H={H} V={V}")
    xb, gb, Wb, tb, cb = _rand_case(3, T, H, V)
    tb[[4, 77, 299]] = [V, -1, V + 12345]
    x, g, W, t, coef = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu), f32(cb, gpu)
    lp, lse = rz.logprob(x, g, W, t)
    dh = rz.backward(x, g, W, t, lse, coef)
    slp, slse, logits = rz.logprob_store(x, g, W, t)
    sdh = rz.backward_stored(x, g, W, t, slse, coef, logits)
    torch.cuda.synchronize()
    assert _same_bits(slp, lp) and _same_bits(slse, lse) and _same_bits(sdh, dh)
    bad = np.zeros(T, bool)
    bad[[4, 77, 299]] = True
    assert np.isnan(host(slp)[bad]).all() and np.isfinite(host(slp)[~bad]).all()
    assert np.isnan(host(sdh)[bad]).all() and np.isfinite(host(sdh)[~bad]).all()


def test_stored_pair_matches_the_oracle(rz, gpu):
    T, H, V = 300, 128, 3000
    say(f"stored logits vs oracle T={T} H={H} V={V}")
    xb, gb, Wb, tb, cb = _rand_case(5, T, H, V)
    x, g, W, t, coef = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu), f32(cb, gpu)
    lp, lse, logits = rz.logprob_store(x, g, W, t)
    dh = rz.backward_stored(x, g, W, t, lse, coef, logits)
    olp, olse = oracle.logprob(xb, gb, 1e-6, Wb, tb)
    odh = oracle.backward(xb, gb, 1e-6, Wb, tb, olse, cb.astype(np.float64))
    e = rel_fro(host(dh), odh)
    say(f"  max|dlogprob|={np.abs(host(lp) - olp).max():.3e} dhidden rel_fro={e:.3e}")
    assert np.abs(host(lp) - olp).max() <= 5e-4
    assert e <= DH_RTOL


def test_stored_buffer_is_reusable_for_a_smaller_batch(rz, gpu):
    """A buffer sized for a large batch serves a smaller one: the layout of
    each chunk depends only on the chunk's own rows."""
    H, V = 128, 1024
    big = rz.logits_bytes(5000, H, V)
    buf = torch.empty(big, dtype=torch.uint8, device=gpu)
    for T in (5000, 777):
        say(f"reused stored-logits buffer T={T}")
        xb, gb, Wb, tb, cb = _rand_case(T, T, H, V)
        x, g, W, t, coef = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu), f32(cb, gpu)
        lp, lse = rz.logprob(x, g, W, t)
        dh = rz.backward(x, g, W, t, lse, coef)
        slp, slse, lg = rz.logprob_store(x, g, W, t, logits=buf)
        assert lg is buf
        sdh = rz.backward_stored(x, g, W, t, slse, coef, buf)
        torch.cuda.synchronize()
        assert _same_bits(slp, lp)
        assert _same_bits(sdh, dh)


def test_binding_rejects_a_short_stored_buffer(rz, gpu):
    H, V, T = 128, 1024, 300
    xb, gb, Wb, tb, cb = _rand_case(1, T, H, V)
    x, g, W, t, coef = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu), f32(cb, gpu)
    short = torch.empty(rz.logits_bytes(T, H, V) - 256, dtype=torch.uint8, device=gpu)
    with pytest.raises(ValueError):
        rz.logprob_store(x, g, W, t, logits=short)
    _, lse, lg = rz.logprob_store(x, g, W, t)
    with pytest.raises(rz.RzError):
        rz.backward_stored(x, g, W, t, lse, coef, lg[:-256])
