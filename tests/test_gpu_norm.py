"""The final RMSNorm alone (rz_rmsnorm) against the float64 oracle.

This is the first stage of the staged parity: the bf16 bits of hhat that the
LM head consumes, and the per-row r, checked directly instead of only through
the log-probabilities.  The second stage feeds the GPU's hhat to the oracle's
logits and log-softmax and compares with rz_logprob."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16, host, i32, say

pytestmark = pytest.mark.gpu

# Input rows come from seed streams of their own (master seeds 11-17), apart
# from the workloads' (0-4).


@pytest.fixture(scope="module")
def rz(gpu):
    import invariant_logprob_is_amd as m
    m.lib()
    return m


def _bits(t: torch.Tensor) -> np.ndarray:
    return host(t.view(torch.int16)).view(np.uint16)


def _oracle_bits(hhat64: np.ndarray) -> np.ndarray:
    # the oracle's hhat values are bf16 numbers: their float32 images carry
    # the bf16 bits in the top half exactly
    return (np.ascontiguousarray(hhat64, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _ulp_gap(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between two arrays of bf16 bits (sign-magnitude
    mapped to an ordered integer line)."""
    def ordered(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def _check_against_oracle(rz, gpu, x_bits, g_bits, eps, what):
    x, g = bf16(x_bits, gpu), bf16(g_bits, gpu)
    hh, rs = rz.rmsnorm(x, g, eps)
    torch.cuda.synchronize()
    o_hh, o_r = oracle.rmsnorm(x_bits, g_bits, eps)
    gb, ob = _bits(hh), _oracle_bits(o_hh)
    gap = _ulp_gap(gb, ob)
    n_diff = int(np.count_nonzero(gap))
    rel_r = float(np.max(np.abs(host(rs).astype(np.float64) - o_r) / o_r))
    say(f"{what}: T={x_bits.shape[0]} H={x_bits.shape[1]}: {n_diff} of {gb.size} hhat "
        f"elements differ (max {int(gap.max())} bf16 steps); max rel err of r {rel_r:.2e}")
    # staged parity, first stage: >= 99.99% of the elements bit-equal, none
    # more than one bf16 step apart; r to 1e-6
    assert n_diff <= 1e-4 * gb.size
    assert int(gap.max()) <= 1
    assert rel_r <= 1e-6
    return hh, rs


def test_tiny_hhat_bits_and_rstd(rz, gpu):
    b = workloads.tiny()
    _check_against_oracle(rz, gpu, b.x, b.gamma, b.eps, "tiny")


def test_workload_shaped_rows(rz, gpu):
    # 1.5B-shaped rows (H = 1536) with that workload's gamma
    g15 = workloads.qwen15b(with_W=False, with_x=False).gamma
    x, _ = workloads.rows_only(11, 1, 4096, 1536, 151936)
    _check_against_oracle(rz, gpu, x, g15, 1e-6, "1.5B-shaped rows")
    # 30B-head-shaped rows (H = 2048) with outlier rows scaled by 20 before
    # the bf16 rounding, as in that workload (1% here, so 4096 rows hold 41)
    g30 = workloads.a3b30_head(with_W=False, with_x=False).gamma
    x, _ = workloads.rows_only(12, 1, 4096, 2048, 151936)
    rows = np.random.default_rng(7).choice(4096, 41, replace=False)
    xf = workloads.bf16_bits_to_f32(x)
    xf[rows] *= np.float32(20.0)
    x = workloads.f32_to_bf16_bits(xf)
    _check_against_oracle(rz, gpu, x, g30, 1e-6, "30B-head-shaped rows with outliers")
    # 4B-shaped rows (H = 2560) with that workload's gamma
    g4 = workloads.qwen4b_lag64(with_W=False, with_x=False).gamma
    x, _ = workloads.rows_only(17, 1, 2048, 2560, 151936)
    _check_against_oracle(rz, gpu, x, g4, 1e-6, "4B-shaped rows")


@pytest.mark.parametrize("H", [64, 16384])
def test_extreme_hidden_sizes(rz, gpu, H):
    x, _ = workloads.rows_only(13 if H == 64 else 14, 1, 37, H, 1024)
    g = workloads.f32_to_bf16_bits(
        (1.0 + 0.1 * np.random.default_rng(H).standard_normal(H)).astype(np.float32))
    _check_against_oracle(rz, gpu, x, g, 1e-6, f"H={H}")


def test_chunk_boundary_and_row_independence(rz, gpu):
    # two launch chunks (32768 rows each at most): every row against the
    # oracle, and rows around the boundary recomputed alone give equal bits
    T, H = 32768 + 300, 128
    x_bits, _ = workloads.rows_only(15, 1, T, H, 1024)
    g_bits = workloads.tiny().gamma
    hh, rs = _check_against_oracle(rz, gpu, x_bits, g_bits, 1e-6, "two chunks")
    x, g = bf16(x_bits, gpu), bf16(g_bits, gpu)
    for a, n in ((32760, 20), (0, 1), (T - 1, 1), (12345, 7)):
        h1, r1 = rz.rmsnorm(x[a:a + n].contiguous(), g, 1e-6)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(h1), _bits(hh[a:a + n])), (a, n)
        assert np.array_equal(host(r1).view(np.uint32), host(rs[a:a + n]).view(np.uint32)), (a, n)


def test_constant_rows_closed_form(rz, gpu):
    # x = c * 1 gives mean x^2 = c^2, so hhat_k = bf16(gamma_k c / sqrt(c^2 + eps))
    H, eps = 256, 1e-6
    cs = np.array([1.0, -2.25, 0.5, 3.0, 1e-3, -7.5, 96.0, 2.0 ** -20], dtype=np.float32)
    cs = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(cs)).astype(np.float64)
    x_bits = workloads.f32_to_bf16_bits(np.repeat(cs[:, None], H, 1).astype(np.float32))
    g_bits = workloads.f32_to_bf16_bits(
        (1.0 + 0.1 * np.random.default_rng(3).standard_normal(H)).astype(np.float32))
    g64 = workloads.bf16_bits_to_f32(g_bits).astype(np.float64)
    hh, rs = rz.rmsnorm(bf16(x_bits, gpu), bf16(g_bits, gpu), eps)
    torch.cuda.synchronize()
    eps64 = float(np.float32(eps))
    r = 1.0 / np.sqrt(cs * cs + eps64)
    want = _oracle_bits(oracle.bf16_round(g64[None, :] * cs[:, None] * r[:, None]))
    assert np.array_equal(_bits(hh), want)
    assert np.allclose(host(rs).astype(np.float64), r, rtol=1e-7, atol=0)


def test_power_of_two_scale_invariance_at_zero_eps(rz, gpu):
    # with eps = 0, scaling a row by 16 scales mean x^2 by 256 and r by 1/16,
    # all exactly in binary floating point: hhat keeps its bits, rstd is /16
    T, H = 513, 1536
    x_bits, _ = workloads.rows_only(16, 1, T, H, 151936)
    x16 = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x_bits) * np.float32(16.0))
    assert np.array_equal(workloads.bf16_bits_to_f32(x16), 16 * workloads.bf16_bits_to_f32(x_bits))
    g = bf16(workloads.qwen15b(with_W=False, with_x=False).gamma, gpu)
    h1, r1 = rz.rmsnorm(bf16(x_bits, gpu), g, 0.0)
    h2, r2 = rz.rmsnorm(bf16(x16, gpu), g, 0.0)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(h1), _bits(h2))
    assert np.array_equal(host(r1), host(r2) * np.float32(16.0))


def test_logprob_consumes_these_bits(rz, gpu):
    # staged parity, second stage: the oracle's logits and log-softmax fed
    # the GPU's hhat reproduce rz_logprob to the logprob bound
    b = workloads.tiny()
    x, g, W, t = bf16(b.x, gpu), bf16(b.gamma, gpu), bf16(b.W, gpu), i32(b.target, gpu)
    hh, _ = rz.rmsnorm(x, g, b.eps)
    lp, lse = rz.logprob(x, g, W, t, b.eps)
    torch.cuda.synchronize()
    hh64 = oracle.bf16_decode(_bits(hh))
    z = oracle.logits(hh64, oracle.bf16_decode(b.W))
    o_lp, o_lse = oracle.log_softmax_gather(z, b.target)
    d_lp = float(np.max(np.abs(host(lp) - o_lp)))
    d_lse = float(np.max(np.abs(host(lse) - o_lse)))
    say(f"oracle on the GPU's hhat: max |dlogprob| {d_lp:.2e}, max |dlse| {d_lse:.2e}")
    assert d_lp <= 5e-4 and d_lse <= 5e-4
