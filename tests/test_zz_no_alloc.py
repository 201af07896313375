"""The allocation-free entry point, rz_logprob_noalloc, through the C ABI:
the same bits as rz_logprob on two calls in a row, the second smaller (the
built-in scratch keeps the first call's contents), and the size limit."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import bf16, bits32, i32, say

pytestmark = pytest.mark.gpu


def test_noalloc_matches_logprob_on_two_calls(gpu):
    import invariant_logprob_is_amd as rz
    rz.lib()
    H, V = 1536, 151936
    rng = np.random.default_rng(0)
    W = bf16(workloads.f32_to_bf16_bits((0.02 * rng.standard_normal((V, H))).astype(np.float32)),
             gpu)
    g = bf16(workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32)),
             gpu)
    for T, child in ((8000, 3), (900, 5)):          # the second call smaller
        say(f"noalloc T={T} H={H} V={V}")
        xb, tb = workloads.rows_only(7, child, T, H, V)
        x, t = bf16(xb, gpu), i32(tb, gpu)
        lp0, lse0 = rz.logprob(x, g, W, t)
        lp = torch.full((T,), float("nan"), dtype=torch.float32, device=gpu)
        lse = torch.full((T,), float("nan"), dtype=torch.float32, device=gpu)
        rz.logprob_noalloc(x, g, W, t, out=lp, lse_out=lse)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits32(lp), bits32(lp0))
        np.testing.assert_array_equal(bits32(lse), bits32(lse0))
    # one row more than the scratch holds at these shapes: rejected
    T = 8573
    xb, tb = workloads.rows_only(7, 9, T, H, V)
    with pytest.raises(rz.RzError) as ei:
        rz.logprob_noalloc(bf16(xb, gpu), g, W, i32(tb, gpu))
    assert ei.value.status == rz.RZ_EWORKSPACE
