"""Batch invariance at the 1.5B shapes (H=1536, V=151936): a fixed set of 512
rows evaluated alone (single-row decode calls), inside batches of 7, 64, 100,
200, 1024 and 65536 rows at random offsets among filler rows (each batch size
up to 256 rows takes one of the small-batch forwards), inside 2048-row
prefill chunks, and through the forward that stores the logits
(rz_logprob_store) in the 1024- and 65536-row batches.  The bits of logprob and lse must be
identical across all of them: the kernel-mismatch term of the log-ratio
decomposition is then exactly zero for these rows."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import bf16, bits32, i32, say

pytestmark = pytest.mark.gpu


def test_invariance_sweep_15b(gpu):
    import invariant_logprob_is_amd as rz
    sw = workloads.invariance_sweep()
    H, V = sw.H, sw.V
    b = workloads.qwen15b(with_x=False)      # gamma and W of the 1.5B-shaped workload
    g, W = bf16(b.gamma, gpu), bf16(b.W, gpu)
    ws = torch.empty(rz.workspace_bytes(65536, H, V), dtype=torch.uint8, device=gpu)
    n = sw.fixed_x.shape[0]
    seen = {}
    for label, plan in sw.batches.items():
        lp_bits = np.zeros(n, np.uint32)
        lse_bits = np.zeros(n, np.uint32)
        for ids, pos, B in plan:
            bx, bt = workloads.compose_batch(sw, ids, pos, B)
            lp, lse = rz.logprob(bf16(bx, gpu), g, W, i32(bt, gpu), b.eps, workspace=ws)
            lp_bits[ids] = bits32(lp)[pos]
            lse_bits[ids] = bits32(lse)[pos]
        say(f"  {label}: {len(plan)} calls")
        seen[label] = (lp_bits, lse_bits)
    # the forward with the stored logits (rz_logprob_store), in the 1024- and
    # 65536-row batches
    for B in (1024, 65536):
        lp_bits = np.zeros(n, np.uint32)
        lse_bits = np.zeros(n, np.uint32)
        for ids, pos, BB in sw.batches[f"batch{B}"]:
            bx, bt = workloads.compose_batch(sw, ids, pos, BB)
            lp, lse, lg = rz.logprob_store(bf16(bx, gpu), g, W, i32(bt, gpu), b.eps, workspace=ws)
            lp_bits[ids] = bits32(lp)[pos]
            lse_bits[ids] = bits32(lse)[pos]
            del lg
        say(f"  store{B}: {len(sw.batches[f'batch{B}'])} calls")
        seen[f"store{B}"] = (lp_bits, lse_bits)
    ref_label = "batch1"
    for label, (a, c) in seen.items():
        np.testing.assert_array_equal(a, seen[ref_label][0], err_msg=f"logprob bits {label}")
        np.testing.assert_array_equal(c, seen[ref_label][1], err_msg=f"lse bits {label}")
    lp = seen[ref_label][0].view(np.float32)
    assert np.all(np.isfinite(lp)) and np.all(lp <= 0)


# The forward's raster group depends on H (8 vocabulary tiles up to
# H = 2048, 4 at 2560, 2 beyond) and is used once a batch has more than 32
# token tiles (8192 rows).  It decides only which workgroup computes which
# tile, so a row's bits must not depend on it: rows alone and inside a
# 9000-row batch, at the hidden sizes that select each group.
@pytest.mark.parametrize("H", [1536, 2560, 3072])
def test_invariance_across_raster_groups(gpu, H):
    import invariant_logprob_is_amd as rz
    V, n, B = 1000, 40, 9000
    say(f"raster-group invariance H={H}: {n} rows alone and inside a {B}-row batch")
    xb, tb = workloads.rows_only(18, 1, n, H, V)
    fx, ft = workloads.rows_only(19, 1, B, H, V)
    rng = np.random.default_rng(H)
    g = bf16(workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32)), gpu)
    W = bf16(workloads.f32_to_bf16_bits((0.02 * rng.standard_normal((V, H))).astype(np.float32)), gpu)
    alone = [rz.logprob(bf16(xb[i:i + 1], gpu), g, W, i32(tb[i:i + 1], gpu)) for i in range(n)]
    ref_lp = np.concatenate([bits32(a[0]) for a in alone])
    ref_lse = np.concatenate([bits32(a[1]) for a in alone])
    pos = np.sort(rng.choice(B, n, replace=False))
    bx, bt = fx.copy(), ft.copy()
    bx[pos], bt[pos] = xb, tb
    lp, lse = rz.logprob(bf16(bx, gpu), g, W, i32(bt, gpu))
    np.testing.assert_array_equal(bits32(lp)[pos], ref_lp)
    np.testing.assert_array_equal(bits32(lse)[pos], ref_lse)
