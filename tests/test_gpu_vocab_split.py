"""Vocabulary splits through the C ABI.

The partials of any whole number of consecutive splits (rz_logprob_shard,
what one device of a vocabulary-parallel head computes on its share of W)
merge (rz_logprob_merge) into logprob and lse bit for bit equal to
rz_logprob's.  The vocabulary is spread over 1, 2, 4 or 8 equal shares; the
shares run one after another on this one GPU, each given only its rows of W.
A split's records must not depend on which share computed it, and the merged
logprob meets the oracle's 5e-4 bound like rz_logprob's."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16, bits32, host, i32, say

pytestmark = pytest.mark.gpu

SHARE_COUNTS = (1, 2, 4, 8)


@pytest.fixture(scope="module")
def rz():
    import invariant_logprob_is_amd as m
    m.lib()
    return m


def _shares(rz, d):
    k = rz.VOCAB_SPLITS // d
    return [(r * k, (r + 1) * k) for r in range(d)]


def _sharded(rz, x, g, W, t, V, d, eps, ws):
    recs = []
    for s0, s1 in _shares(rz, d):
        a, b = rz.vocab_split_begin(V, s0), rz.vocab_split_begin(V, s1)
        recs.append(rz.logprob_shard(x, g, W[a:b], t, V, s0, s1, eps, workspace=ws))
    parts = torch.cat(recs, 0)
    lp, lse = rz.logprob_merge(parts, t, V)
    return parts, lp, lse


def _case(seed, T, H, V):
    rng = np.random.default_rng(seed)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    g = workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    W = workloads.f32_to_bf16_bits((0.5 * rng.standard_normal((V, H))).astype(np.float32))
    t = rng.integers(0, V, T).astype(np.int32)
    return x, g, W, t


def _check_records(rz, recs, t, V):
    """Record semantics: m integer-valued or -inf, empty splits empty, the
    target logit in exactly the split that holds the target row."""
    starts = [rz.vocab_split_begin(V, s) for s in range(rz.VOCAB_SPLITS + 1)]
    m = recs["m"]
    assert np.all((m == np.floor(m)) | (m == -np.inf))
    assert np.all(recs["reserved"] == 0)
    for s in range(rz.VOCAB_SPLITS):
        if starts[s + 1] == starts[s]:
            assert np.all(recs["s"][s] == 0) and np.all(m[s] == -np.inf)
            assert np.all(recs["max_logit"][s] == -np.inf)
        else:
            assert np.all(recs["s"][s] >= 0.5) and np.all(np.isfinite(m[s]))
        owner = (t >= starts[s]) & (t < starts[s + 1])
        assert np.all(recs["z_target"][s][~owner] == 0)
        assert np.all(recs["z_target"][s][owner] <= recs["max_logit"][s][owner])


@pytest.mark.parametrize("T,H,V", [(300, 128, 3000), (257, 192, 513), (70, 64, 65),
                                   (1, 64, 2049), (600, 128, 20000),
                                   (33000, 64, 1300)])     # two chunks, ragged last one
def test_shards_merge_to_logprob_bits(rz, gpu, T, H, V):
    say(f"vocab splits T={T} H={H} V={V}")
    xb, gb, Wb, tb = _case(T * 7 + V, T, H, V)
    x, g, W, t = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu)
    ws = torch.empty(rz.workspace_bytes(T, H, V), dtype=torch.uint8, device=gpu)
    ref_lp, ref_lse = rz.logprob(x, g, W, t, 1e-6, workspace=ws)
    parts1 = None
    for d in SHARE_COUNTS:
        parts, lp, lse = _sharded(rz, x, g, W, t, V, d, 1e-6, ws)
        np.testing.assert_array_equal(bits32(lp), bits32(ref_lp), err_msg=f"logprob, {d} shares")
        np.testing.assert_array_equal(bits32(lse), bits32(ref_lse), err_msg=f"lse, {d} shares")
        if parts1 is None:
            parts1 = host(parts)
        else:
            np.testing.assert_array_equal(host(parts).view(np.uint64), parts1.view(np.uint64),
                                          err_msg=f"records, {d} shares")
    _check_records(rz, rz.split_records(torch.from_numpy(parts1)), tb, V)
    if T > 4096:                # the oracle on a sample of rows
        rows = np.r_[0:64, 32700:32830, T - 64:T]
        xb, tb = xb[rows], tb[rows]
        ref_lp = ref_lp[torch.from_numpy(rows).to(gpu)]
    olp, _ = oracle.logprob(xb, gb, 1e-6, Wb, tb)
    err = float(np.abs(host(ref_lp).astype(np.float64) - olp).max())
    say(f"  max |dlogprob| vs oracle {err:.2e}")
    assert err <= 5e-4


def test_shards_at_15b_shapes(rz, gpu):
    b = workloads.qwen15b(with_x=False)
    H, V = b.W.shape[1], b.W.shape[0]
    xb, tb = workloads.rows_only(5, 1, 4100, H, V)   # rows of their own seed stream
    x, g, W, t = bf16(xb, gpu), bf16(b.gamma, gpu), bf16(b.W, gpu), i32(tb, gpu)
    ws = torch.empty(rz.workspace_bytes(4100, H, V), dtype=torch.uint8, device=gpu)
    ref_lp, ref_lse = rz.logprob(x, g, W, t, b.eps, workspace=ws)
    for d in SHARE_COUNTS:
        say(f"1.5B shapes, {d} shares")
        parts, lp, lse = _sharded(rz, x, g, W, t, V, d, b.eps, ws)
        np.testing.assert_array_equal(bits32(lp), bits32(ref_lp), err_msg=f"logprob, {d} shares")
        np.testing.assert_array_equal(bits32(lse), bits32(ref_lse), err_msg=f"lse, {d} shares")
    recs = rz.split_records(parts)
    _check_records(rz, recs, tb, V)
    # every split of the 1.5B vocabulary holds 74 or 75 tiles
    starts = np.array([rz.vocab_split_begin(V, s) for s in range(9)])
    assert set(np.diff(starts)) <= {74 * 256, 75 * 256, V - starts[7]}
    # the merge of the records, evaluated on the host in the documented
    # order, reproduces lse to float rounding
    m = recs["m"].astype(np.float64)
    mm = m.max(0)
    S = np.zeros(4100)
    for s in range(8):
        S += np.ldexp(recs["s"][s], (m[s] - mm).astype(np.int64))
    lse_host = np.maximum(mm * math.log(2) + np.log(S), recs["max_logit"].max(0))
    assert np.abs(lse_host - host(ref_lse)).max() <= 1e-5 * np.abs(lse_host).max()


def test_out_of_range_targets_merge_to_nan(rz, gpu):
    T, H, V = 200, 128, 1500
    xb, gb, Wb, tb = _case(3, T, H, V)
    tb[5], tb[77] = -1, V
    x, g, W, t = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu)
    ws = torch.empty(rz.workspace_bytes(T, H, V), dtype=torch.uint8, device=gpu)
    ref_lp, ref_lse = rz.logprob(x, g, W, t, 1e-6, workspace=ws)
    for d in (1, 4):
        parts, lp, lse = _sharded(rz, x, g, W, t, V, d, 1e-6, ws)
        a = host(lp)
        assert np.isnan(a[5]) and np.isnan(a[77]) and np.count_nonzero(np.isnan(a)) == 2
        np.testing.assert_array_equal(bits32(lp), bits32(ref_lp))
        np.testing.assert_array_equal(bits32(lse), bits32(ref_lse))
        recs = rz.split_records(parts)
        assert np.all(recs["z_target"][:, 5] == 0) and np.all(recs["z_target"][:, 77] == 0)
