"""The learner step, the forward, and the stored-logits forward with the
weight-gradient backward, captured in a HIP graph (torch.cuda.graph around
the C-ABI calls) and replayed: the library launches only kernels on the caller's
stream (no memset, no allocation, no host sync), so every replay must give
the eager call's bits, with other eager work and synchronizations between the
replays, and must follow inputs changed in place."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import bf16, bits32, f32, host, i32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rz():
    import invariant_logprob_is_amd as m
    m.lib()
    return m


def _case(seed, T, H, V, R, G):
    rng = np.random.default_rng(seed)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    g = workloads.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    W = workloads.f32_to_bf16_bits((0.05 * rng.standard_normal((V, H))).astype(np.float32))
    t = rng.integers(0, V, T).astype(np.int32)
    cuts = np.sort(rng.choice(np.arange(1, T), R - 1, replace=False))
    ro = np.concatenate([[0], cuts, [T]]).astype(np.int64)
    go = np.linspace(0, R, G + 1).astype(np.int64)
    reward = rng.integers(0, 2, R).astype(np.float32)
    return x, g, W, t, ro, go, reward


def _bits(t):
    a = host(t)
    return a.view(np.uint64) if a.dtype == np.float64 else a.view(np.uint32)


def _same(a, b):
    return all(np.array_equal(_bits(a[k]), _bits(b[k])) for k in a)


@pytest.mark.parametrize("weight_grads", [False, True])
def test_learner_step_replays_from_a_graph(rz, gpu, weight_grads):
    T, H, V, R, G = 40000, 128, 1000, 16, 4     # two chunks, the second ragged
    say(f"graph replay of learner_step T={T} H={H} V={V} weight_grads={weight_grads}")
    xb, gb, Wb, tb, ro, go, rw = _case(11, T, H, V, R, G)
    x, g, W, t = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu)
    ro_d, go_d = torch.from_numpy(ro).to(gpu), torch.from_numpy(go).to(gpu)
    rw_d = f32(rw, gpu)
    lp0, _ = rz.logprob(x, g, W, t)
    mu = (lp0 + 0.05 * torch.randn(T, device=gpu, generator=torch.Generator(gpu).manual_seed(3))
          ).contiguous()
    need = (rz.workspace_bytes_grads if weight_grads else rz.workspace_bytes)(T, H, V)
    ws_e = torch.empty(need, dtype=torch.uint8, device=gpu)
    ws_g = torch.empty(need, dtype=torch.uint8, device=gpu)

    def eager():
        o = rz.learner_step(x, g, W, t, mu, ro_d, go_d, rw_d, workspace=ws_e,
                            weight_grads=weight_grads)
        torch.cuda.synchronize()
        return {k: v.clone() for k, v in o.items()}

    ref = eager()
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rz.learner_step(x, g, W, t, mu, ro_d, go_d, rw_d, workspace=ws_g, out=out,
                        weight_grads=weight_grads)
    torch.cuda.synchronize()
    for rep in range(3):
        for v in out.values():
            v.fill_(float("nan"))
        ws_g.fill_(0xA5)                        # stale workspace between replays
        rz.logprob(x, g, W, t, workspace=ws_e)  # other eager library work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert _same(out, ref), f"replay {rep}"
    # inputs changed in place: the replay follows them
    x2b, _, _, t2b, _, _, _ = _case(12, T, H, V, R, G)
    x.copy_(bf16(x2b, gpu))
    t.copy_(i32(t2b, gpu))
    ref2 = eager()
    assert not np.array_equal(_bits(ref2["logprob"]), _bits(ref["logprob"]))
    graph.replay()
    torch.cuda.synchronize()
    assert _same(out, ref2)
    assert np.isfinite(host(out["dhidden"])).all()


def test_logprob_replays_from_a_graph(rz, gpu):
    T, H, V = 777, 256, 5000
    say(f"graph replay of logprob T={T} H={H} V={V}")
    xb, gb, Wb, tb, _, _, _ = _case(5, T, H, V, 2, 1)
    x, g, W, t = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu)
    ref_lp, ref_lse = rz.logprob(x, g, W, t)
    torch.cuda.synchronize()
    ws = torch.empty(rz.workspace_bytes(T, H, V), dtype=torch.uint8, device=gpu)
    lp = torch.empty(T, dtype=torch.float32, device=gpu)
    lse = torch.empty(T, dtype=torch.float32, device=gpu)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rz.logprob(x, g, W, t, workspace=ws, out=lp, lse_out=lse)
    for rep in range(3):
        lp.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits32(lp), bits32(ref_lp)), f"replay {rep}"
        assert np.array_equal(bits32(lse), bits32(ref_lse)), f"replay {rep}"


def test_stored_pair_and_weight_grads_replay_from_a_graph(rz, gpu):
    T, H, V = 5000, 128, 1000
    say(f"graph replay of logprob_store + backward_grads T={T} H={H} V={V}")
    xb, gb, Wb, tb, _, _, _ = _case(7, T, H, V, 2, 1)
    x, g, W, t = bf16(xb, gpu), bf16(gb, gpu), bf16(Wb, gpu), i32(tb, gpu)
    coef = (0.01 * torch.randn(T, device=gpu, generator=torch.Generator(gpu).manual_seed(8))
            ).contiguous()
    lp_e, lse_e, lg_e = rz.logprob_store(x, g, W, t)
    ref = rz.backward_grads(x, g, W, t, lse_e, coef, logits=lg_e)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}
    ref_lp = lp_e.clone()
    ws = torch.empty(rz.workspace_bytes_grads(T, H, V), dtype=torch.uint8, device=gpu)
    lg = torch.empty(rz.logits_bytes(T, H, V), dtype=torch.uint8, device=gpu)
    lp = torch.empty(T, dtype=torch.float32, device=gpu)
    lse = torch.empty(T, dtype=torch.float32, device=gpu)
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rz.logprob_store(x, g, W, t, logits=lg, workspace=ws, out=lp, lse_out=lse)
        rz.backward_grads(x, g, W, t, lse, coef, logits=lg, workspace=ws, out=out)
    for rep in range(3):
        for v in list(out.values()) + [lp]:
            v.fill_(float("nan"))
        lg.fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits32(lp), bits32(ref_lp)), f"replay {rep}"
        for k in ref:
            assert np.array_equal(bits32(out[k]), bits32(ref[k])), f"replay {rep} {k}"
