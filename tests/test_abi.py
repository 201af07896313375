"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import invariant_logprob_is_amd as rz

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rz.h")

pytestmark = pytest.mark.skipif(not os.path.exists(rz.LIB_PATH), reason="librz.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rz_[a-z0-9_]+)\s*\(", src)))


def _gpu_present():
    if os.path.exists("/dev/kfd"):
        return True
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


FAKE = 1 << 20  # a 256-byte aligned non-null address, never dereferenced


def test_exports_every_declared_symbol():
    L = rz.lib()
    names = _declared()
    assert set(names) == set(rz.SYMBOLS), "binding table and header disagree"
    for n in names:
        assert hasattr(L, n), n


def test_exports_are_visible_with_dlsym():
    raw = ctypes.CDLL(rz.LIB_PATH)
    for n in _declared():
        assert ctypes.cast(getattr(raw, n), ctypes.c_void_p).value


def test_internal_host_functions_are_not_exported():
    # the library is built with hidden visibility: the C entry points of
    # include/rz.h are exported, the C++ launchers and helpers behind them
    # are not (HIP keeps its kernel stubs visible, which is harmless)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", rz.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    names = [line.split()[-1] for line in out.splitlines() if line.strip()]
    c_names = [n for n in names if n.startswith("rz_")]
    assert set(c_names) == set(_declared())
    for n in names:
        assert "launch_" not in n and "profile_record" not in n and "ws_layout" not in n, n


def test_version_and_status_strings():
    assert rz.version() == (0 << 16) | (1 << 8)
    L = rz.lib()
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported shape"),
                       (3, b"no HIP device"), (4, b"HIP runtime error"), (5, b"workspace too small")]:
        assert L.rz_status_string(code) == text
    assert L.rz_status_string(99) == b"unknown status"


def test_workspace_bytes():
    assert rz.workspace_bytes(0, 128, 1024) == 0
    assert rz.workspace_bytes(10, 0, 1024) == 0
    small = rz.workspace_bytes(300, 128, 1024)
    big = rz.workspace_bytes(300000, 1536, 151936)
    assert 0 < small < big
    assert small % 256 == 0 and big % 256 == 0
    # the forward needs at least hhat + partials; the backward at least W^T + P chunk
    assert big >= 1536 * 151936 * 2 + 32768 * 151936 * 2


def _logprob(**kw):
    a = dict(x=FAKE, gamma=FAKE, eps=1e-6, W=FAKE, target=FAKE, T=300, H=128, V=1024,
             logprob=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return rz.lib().rz_logprob(a["x"], a["gamma"], a["eps"], a["W"], a["target"], a["T"], a["H"],
                               a["V"], a["logprob"], a["lse"], a["ws"], a["wsb"], a["stream"])


def _backward(**kw):
    a = dict(x=FAKE, gamma=FAKE, eps=1e-6, W=FAKE, target=FAKE, lse=FAKE, coef=FAKE, T=300,
             H=128, V=1024, dh=FAKE, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return rz.lib().rz_backward(a["x"], a["gamma"], a["eps"], a["W"], a["target"], a["lse"],
                                a["coef"], a["T"], a["H"], a["V"], a["dh"], a["ws"], a["wsb"],
                                a["stream"])


def _logprob_store(**kw):
    a = dict(x=FAKE, gamma=FAKE, eps=1e-6, W=FAKE, target=FAKE, T=300, H=128, V=1024,
             logprob=FAKE, lse=FAKE, logits=FAKE, lgb=1 << 40, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return rz.lib().rz_logprob_store(a["x"], a["gamma"], a["eps"], a["W"], a["target"], a["T"],
                                     a["H"], a["V"], a["logprob"], a["lse"], a["logits"], a["lgb"],
                                     a["ws"], a["wsb"], a["stream"])


def _backward_stored(**kw):
    a = dict(x=FAKE, gamma=FAKE, eps=1e-6, W=FAKE, target=FAKE, lse=FAKE, coef=FAKE, T=300,
             H=128, V=1024, logits=FAKE, lgb=1 << 40, dh=FAKE, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return rz.lib().rz_backward_stored(a["x"], a["gamma"], a["eps"], a["W"], a["target"],
                                       a["lse"], a["coef"], a["T"], a["H"], a["V"], a["logits"],
                                       a["lgb"], a["dh"], a["ws"], a["wsb"], a["stream"])


def _backward_grads(**kw):
    a = dict(x=FAKE, gamma=FAKE, eps=1e-6, W=FAKE, target=FAKE, lse=FAKE, coef=FAKE, T=300,
             H=128, V=1024, logits=None, lgb=0, dh=FAKE, dW=FAKE, dg=FAKE, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(kw)
    return rz.lib().rz_backward_grads(a["x"], a["gamma"], a["eps"], a["W"], a["target"],
                                      a["lse"], a["coef"], a["T"], a["H"], a["V"], a["logits"],
                                      a["lgb"], a["dh"], a["dW"], a["dg"], a["ws"], a["wsb"],
                                      a["stream"])


def _rmsnorm(**kw):
    a = dict(x=FAKE, gamma=FAKE, eps=1e-6, T=300, H=128, hhat=FAKE, rstd=FAKE, stream=None)
    a.update(kw)
    return rz.lib().rz_rmsnorm(a["x"], a["gamma"], a["eps"], a["T"], a["H"], a["hhat"],
                               a["rstd"], a["stream"])


def test_rmsnorm_argument_validation():
    for k in ("x", "gamma", "hhat"):
        assert _rmsnorm(**{k: None}) == rz.RZ_EINVAL, k
    for k in ("x", "gamma", "hhat"):
        assert _rmsnorm(**{k: FAKE + 8}) == rz.RZ_EINVAL, k   # 16-byte alignment
    assert _rmsnorm(rstd=FAKE + 2) == rz.RZ_EINVAL
    assert _rmsnorm(T=0) == rz.RZ_EINVAL
    assert _rmsnorm(T=-1) == rz.RZ_EINVAL
    assert _rmsnorm(H=0) == rz.RZ_EINVAL
    assert _rmsnorm(eps=-1e-6) == rz.RZ_EINVAL
    assert _rmsnorm(eps=float("nan")) == rz.RZ_EINVAL
    assert _rmsnorm(H=96) == rz.RZ_EUNSUPPORTED
    assert _rmsnorm(H=16384 + 64) == rz.RZ_EUNSUPPORTED


@pytest.mark.parametrize("fn", [_logprob, _backward, _logprob_store, _backward_stored,
                                _backward_grads])
def test_head_argument_validation(fn):
    for k in ("x", "gamma", "W", "target", "ws"):
        assert fn(**{k: None}) == rz.RZ_EINVAL, k
    assert fn(x=FAKE + 8) == rz.RZ_EINVAL          # bf16 rows need 16-byte alignment
    assert fn(target=FAKE + 2) == rz.RZ_EINVAL
    assert fn(ws=FAKE + 64) == rz.RZ_EINVAL        # workspace needs 256-byte alignment
    assert fn(T=0) == rz.RZ_EINVAL
    assert fn(T=-5) == rz.RZ_EINVAL
    assert fn(H=0) == rz.RZ_EINVAL
    assert fn(V=0) == rz.RZ_EINVAL
    assert fn(eps=-1.0) == rz.RZ_EINVAL
    assert fn(eps=float("nan")) == rz.RZ_EINVAL
    assert fn(H=100) == rz.RZ_EUNSUPPORTED         # not a multiple of 64
    assert fn(H=16384 + 64) == rz.RZ_EUNSUPPORTED
    assert fn(V=4000001) == rz.RZ_EUNSUPPORTED
    assert fn(wsb=rz.workspace_bytes(300, 128, 1024) - 1) == rz.RZ_EWORKSPACE


def test_backward_needs_lse_coef_dh():
    for k in ("lse", "coef", "dh"):
        assert _backward(**{k: None}) == rz.RZ_EINVAL, k
        assert _backward_stored(**{k: None}) == rz.RZ_EINVAL, k


def test_logits_bytes():
    assert rz.logits_bytes(0, 128, 1024) == 0
    assert rz.logits_bytes(10, 0, 1024) == 0
    assert rz.logits_bytes(10, 128, 0) == 0
    # one chunk: the e values (rows padded for the shift table, vocabulary to
    # whole tiles) in bf16, one max per row and vocabulary tile, one target
    # logit per row, each region 256-byte aligned
    b = rz.logits_bytes(300, 128, 1024)
    assert b % 256 == 0
    assert 300 * 1024 * 2 <= b < 2 * 300 * 1024 * 2
    # independent of H; chunks of 32,768 rows each take the first chunk's stride
    assert rz.logits_bytes(300, 4096, 1024) == b
    one = rz.logits_bytes(32768, 128, 1024)
    assert rz.logits_bytes(32769, 128, 1024) == 2 * one
    assert rz.logits_bytes(65536, 128, 1024) == 2 * one
    # the 1.5B-shaped head keeps about 2 bytes per logit
    big = rz.logits_bytes(8192, 1536, 151936)
    assert 8192 * 151936 * 2 <= big < 1.05 * 8192 * 151936 * 2


def test_stored_logits_argument_validation():
    for k in ("logits", "logprob"):
        assert _logprob_store(**{k: None}) == rz.RZ_EINVAL, k
    assert _backward_stored(logits=None) == rz.RZ_EINVAL
    # the stored logits need 256-byte alignment and the full size
    assert _logprob_store(logits=FAKE + 16) == rz.RZ_EINVAL
    assert _backward_stored(logits=FAKE + 16) == rz.RZ_EINVAL
    need = rz.logits_bytes(300, 128, 1024)
    assert _logprob_store(lgb=need - 1) == rz.RZ_EWORKSPACE
    assert _backward_stored(lgb=need - 1) == rz.RZ_EWORKSPACE
    assert _logprob_store(lse=FAKE + 2) == rz.RZ_EINVAL


def test_backward_grads_argument_validation():
    for k in ("lse", "coef", "dh", "dW", "dg"):
        assert _backward_grads(**{k: None}) == rz.RZ_EINVAL, k
    assert _backward_grads(dW=FAKE + 8) == rz.RZ_EINVAL
    assert _backward_grads(dg=FAKE + 2) == rz.RZ_EINVAL
    # the weight gradients need the larger workspace
    small, grads = rz.workspace_bytes(300, 128, 1024), rz.workspace_bytes_grads(300, 128, 1024)
    assert small < grads
    assert _backward_grads(wsb=grads - 1) == rz.RZ_EWORKSPACE
    # stored logits: aligned, and of the full size
    need = rz.logits_bytes(300, 128, 1024)
    assert _backward_grads(logits=FAKE + 16, lgb=need) == rz.RZ_EINVAL
    assert _backward_grads(logits=FAKE, lgb=need - 1) == rz.RZ_EWORKSPACE


def _is_loss(**kw):
    a = dict(lp=FAKE, mu=FAKE, T=300, ro=FAKE, R=16, go=FAKE, G=4, reward=FAKE, loss=FAKE,
             coef=FAKE, adv=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return rz.lib().rz_is_loss(a["lp"], a["mu"], a["T"], a["ro"], a["R"], a["go"], a["G"],
                               a["reward"], a["loss"], a["coef"], a["adv"], a["ws"], a["wsb"],
                               a["stream"])


def test_is_loss_argument_validation():
    for k in ("lp", "mu", "ro", "go", "reward", "loss", "ws"):
        assert _is_loss(**{k: None}) == rz.RZ_EINVAL, k
    assert _is_loss(T=0) == rz.RZ_EINVAL
    assert _is_loss(R=0) == rz.RZ_EINVAL
    assert _is_loss(G=0) == rz.RZ_EINVAL
    assert _is_loss(R=301) == rz.RZ_EINVAL         # more responses than tokens
    assert _is_loss(G=17) == rz.RZ_EINVAL          # more groups than responses
    assert _is_loss(ro=FAKE + 4) == rz.RZ_EINVAL   # int64 offsets need 8-byte alignment
    assert _is_loss(wsb=16) == rz.RZ_EWORKSPACE


def test_d3_argument_validation():
    L = rz.lib()
    assert L.rz_d3(None, FAKE, 10, FAKE, FAKE, 1 << 20, None) == rz.RZ_EINVAL
    assert L.rz_d3(FAKE, FAKE, 0, FAKE, FAKE, 1 << 20, None) == rz.RZ_EINVAL
    assert L.rz_d3(FAKE, FAKE, 10, FAKE + 4, FAKE, 1 << 20, None) == rz.RZ_EINVAL
    assert L.rz_d3(FAKE, FAKE, 10, FAKE, FAKE, 8, None) == rz.RZ_EWORKSPACE


def test_kl_argument_validation():
    L = rz.lib()
    assert L.rz_kl(None, FAKE, 10, FAKE, FAKE, 1 << 20, None) == rz.RZ_EINVAL
    assert L.rz_kl(FAKE, None, 10, FAKE, FAKE, 1 << 20, None) == rz.RZ_EINVAL
    assert L.rz_kl(FAKE, FAKE, 10, None, FAKE, 1 << 20, None) == rz.RZ_EINVAL
    assert L.rz_kl(FAKE, FAKE, 0, FAKE, FAKE, 1 << 20, None) == rz.RZ_EINVAL
    assert L.rz_kl(FAKE, FAKE, 10, FAKE + 4, FAKE, 1 << 20, None) == rz.RZ_EINVAL
    assert L.rz_kl(FAKE, FAKE, 10, FAKE, FAKE, 8, None) == rz.RZ_EWORKSPACE


def _dec(**kw):
    a = dict(xn=FAKE, gn=FAKE, Wn=FAKE, xo=FAKE, go=FAKE, Wo=FAKE, eps=1e-6, target=FAKE,
             mu=FAKE + 4096, T=300, H=128, V=1024, lag=FAKE + 8192, mis=FAKE + 16384,
             summ=FAKE, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return rz.lib().rz_decompose(a["xn"], a["gn"], a["Wn"], a["xo"], a["go"], a["Wo"], a["eps"],
                                 a["target"], a["mu"], a["T"], a["H"], a["V"], a["lag"],
                                 a["mis"], a["summ"], a["ws"], a["wsb"], a["stream"])


def test_decompose_argument_validation():
    for k in ("xn", "gn", "Wn", "xo", "go", "Wo", "target", "mu", "lag", "mis", "summ", "ws"):
        assert _dec(**{k: None}) == rz.RZ_EINVAL, k
    assert _dec(xo=FAKE + 8) == rz.RZ_EINVAL
    assert _dec(summ=FAKE + 4) == rz.RZ_EINVAL
    assert _dec(mis=FAKE + 8192) == rz.RZ_EINVAL      # lag and mismatch must differ
    assert _dec(mu=FAKE + 8192) == rz.RZ_EINVAL       # mu may not alias an output
    assert _dec(T=0) == rz.RZ_EINVAL
    assert _dec(eps=-1.0) == rz.RZ_EINVAL
    assert _dec(H=96) == rz.RZ_EUNSUPPORTED
    assert _dec(wsb=rz.workspace_bytes(300, 128, 1024) - 1) == rz.RZ_EWORKSPACE


def _step(**kw):
    a = dict(x=FAKE, gamma=FAKE, eps=1e-6, W=FAKE, target=FAKE, mu=FAKE, T=300, H=128, V=1024,
             ro=FAKE, R=16, go=FAKE, G=4, reward=FAKE, lp=FAKE, lse=FAKE, loss=FAKE, d3=FAKE,
             kl=FAKE, coef=FAKE, dh=FAKE, dW=None, dg=None, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return rz.lib().rz_learner_step(a["x"], a["gamma"], a["eps"], a["W"], a["target"], a["mu"],
                                    a["T"], a["H"], a["V"], a["ro"], a["R"], a["go"], a["G"],
                                    a["reward"], a["lp"], a["lse"], a["loss"], a["d3"], a["kl"],
                                    a["coef"], a["dh"], a["dW"], a["dg"], a["ws"], a["wsb"],
                                    a["stream"])


def test_learner_step_argument_validation():
    for k in ("x", "gamma", "W", "target", "mu", "ro", "go", "reward", "lp", "loss", "d3", "dh", "ws"):
        assert _step(**{k: None}) == rz.RZ_EINVAL, k
    assert _step(x=FAKE + 8) == rz.RZ_EINVAL
    assert _step(dh=FAKE + 4) == rz.RZ_EINVAL
    assert _step(kl=FAKE + 4) == rz.RZ_EINVAL      # fp64 output needs 8-byte alignment
    assert _step(dW=FAKE) == rz.RZ_EINVAL          # dW and dgamma come together
    assert _step(dg=FAKE) == rz.RZ_EINVAL
    assert _step(dW=FAKE, dg=FAKE + 2) == rz.RZ_EINVAL
    # the weight gradients need the larger workspace
    assert rz.workspace_bytes_grads(300, 128, 1024) > rz.workspace_bytes(300, 128, 1024)
    assert _step(dW=FAKE, dg=FAKE, wsb=rz.workspace_bytes(300, 128, 1024)) == rz.RZ_EWORKSPACE
    assert rz.workspace_bytes_grads(0, 128, 1024) == 0
    assert _step(ro=FAKE + 4) == rz.RZ_EINVAL
    assert _step(T=0) == rz.RZ_EINVAL
    assert _step(R=0) == rz.RZ_EINVAL
    assert _step(G=0) == rz.RZ_EINVAL
    assert _step(R=301) == rz.RZ_EINVAL
    assert _step(G=17) == rz.RZ_EINVAL
    assert _step(eps=-1.0) == rz.RZ_EINVAL
    assert _step(H=96) == rz.RZ_EUNSUPPORTED
    assert _step(wsb=rz.workspace_bytes(300, 128, 1024) - 1) == rz.RZ_EWORKSPACE


def test_vocab_split_boundaries():
    # split s starts at tile floor(s * n / 8), n = ceil(V / 256), clipped to V
    L = rz.lib()
    for V in (1, 65, 255, 256, 257, 513, 3000, 151936, 4000000):
        n = -(-V // 256)
        want = [min(n * s // 8 * 256, V) for s in range(9)]
        assert [L.rz_vocab_split_begin(V, s) for s in range(9)] == want
        assert want[0] == 0 and want[-1] == V and want == sorted(want)
    assert L.rz_vocab_split_begin(151936, 1) == 74 * 256
    assert L.rz_vocab_split_begin(0, 0) == -1
    assert L.rz_vocab_split_begin(4000001, 0) == -1
    assert L.rz_vocab_split_begin(100, -1) == -1
    assert L.rz_vocab_split_begin(100, 9) == -1


def _shard(**kw):
    a = dict(x=FAKE, g=FAKE, eps=1e-6, W=FAKE, target=FAKE, T=300, H=128, V=1024, s0=0, s1=8,
             parts=FAKE, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return rz.lib().rz_logprob_shard(a["x"], a["g"], a["eps"], a["W"], a["target"], a["T"],
                                     a["H"], a["V"], a["s0"], a["s1"], a["parts"], a["ws"],
                                     a["wsb"], a["stream"])


def test_shard_and_merge_argument_validation():
    for k in ("x", "g", "W", "target", "parts", "ws"):
        assert _shard(**{k: None}) == rz.RZ_EINVAL, k
    assert _shard(parts=FAKE + 4) == rz.RZ_EINVAL          # records are 8-byte aligned
    assert _shard(W=FAKE + 8) == rz.RZ_EINVAL
    assert _shard(eps=-1.0) == rz.RZ_EINVAL
    for s0, s1 in ((0, 0), (3, 2), (-1, 4), (0, 9), (8, 8)):
        assert _shard(s0=s0, s1=s1) == rz.RZ_EINVAL, (s0, s1)
    assert _shard(T=0) == rz.RZ_EINVAL
    assert _shard(H=100) == rz.RZ_EUNSUPPORTED
    assert _shard(wsb=rz.workspace_bytes(300, 128, 1024) - 1) == rz.RZ_EWORKSPACE
    L = rz.lib()
    assert L.rz_logprob_merge(None, FAKE, 10, 100, FAKE, FAKE, None) == rz.RZ_EINVAL
    assert L.rz_logprob_merge(FAKE, None, 10, 100, FAKE, FAKE, None) == rz.RZ_EINVAL
    assert L.rz_logprob_merge(FAKE, FAKE, 10, 100, None, FAKE, None) == rz.RZ_EINVAL
    assert L.rz_logprob_merge(FAKE + 4, FAKE, 10, 100, FAKE, FAKE, None) == rz.RZ_EINVAL
    assert L.rz_logprob_merge(FAKE, FAKE, 0, 100, FAKE, FAKE, None) == rz.RZ_EINVAL
    assert L.rz_logprob_merge(FAKE, FAKE, 10, 0, FAKE, FAKE, None) == rz.RZ_EINVAL
    assert L.rz_logprob_merge(FAKE, FAKE, 10, 4000001, FAKE, FAKE, None) == rz.RZ_EINVAL


def test_noalloc_argument_validation():
    f = rz.lib().rz_logprob_noalloc
    ok = (FAKE, FAKE, 1e-6, FAKE, FAKE, 10, 128, 1024, FAKE, FAKE, None)

    def call(**kw):
        a = list(ok)
        names = ["x", "gamma", "eps", "W", "target", "T", "H", "V", "logprob", "lse", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    for k in ("x", "gamma", "W", "target", "logprob"):
        assert call(**{k: None}) == rz.RZ_EINVAL, k
    assert call(x=FAKE + 8) == rz.RZ_EINVAL
    assert call(target=FAKE + 2) == rz.RZ_EINVAL
    assert call(eps=-1.0) == rz.RZ_EINVAL
    assert call(T=0) == rz.RZ_EINVAL
    assert call(H=100) == rz.RZ_EUNSUPPORTED
    # beyond the built-in scratch (8,572 rows at the 1.5B-shaped head):
    # rejected on the host, before any HIP call
    assert call(T=8573, H=1536, V=151936) == rz.RZ_EWORKSPACE
    assert call(T=4096, H=16384, V=1024) == rz.RZ_EWORKSPACE
    # the path runs in chunks of 32,768 rows: a long batch on a small head fits
    if not _gpu_present():
        assert call(T=1 << 20, H=128, V=1024) == rz.RZ_ENODEV
    assert rz.NOALLOC_SCRATCH_BYTES == 64 << 20


@pytest.mark.skipif(_gpu_present(), reason="valid arguments would reach the GPU")
def test_no_device_is_reported():
    assert rz.lib().rz_logprob_noalloc(FAKE, FAKE, 1e-6, FAKE, FAKE, 8572, 1536, 151936, FAKE,
                                       FAKE, None) == rz.RZ_ENODEV
    assert _rmsnorm() == rz.RZ_ENODEV
    assert _rmsnorm(rstd=None) == rz.RZ_ENODEV
    assert _logprob() == rz.RZ_ENODEV
    assert _backward() == rz.RZ_ENODEV
    assert _logprob_store() == rz.RZ_ENODEV
    assert _logprob_store(lse=None) == rz.RZ_ENODEV
    assert _backward_stored() == rz.RZ_ENODEV
    assert _backward_grads() == rz.RZ_ENODEV
    assert _backward_grads(logits=FAKE, lgb=1 << 40) == rz.RZ_ENODEV
    assert _is_loss() == rz.RZ_ENODEV
    assert rz.lib().rz_d3(FAKE, FAKE, 10, FAKE, FAKE, 1 << 20, None) == rz.RZ_ENODEV
    assert _step() == rz.RZ_ENODEV
    assert _shard() == rz.RZ_ENODEV
    assert rz.lib().rz_logprob_merge(FAKE, FAKE, 10, 100, FAKE, FAKE, None) == rz.RZ_ENODEV


def test_host_offset_validation():
    rz.validate_offsets([0, 3, 5], [0, 2], 5)
    with pytest.raises(ValueError):
        rz.validate_offsets([0, 3, 3, 5], [0, 3], 5)   # zero-length response
    with pytest.raises(ValueError):
        rz.validate_offsets([0, 3, 5], [0, 2], 6)      # does not end at T
    with pytest.raises(ValueError):
        rz.validate_offsets([0, 3, 5], [0, 1], 5)      # groups do not cover R
    with pytest.raises(ValueError):
        rz.validate_offsets([1, 3, 5], [0, 2], 5)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import importlib
    mod = importlib.import_module("invariant_logprob_is_amd")
    monkeypatch.setattr(mod, "_lib", None)
    monkeypatch.setattr(mod, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        mod.lib()


def test_stored_binding_checks_before_the_call():
    # CPU tensors with a wrong dtype or shape never reach the library
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    g = torch.zeros(64, dtype=torch.bfloat16)
    W = torch.zeros(100, 64, dtype=torch.bfloat16)
    t = torch.zeros(4, dtype=torch.int32)
    f = torch.zeros(4, dtype=torch.float32)
    lg = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(TypeError):
        rz.logprob_store(x.float(), g, W, t)
    with pytest.raises(TypeError):
        rz.logprob_store(x, g, W, t.long())
    with pytest.raises(ValueError):
        rz.logprob_store(x, g[:32], W, t)
    with pytest.raises(ValueError):
        rz.logprob_store(x, g, W, t[:3])
    with pytest.raises(TypeError):
        rz.backward_stored(x, g, W, t, f, f, lg.float())
    with pytest.raises(ValueError):
        rz.backward_stored(x, g, W, t, f[:3], f, lg)
    with pytest.raises(ValueError):
        rz.backward_stored(x, g, W, t, f, f[:2], lg)
    with pytest.raises(ValueError):
        rz.backward_stored(x, g, W, t, f, f, lg.view(32, 32))


def test_a_plain_c_caller(tmp_path):
    """include/rz.h from C: compiled with gcc, linked against the library,
    run with the host-side checks only."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    # the plain library, and no preloaded sanitizer runtime (the sanitized
    # run of these tests preloads one for the Python process only)
    libdir = os.path.join(ROOT, "invariant_logprob_is_amd")
    lib = os.path.join(libdir, "librz.so")
    if not os.path.exists(lib):
        pytest.skip("librz.so not built")
    env = {k: v for k, v in os.environ.items() if k not in ("LD_PRELOAD", "ASAN_OPTIONS",
                                                            "UBSAN_OPTIONS")}
    exe = tmp_path / "abi_check"
    subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", str(exe), lib,
                    f"-Wl,-rpath,{libdir}"], check=True, capture_output=True, text=True, env=env)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check: ok" in r.stdout
