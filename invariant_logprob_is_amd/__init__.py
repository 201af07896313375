"""Python binding of librz.so, the HIP library declared in include/rz.h.

Argument marshalling only: every step of the learner head runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  There is no CPU fallback: if librz.so is missing, every call raises.

    import invariant_logprob_is_amd as rz
    lp, lse = rz.logprob(x, gamma, W, target)             # batch-invariant
    loss, coef, adv = rz.is_loss(lp, mu, resp_offsets, group_offsets, reward)
    d3 = rz.d3(lp, mu)
    dx = rz.backward(x, gamma, W, target, lse, coef)
    out = rz.learner_step(x, gamma, W, target, mu, resp_offsets, group_offsets, reward)

bf16 tensors are torch.bfloat16; log-probabilities fp32; offsets int64.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "RzError", "lib", "version", "workspace_bytes", "workspace_bytes_grads", "rmsnorm", "logprob",
    "logprob_noalloc", "NOALLOC_SCRATCH_BYTES", "is_loss", "d3", "kl",
    "decompose", "backward", "logits_bytes", "logprob_store", "backward_stored",
    "backward_grads", "logprob_fn",
    "learner_step", "validate_offsets", "profile_enable", "profile_read", "LIB_PATH",
    "VOCAB_SPLITS", "vocab_split_begin", "logprob_shard", "logprob_merge", "split_records",
    "RZ_OK", "RZ_EINVAL", "RZ_EUNSUPPORTED", "RZ_ENODEV",
    "RZ_EHIP", "RZ_EWORKSPACE", "SYMBOLS",
]

# RZ_LIB_PATH selects another build of the same library (the sanitized
# librz_san.so of the CPU tests); there is no fallback of any kind.
LIB_PATH = os.environ.get("RZ_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "librz.so")

RZ_OK, RZ_EINVAL, RZ_EUNSUPPORTED, RZ_ENODEV, RZ_EHIP, RZ_EWORKSPACE = range(6)

VOCAB_SPLITS = 8        # RZ_VOCAB_SPLITS
_SPLIT_RECORD = 24      # sizeof(rz_vocab_split)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/rz.h
SYMBOLS = {
    "rz_version": (ctypes.c_int, []),
    "rz_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "rz_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "rz_workspace_bytes_grads": (_SZ, [_I64, _I32, _I32]),
    "rz_rmsnorm": (ctypes.c_int, [_P, _P, _F32, _I64, _I32, _P, _P, _P]),
    "rz_logprob": (ctypes.c_int, [_P, _P, _F32, _P, _P, _I64, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "rz_logprob_noalloc": (ctypes.c_int, [_P, _P, _F32, _P, _P, _I64, _I32, _I32, _P, _P, _P]),
    "rz_is_loss": (ctypes.c_int, [_P, _P, _I64, _P, _I32, _P, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "rz_d3": (ctypes.c_int, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "rz_backward": (ctypes.c_int, [_P, _P, _F32, _P, _P, _P, _P, _I64, _I32, _I32, _P, _P, _SZ, _P]),
    "rz_logits_bytes": (_SZ, [_I64, _I32, _I32]),
    "rz_logprob_store": (ctypes.c_int, [_P, _P, _F32, _P, _P, _I64, _I32, _I32, _P, _P, _P, _SZ,
                                        _P, _SZ, _P]),
    "rz_backward_stored": (ctypes.c_int, [_P, _P, _F32, _P, _P, _P, _P, _I64, _I32, _I32, _P,
                                          _SZ, _P, _P, _SZ, _P]),
    "rz_backward_grads": (ctypes.c_int, [_P, _P, _F32, _P, _P, _P, _P, _I64, _I32, _I32, _P, _SZ,
                                         _P, _P, _P, _P, _SZ, _P]),
    "rz_kl": (ctypes.c_int, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "rz_decompose": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _F32, _P, _P, _I64, _I32, _I32, _P, _P,
                                    _P, _P, _SZ, _P]),
    "rz_learner_step": (ctypes.c_int, [_P, _P, _F32, _P, _P, _P, _I64, _I32, _I32, _P, _I32, _P,
                                       _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                       _P]),
    "rz_vocab_split_begin": (_I64, [_I32, _I32]),
    "rz_logprob_shard": (ctypes.c_int, [_P, _P, _F32, _P, _P, _I64, _I32, _I32, _I32, _I32, _P,
                                        _P, _SZ, _P]),
    "rz_logprob_merge": (ctypes.c_int, [_P, _P, _I64, _I32, _P, _P, _P]),
    "rz_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "rz_profile_count": (ctypes.c_int, []),
    "rz_profile_get": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                      ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)]),
}

_lib = None


class RzError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().rz_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed: {msg} (status {status})")


def lib() -> ctypes.CDLL:
    """Load librz.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m invariant_logprob_is_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SYMBOLS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def version() -> int:
    return lib().rz_version()


def workspace_bytes(T: int, H: int, V: int) -> int:
    return int(lib().rz_workspace_bytes(T, H, V))


def workspace_bytes_grads(T: int, H: int, V: int) -> int:
    """Workspace of learner_step with weight_grads (rz_workspace_bytes_grads)."""
    return int(lib().rz_workspace_bytes_grads(T, H, V))


def _check(fn: str, status: int):
    if status != RZ_OK:
        raise RzError(fn, status)


def _torch():
    import torch
    return torch


def _stream(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, device, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _workspace(nbytes: int, device, workspace):
    torch = _torch()
    if workspace is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace too small: {workspace.numel()} < {nbytes} bytes")
    return workspace


def rmsnorm(x, gamma, eps: float = 1e-6, *, out=None, rstd_out=None):
    """The final RMSNorm alone (rz_rmsnorm): the hhat bits the LM head of
    logprob / backward / learner_step consumes.

    x [T,H] bf16, gamma [H] bf16.  Returns (hhat [T,H] bf16, rstd [T] fp32)."""
    torch = _torch()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    T, H = x.shape
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    if gamma.shape[0] != H:
        raise ValueError("shape mismatch between x and gamma")
    hh = out if out is not None else torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    rs = rstd_out if rstd_out is not None else torch.empty(T, dtype=torch.float32, device=dev)
    _need(hh, "out", torch.bfloat16, dev, 2)
    _need(rs, "rstd_out", torch.float32, dev, 1)
    if tuple(hh.shape) != (T, H) or rs.shape[0] != T:
        raise ValueError("output shapes do not match x")
    st = lib().rz_rmsnorm(x.data_ptr(), gamma.data_ptr(), float(eps), T, H, hh.data_ptr(),
                          rs.data_ptr(), _stream(dev))
    _check("rz_rmsnorm", st)
    return hh, rs


def logprob(x, gamma, W, target, eps: float = 1e-6, *, workspace=None, out=None,
            lse_out=None):
    """Batch-invariant per-token log-probabilities (rz_logprob).

    x [T,H] bf16, gamma [H] bf16, W [V,H] bf16, target [T] int32, all on one
    GPU.  Returns (logprob [T] fp32, lse [T] fp32)."""
    torch = _torch()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    T, H = x.shape
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    _need(W, "W", torch.bfloat16, dev, 2)
    _need(target, "target", torch.int32, dev, 1)
    V = W.shape[0]
    if gamma.shape[0] != H or W.shape[1] != H or target.shape[0] != T:
        raise ValueError("shape mismatch among x, gamma, W, target")
    lp = out if out is not None else torch.empty(T, dtype=torch.float32, device=dev)
    ls = lse_out if lse_out is not None else torch.empty(T, dtype=torch.float32, device=dev)
    _need(lp, "out", torch.float32, dev, 1)
    _need(ls, "lse_out", torch.float32, dev, 1)
    nb = workspace_bytes(T, H, V)
    ws = _workspace(nb, dev, workspace)
    st = lib().rz_logprob(x.data_ptr(), gamma.data_ptr(), float(eps), W.data_ptr(),
                          target.data_ptr(), T, H, V, lp.data_ptr(), ls.data_ptr(),
                          ws.data_ptr(), ws.numel(), _stream(dev))
    _check("rz_logprob", st)
    return lp, ls


NOALLOC_SCRATCH_BYTES = 64 << 20   # RZ_NOALLOC_SCRATCH_BYTES


def logprob_noalloc(x, gamma, W, target, eps: float = 1e-6, *, out=None, lse_out=None):
    """rz_logprob_noalloc: logprob() on the library's built-in device scratch,
    with no workspace (same bits as logprob()).  For callers that cannot
    allocate, pass preallocated `out` and `lse_out`.  Calls that overlap on
    one GPU race on the scratch.  Returns (logprob [T] fp32, lse [T] fp32)."""
    torch = _torch()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    T, H = x.shape
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    _need(W, "W", torch.bfloat16, dev, 2)
    _need(target, "target", torch.int32, dev, 1)
    V = W.shape[0]
    if gamma.shape[0] != H or W.shape[1] != H or target.shape[0] != T:
        raise ValueError("shape mismatch among x, gamma, W, target")
    lp = out if out is not None else torch.empty(T, dtype=torch.float32, device=dev)
    ls = lse_out if lse_out is not None else torch.empty(T, dtype=torch.float32, device=dev)
    _need(lp, "out", torch.float32, dev, 1)
    _need(ls, "lse_out", torch.float32, dev, 1)
    st = lib().rz_logprob_noalloc(x.data_ptr(), gamma.data_ptr(), float(eps), W.data_ptr(),
                                  target.data_ptr(), T, H, V, lp.data_ptr(), ls.data_ptr(),
                                  _stream(dev))
    _check("rz_logprob_noalloc", st)
    return lp, ls


def vocab_split_begin(V: int, s: int) -> int:
    """First vocabulary row of split s (rz_vocab_split_begin); s = VOCAB_SPLITS gives V."""
    r = int(lib().rz_vocab_split_begin(V, s))
    if r < 0:
        raise ValueError(f"invalid split {s} for V = {V}")
    return r


def logprob_shard(x, gamma, W_rows, target, V: int, s0: int, s1: int, eps: float = 1e-6, *,
                  workspace=None, out=None):
    """Partials of vocabulary splits [s0, s1) (rz_logprob_shard).

    W_rows holds rows [vocab_split_begin(V, s0), vocab_split_begin(V, s1)) of
    the [V,H] weight (a view of W, or a device's own share of it).  Returns
    the records as a [s1 - s0, T, 3] float64 tensor holding rz_vocab_split
    structs (decode with split_records)."""
    torch = _torch()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    T, H = x.shape
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    _need(W_rows, "W_rows", torch.bfloat16, dev, 2)
    _need(target, "target", torch.int32, dev, 1)
    if not (0 <= s0 < s1 <= VOCAB_SPLITS):
        raise ValueError(f"need 0 <= s0 < s1 <= {VOCAB_SPLITS}")
    rows = vocab_split_begin(V, s1) - vocab_split_begin(V, s0)
    if W_rows.shape != (rows, H) and not (rows == 0 and W_rows.shape[1] == H):
        raise ValueError(f"W_rows must hold the {rows} rows of splits [{s0}, {s1})")
    if gamma.shape[0] != H or target.shape[0] != T:
        raise ValueError("shape mismatch among x, gamma, target")
    recs = out if out is not None else torch.empty((s1 - s0, T, 3), dtype=torch.float64,
                                                   device=dev)
    _need(recs, "out", torch.float64, dev, 3)
    if tuple(recs.shape) != (s1 - s0, T, 3):
        raise ValueError("out must be [s1 - s0, T, 3] float64")
    ws = _workspace(workspace_bytes(T, H, V), dev, workspace)
    # an empty share still needs a valid, aligned pointer
    wp = W_rows.data_ptr() if W_rows.numel() else gamma.data_ptr()
    st = lib().rz_logprob_shard(x.data_ptr(), gamma.data_ptr(), float(eps), wp,
                                target.data_ptr(), T, H, V, s0, s1, recs.data_ptr(),
                                ws.data_ptr(), ws.numel(), _stream(dev))
    _check("rz_logprob_shard", st)
    return recs


def logprob_merge(partials, target, V: int, *, out=None, lse_out=None):
    """logprob and lse from the records of all splits (rz_logprob_merge).

    partials: [VOCAB_SPLITS, T, 3] float64 (the shards' outputs concatenated
    in split order).  Returns (logprob [T] fp32, lse [T] fp32)."""
    torch = _torch()
    dev = partials.device
    _need(partials, "partials", torch.float64, dev, 3)
    _need(target, "target", torch.int32, dev, 1)
    T = target.shape[0]
    if tuple(partials.shape) != (VOCAB_SPLITS, T, 3):
        raise ValueError(f"partials must be [{VOCAB_SPLITS}, T, 3] float64")
    lp = out if out is not None else torch.empty(T, dtype=torch.float32, device=dev)
    ls = lse_out if lse_out is not None else torch.empty(T, dtype=torch.float32, device=dev)
    _need(lp, "out", torch.float32, dev, 1)
    _need(ls, "lse_out", torch.float32, dev, 1)
    st = lib().rz_logprob_merge(partials.data_ptr(), target.data_ptr(), T, V, lp.data_ptr(),
                                ls.data_ptr(), _stream(dev))
    _check("rz_logprob_merge", st)
    return lp, ls


def split_records(partials):
    """Host copy of split records as a numpy structured array with fields
    s (f8), m, max_logit, z_target, reserved (f4)."""
    import numpy as np
    raw = partials.detach().cpu().contiguous().numpy().view(np.uint8)
    dt = np.dtype([("s", "<f8"), ("m", "<f4"), ("max_logit", "<f4"), ("z_target", "<f4"),
                   ("reserved", "<f4")])
    return raw.reshape(-1).view(dt).reshape(partials.shape[:-1])


def validate_offsets(resp_offsets, group_offsets, T: int):
    """Host-side check of the ragged structure (the library itself can only
    detect malformed device offsets as a NaN loss)."""
    import numpy as np
    ro = np.asarray(resp_offsets, dtype=np.int64)
    go = np.asarray(group_offsets, dtype=np.int64)
    R, G = len(ro) - 1, len(go) - 1
    if R < 1 or G < 1:
        raise ValueError("need at least one response and one group")
    if ro[0] != 0 or ro[-1] != T or np.any(np.diff(ro) <= 0):
        raise ValueError("resp_offsets must start at 0, end at T and strictly increase")
    if go[0] != 0 or go[-1] != R or np.any(np.diff(go) <= 0):
        raise ValueError("group_offsets must start at 0, end at R and strictly increase")


def _offsets_on(t, dev, name):
    torch = _torch()
    t = torch.as_tensor(t, dtype=torch.int64)
    if t.device != dev:
        t = t.to(dev)
    return _need(t.contiguous(), name, torch.int64, dev, 1)


def is_loss(logprob, rollout_logprob, resp_offsets, group_offsets, reward, *,
            workspace=None, want_coef: bool = True, want_advantage: bool = True):
    """Unclipped token-level IS REINFORCE loss (rz_is_loss).

    Offsets given on the host are validated there first.  Returns
    (loss [1] fp64, coef [T] fp32 or None, advantage [R] fp32 or None)."""
    torch = _torch()
    dev = logprob.device
    _need(logprob, "logprob", torch.float32, dev, 1)
    _need(rollout_logprob, "rollout_logprob", torch.float32, dev, 1)
    T = logprob.shape[0]
    if rollout_logprob.shape[0] != T:
        raise ValueError("logprob and rollout_logprob differ in length")
    if not (isinstance(resp_offsets, torch.Tensor) and resp_offsets.is_cuda):
        validate_offsets(resp_offsets, group_offsets, T)
    ro = _offsets_on(resp_offsets, dev, "resp_offsets")
    go = _offsets_on(group_offsets, dev, "group_offsets")
    R, G = ro.shape[0] - 1, go.shape[0] - 1
    rw = _need(torch.as_tensor(reward, dtype=torch.float32).to(dev).contiguous(), "reward",
               torch.float32, dev, 1)
    if rw.shape[0] != R:
        raise ValueError("reward must have one entry per response")
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    coef = torch.empty(T, dtype=torch.float32, device=dev) if want_coef else None
    adv = torch.empty(R, dtype=torch.float32, device=dev) if want_advantage else None
    ws = _workspace(workspace_bytes(T, 64, 1), dev, workspace)
    st = lib().rz_is_loss(logprob.data_ptr(), rollout_logprob.data_ptr(), T, ro.data_ptr(), R,
                          go.data_ptr(), G, rw.data_ptr(), loss.data_ptr(),
                          coef.data_ptr() if coef is not None else None,
                          adv.data_ptr() if adv is not None else None,
                          ws.data_ptr(), ws.numel(), _stream(dev))
    _check("rz_is_loss", st)
    return loss, coef, adv


def d3(logprob, rollout_logprob, *, workspace=None):
    """D3 diagnostic (rz_d3): token mean of w - 1 - log w.  Returns [1] fp64."""
    torch = _torch()
    dev = logprob.device
    _need(logprob, "logprob", torch.float32, dev, 1)
    _need(rollout_logprob, "rollout_logprob", torch.float32, dev, 1)
    T = logprob.shape[0]
    if rollout_logprob.shape[0] != T:
        raise ValueError("logprob and rollout_logprob differ in length")
    out = torch.empty(1, dtype=torch.float64, device=dev)
    ws = _workspace(workspace_bytes(T, 64, 1), dev, workspace)
    st = lib().rz_d3(logprob.data_ptr(), rollout_logprob.data_ptr(), T, out.data_ptr(),
                     ws.data_ptr(), ws.numel(), _stream(dev))
    _check("rz_d3", st)
    return out


def kl(logprob, rollout_logprob, *, workspace=None):
    """KL estimators (rz_kl): (k1, k2, k3) = token means of -delta,
    delta^2/2 and expm1(delta) - delta.  Returns [3] fp64."""
    torch = _torch()
    dev = logprob.device
    _need(logprob, "logprob", torch.float32, dev, 1)
    _need(rollout_logprob, "rollout_logprob", torch.float32, dev, 1)
    T = logprob.shape[0]
    if rollout_logprob.shape[0] != T:
        raise ValueError("logprob and rollout_logprob differ in length")
    out = torch.empty(3, dtype=torch.float64, device=dev)
    ws = _workspace(workspace_bytes(T, 64, 1), dev, workspace)
    st = lib().rz_kl(logprob.data_ptr(), rollout_logprob.data_ptr(), T, out.data_ptr(),
                     ws.data_ptr(), ws.numel(), _stream(dev))
    _check("rz_kl", st)
    return out


def decompose(x_new, gamma_new, W_new, x_old, gamma_old, W_old, target, rollout_logprob,
              eps: float = 1e-6, *, workspace=None):
    """Token-level log-ratio decomposition (rz_decompose).  Returns a dict
    with lag, mismatch [T] fp32 and summary [4] fp64 (max |lag|, mean lag,
    max |mismatch|, tokens with mismatch != 0)."""
    torch = _torch()
    dev = x_new.device
    _need(x_new, "x_new", torch.bfloat16, dev, 2)
    T, H = x_new.shape
    _need(x_old, "x_old", torch.bfloat16, dev, 2)
    for n, g in (("gamma_new", gamma_new), ("gamma_old", gamma_old)):
        _need(g, n, torch.bfloat16, dev, 1)
    for n, w in (("W_new", W_new), ("W_old", W_old)):
        _need(w, n, torch.bfloat16, dev, 2)
    _need(target, "target", torch.int32, dev, 1)
    _need(rollout_logprob, "rollout_logprob", torch.float32, dev, 1)
    V = W_new.shape[0]
    if (tuple(x_old.shape) != (T, H) or gamma_new.shape[0] != H or gamma_old.shape[0] != H
            or tuple(W_new.shape) != (V, H) or tuple(W_old.shape) != (V, H)
            or target.shape[0] != T or rollout_logprob.shape[0] != T):
        raise ValueError("shape mismatch among decompose arguments")
    lag = torch.empty(T, dtype=torch.float32, device=dev)
    mis = torch.empty(T, dtype=torch.float32, device=dev)
    summary = torch.empty(4, dtype=torch.float64, device=dev)
    ws = _workspace(workspace_bytes(T, H, V), dev, workspace)
    st = lib().rz_decompose(x_new.data_ptr(), gamma_new.data_ptr(), W_new.data_ptr(),
                            x_old.data_ptr(), gamma_old.data_ptr(), W_old.data_ptr(), float(eps),
                            target.data_ptr(), rollout_logprob.data_ptr(), T, H, V,
                            lag.data_ptr(), mis.data_ptr(), summary.data_ptr(), ws.data_ptr(),
                            ws.numel(), _stream(dev))
    _check("rz_decompose", st)
    return {"lag": lag, "mismatch": mis, "summary": summary}


def backward(x, gamma, W, target, lse, coef, eps: float = 1e-6, *, workspace=None, out=None):
    """Gradient of the loss with respect to the pre-norm hidden states
    (rz_backward).  Returns dhidden [T,H] fp32."""
    torch = _torch()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    T, H = x.shape
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    _need(W, "W", torch.bfloat16, dev, 2)
    _need(target, "target", torch.int32, dev, 1)
    _need(lse, "lse", torch.float32, dev, 1)
    _need(coef, "coef", torch.float32, dev, 1)
    V = W.shape[0]
    if (gamma.shape[0] != H or W.shape[1] != H or target.shape[0] != T or lse.shape[0] != T
            or coef.shape[0] != T):
        raise ValueError("shape mismatch among backward arguments")
    dh = out if out is not None else torch.empty(T, H, dtype=torch.float32, device=dev)
    _need(dh, "out", torch.float32, dev, 2)
    ws = _workspace(workspace_bytes(T, H, V), dev, workspace)
    st = lib().rz_backward(x.data_ptr(), gamma.data_ptr(), float(eps), W.data_ptr(),
                           target.data_ptr(), lse.data_ptr(), coef.data_ptr(), T, H, V,
                           dh.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    _check("rz_backward", st)
    return dh


def logits_bytes(T: int, H: int, V: int) -> int:
    """rz_logits_bytes: size of the stored-logits buffer of logprob_store()."""
    return int(lib().rz_logits_bytes(T, H, V))


def logprob_store(x, gamma, W, target, eps: float = 1e-6, *, logits=None, workspace=None,
                  out=None, lse_out=None):
    """logprob() that also keeps the logits for backward_stored()
    (rz_logprob_store).  Returns (logprob, lse, logits); `logits` is a uint8
    device buffer of logits_bytes(T, H, V) bytes (allocated if not given)."""
    torch = _torch()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    T, H = x.shape
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    _need(W, "W", torch.bfloat16, dev, 2)
    _need(target, "target", torch.int32, dev, 1)
    V = W.shape[0]
    if gamma.shape[0] != H or W.shape[1] != H or target.shape[0] != T:
        raise ValueError("shape mismatch among x, gamma, W, target")
    lp = out if out is not None else torch.empty(T, dtype=torch.float32, device=dev)
    ls = lse_out if lse_out is not None else torch.empty(T, dtype=torch.float32, device=dev)
    _need(lp, "out", torch.float32, dev, 1)
    _need(ls, "lse_out", torch.float32, dev, 1)
    lg = _workspace(logits_bytes(T, H, V), dev, logits)
    ws = _workspace(workspace_bytes(T, H, V), dev, workspace)
    st = lib().rz_logprob_store(x.data_ptr(), gamma.data_ptr(), float(eps), W.data_ptr(),
                                target.data_ptr(), T, H, V, lp.data_ptr(), ls.data_ptr(),
                                lg.data_ptr(), lg.numel(), ws.data_ptr(), ws.numel(), _stream(dev))
    _check("rz_logprob_store", st)
    return lp, ls, lg


def backward_stored(x, gamma, W, target, lse, coef, logits, eps: float = 1e-6, *, workspace=None,
                    out=None):
    """backward() from the logits that logprob_store() kept for the same
    inputs (rz_backward_stored): the same dhidden bits, without recomputing
    the logits."""
    torch = _torch()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    T, H = x.shape
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    _need(W, "W", torch.bfloat16, dev, 2)
    _need(target, "target", torch.int32, dev, 1)
    _need(lse, "lse", torch.float32, dev, 1)
    _need(coef, "coef", torch.float32, dev, 1)
    _need(logits, "logits", torch.uint8, dev, 1)
    V = W.shape[0]
    if (gamma.shape[0] != H or W.shape[1] != H or target.shape[0] != T or lse.shape[0] != T
            or coef.shape[0] != T):
        raise ValueError("shape mismatch among backward arguments")
    dh = out if out is not None else torch.empty(T, H, dtype=torch.float32, device=dev)
    _need(dh, "out", torch.float32, dev, 2)
    ws = _workspace(workspace_bytes(T, H, V), dev, workspace)
    st = lib().rz_backward_stored(x.data_ptr(), gamma.data_ptr(), float(eps), W.data_ptr(),
                                  target.data_ptr(), lse.data_ptr(), coef.data_ptr(), T, H, V,
                                  logits.data_ptr(), logits.numel(), dh.data_ptr(), ws.data_ptr(),
                                  ws.numel(), _stream(dev))
    _check("rz_backward_stored", st)
    return dh


def backward_grads(x, gamma, W, target, lse, coef, eps: float = 1e-6, *, logits=None,
                   workspace=None, out=None):
    """The gradient of sum_t coef_t logprob_t with respect to x, W and gamma
    (rz_backward_grads): dhidden [T,H], dW [V,H] and dgamma [H], all fp32,
    with the learner step's weight-gradient kernels.  `logits` may hold the
    stored logits of logprob_store() for the same inputs (else the logits are
    recomputed); `out` may supply preallocated dhidden, dW, dgamma."""
    torch = _torch()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    T, H = x.shape
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    _need(W, "W", torch.bfloat16, dev, 2)
    _need(target, "target", torch.int32, dev, 1)
    _need(lse, "lse", torch.float32, dev, 1)
    _need(coef, "coef", torch.float32, dev, 1)
    V = W.shape[0]
    if (gamma.shape[0] != H or W.shape[1] != H or target.shape[0] != T or lse.shape[0] != T
            or coef.shape[0] != T):
        raise ValueError("shape mismatch among backward arguments")
    if logits is not None:
        _need(logits, "logits", torch.uint8, dev, 1)
    o = dict(out or {})
    for k, shape in (("dhidden", (T, H)), ("dW", (V, H)), ("dgamma", (H,))):
        if k not in o:
            o[k] = torch.empty(shape, dtype=torch.float32, device=dev)
        _need(o[k], k, torch.float32, dev, len(shape))
        if tuple(o[k].shape) != shape:
            raise ValueError(f"{k}: expected shape {shape}")
    ws = _workspace(workspace_bytes_grads(T, H, V), dev, workspace)
    st = lib().rz_backward_grads(x.data_ptr(), gamma.data_ptr(), float(eps), W.data_ptr(),
                                 target.data_ptr(), lse.data_ptr(), coef.data_ptr(), T, H, V,
                                 logits.data_ptr() if logits is not None else None,
                                 logits.numel() if logits is not None else 0,
                                 o["dhidden"].data_ptr(), o["dW"].data_ptr(),
                                 o["dgamma"].data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    _check("rz_backward_grads", st)
    return o


_logprob_fn = None


def logprob_fn(x, gamma, W, target, eps: float = 1e-6):
    """logprob() as a differentiable PyTorch function: the forward is
    rz_logprob, and the backward hands the incoming gradient of the
    log-probabilities to rz_backward as coef (only x needs a gradient) or to
    rz_backward_grads (gamma or W need one too), so every gradient comes from
    the library's kernels.  Autograd casts the fp32 gradients to the bf16 of
    the inputs; rz.backward_grads gives them in fp32."""
    global _logprob_fn
    if _logprob_fn is None:
        torch = _torch()

        class LogprobFn(torch.autograd.Function):
            @staticmethod
            def forward(ctx, x, gamma, W, target, eps):
                lp, lse = logprob(x, gamma, W, target, eps)
                ctx.save_for_backward(x, gamma, W, target, lse)
                ctx.eps = eps
                return lp

            @staticmethod
            def backward(ctx, grad):
                x, gamma, W, target, lse = ctx.saved_tensors
                coef = grad.to(torch.float32).contiguous()
                need_x, need_g, need_w = ctx.needs_input_grad[:3]
                if not (need_g or need_w):
                    return backward(x, gamma, W, target, lse, coef, ctx.eps), None, None, None, None
                o = backward_grads(x, gamma, W, target, lse, coef, ctx.eps)
                return (o["dhidden"] if need_x else None, o["dgamma"] if need_g else None,
                        o["dW"] if need_w else None, None, None)

        _logprob_fn = LogprobFn
    return _logprob_fn.apply(x, gamma, W, target, float(eps))


def learner_step(x, gamma, W, target, rollout_logprob, resp_offsets, group_offsets, reward,
                 eps: float = 1e-6, *, workspace=None, out=None, weight_grads: bool = False):
    """The whole learner head for one update (rz_learner_step): per-token
    log-probabilities (bit-identical to logprob()), the IS loss, D3, the
    per-token loss gradient coef and dhidden, computing the logits once.

    Returns a dict with logprob, lse, coef [T] fp32, loss, d3 [1] fp64,
    kl [3] fp64 (k1, k2, k3 as kl()) and dhidden [T,H] fp32; with
    weight_grads also dW [V,H] and dgamma [H] fp32 (the larger workspace of
    workspace_bytes_grads).  `out` may supply preallocated tensors for any of
    these keys."""
    torch = _torch()
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    T, H = x.shape
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    _need(W, "W", torch.bfloat16, dev, 2)
    _need(target, "target", torch.int32, dev, 1)
    _need(rollout_logprob, "rollout_logprob", torch.float32, dev, 1)
    V = W.shape[0]
    if (gamma.shape[0] != H or W.shape[1] != H or target.shape[0] != T
            or rollout_logprob.shape[0] != T):
        raise ValueError("shape mismatch among learner_step arguments")
    if not (isinstance(resp_offsets, torch.Tensor) and resp_offsets.is_cuda):
        validate_offsets(resp_offsets, group_offsets, T)
    ro = _offsets_on(resp_offsets, dev, "resp_offsets")
    go = _offsets_on(group_offsets, dev, "group_offsets")
    R, G = ro.shape[0] - 1, go.shape[0] - 1
    rw = _need(torch.as_tensor(reward, dtype=torch.float32).to(dev).contiguous(), "reward",
               torch.float32, dev, 1)
    if rw.shape[0] != R:
        raise ValueError("reward must have one entry per response")
    o = dict(out or {})
    specs = {"logprob": ((T,), torch.float32), "lse": ((T,), torch.float32),
             "coef": ((T,), torch.float32), "loss": ((1,), torch.float64),
             "d3": ((1,), torch.float64), "kl": ((3,), torch.float64),
             "dhidden": ((T, H), torch.float32)}
    if weight_grads:
        specs["dW"] = ((V, H), torch.float32)
        specs["dgamma"] = ((H,), torch.float32)
    for k, (shape, dt) in specs.items():
        if k not in o:
            o[k] = torch.empty(shape, dtype=dt, device=dev)
        _need(o[k], k, dt, dev, len(shape))
    need = workspace_bytes_grads(T, H, V) if weight_grads else workspace_bytes(T, H, V)
    ws = _workspace(need, dev, workspace)
    dW = o["dW"].data_ptr() if weight_grads else None
    dg = o["dgamma"].data_ptr() if weight_grads else None
    st = lib().rz_learner_step(x.data_ptr(), gamma.data_ptr(), float(eps), W.data_ptr(),
                               target.data_ptr(), rollout_logprob.data_ptr(), T, H, V,
                               ro.data_ptr(), R, go.data_ptr(), G, rw.data_ptr(),
                               o["logprob"].data_ptr(), o["lse"].data_ptr(), o["loss"].data_ptr(),
                               o["d3"].data_ptr(), o["kl"].data_ptr(), o["coef"].data_ptr(),
                               o["dhidden"].data_ptr(), dW, dg,
                               ws.data_ptr(), ws.numel(), _stream(dev))
    _check("rz_learner_step", st)
    return o


def profile_enable(on: bool = True) -> None:
    """Start (or stop) per-kernel event timing inside the library; clears
    earlier records."""
    _check("rz_profile_enable", lib().rz_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{kernel name: (total ms, launches)} for the launches recorded since
    profile_enable(True).  Waits for the recorded events."""
    n = lib().rz_profile_count()
    if n < 0:
        raise RzError("rz_profile_count", -n)
    out = {}
    for i in range(n):
        name = ctypes.c_char_p()
        ms = ctypes.c_double()
        cnt = _I64()
        _check("rz_profile_get", lib().rz_profile_get(i, ctypes.byref(name), ctypes.byref(ms),
                                                      ctypes.byref(cnt)))
        out[name.value.decode()] = (ms.value, cnt.value)
    return out
