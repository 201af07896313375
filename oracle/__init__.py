"""Oracle for the REINFORCE Zero learner head: plain, slow, float64 numpy.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product path
(the HIP library and its Python binding) never calls it and shares no code
with it; the two sides meet only in the seeded input generators of the
``workloads`` package, which hold none of the method's arithmetic.

Sources.  Three web pages describe the method:
  [P1] "REINFORCE-Zero: kernel alignment + unclipped IS enables 20K-step
       stable async RL" (agihunt.info summary), sections "Core insight" and
       "Results".
  [P2] "Zero Mismatch, Simple Async RL: REINFORCE Zero, DeepSeek-V4.1 and Kimi
       K3.1" (vLLM blog post), sections "Only one probability gap comes from old
       weights" (with the log-ratio decomposition equation), "Alignment permits
       a simpler learning path", "Keep throughput, lag and quality conditions
       separate" and "Large-model validation exposes concrete failure
       mechanisms".
  [P3] "REINFORCE Zero：为什么内核对齐后，极简 IS 能让异步 RL 稳定训练 20,000 步？"
       (Qingke AI repost), its body text and the captions of Fig. 1 and Fig. 2.

Every function below cites the passage it follows.  Where the pages are silent
(the RMSNorm epsilon and rounding point, the loss value form, the mean over
responses) the function says which reading it takes.

Pins.  Each function is pinned in tests/test_oracle_pins.py against closed
forms, library routines (torch.log_softmax, torch rms_norm, scipy's KL),
brute force and float64 finite differences, and against the hand-derived
golden cases in tests/golden/.  No function here is "parity unpinned"; the
*value form* of the loss (as opposed to its gradient) and the RMSNorm epsilon
are readings the pages do not fix, and are pinned only as readings.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_decode", "bf16_round", "rmsnorm", "logits", "log_softmax_gather",
    "logprob", "advantages", "is_weights", "is_loss", "is_coef_rows", "d3", "kl_estimators",
    "peak_median", "decompose", "logit_grad", "weight_grads",
    "rmsnorm_backward", "backward", "learner_step",
]


# --------------------------------------------------------------------------
# bf16 storage
# --------------------------------------------------------------------------

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 storage bits -> exact float64 values (a bf16 is the top half of
    an IEEE float32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _vals(a) -> np.ndarray:
    """bf16 storage bits (uint16) are decoded; anything else is taken as
    float64 values (the finite-difference pins perturb continuous values)."""
    a = np.asarray(a)
    return bf16_decode(a) if a.dtype == np.uint16 else a.astype(np.float64)


def bf16_round(y: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, directly
    from float64 (one rounding).  bf16 keeps 8 significant bits and the float32
    exponent range; values below the smallest normal keep the fixed subnormal
    quantum 2**-133.  Returns float64."""
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros_like(y)
    fin = np.isfinite(y) & (y != 0.0)
    m, e = np.frexp(y[fin])                      # y = m * 2**e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)                  # quantum exponent
    out[fin] = np.ldexp(np.rint(np.ldexp(y[fin], -q)), q)   # rint: half to even
    out[~np.isfinite(y)] = y[~np.isfinite(y)]
    big = np.abs(out) > 3.3895313892515355e38   # above the largest finite bf16
    out[big] = np.copysign(np.inf, out[big])
    return out


# --------------------------------------------------------------------------
# Forward: final RMSNorm, LM head, log-softmax at the target
# --------------------------------------------------------------------------

def rmsnorm(x_bits, gamma_bits, eps: float, round_output: bool = True):
    """Final RMSNorm of each row, then one rounding to bf16.

    The pages ask that the learner and the rollout run the *same* forward
    computation for a given row ([P3] body: batch-invariant kernels plus a
    matching forward pass).  They do not print the norm; the reading taken
    here is the usual final RMSNorm of the Qwen-family models the pages train:
    ms = mean_k x_k^2, r = (ms + eps)^(-1/2), y_k = gamma_k * x_k * r, and the
    LM head consumes y rounded once to bf16 (round to nearest even).

    Returns (hhat [T,H] float64, r [T] float64).  With round_output=False the
    rounding is skipped (used by the finite-difference pins)."""
    x = _vals(x_bits)
    g = _vals(gamma_bits)
    eps64 = float(np.float32(eps))
    ms = np.mean(x * x, axis=1)
    r = 1.0 / np.sqrt(ms + eps64)
    y = (g[None, :] * x) * r[:, None]
    return (bf16_round(y) if round_output else y), r


def logits(hhat: np.ndarray, Wv: np.ndarray) -> np.ndarray:
    """z[t, v] = sum_k hhat[t, k] * W[v, k]: the LM-head product in float64
    (exact for all practical purposes on bf16 operands)."""
    return np.asarray(hhat, np.float64) @ np.asarray(Wv, np.float64).T


def log_softmax_gather(z: np.ndarray, target: np.ndarray):
    """Per-token log-probability of the target token under softmax(z).

    [P2] "Only one probability gap comes from old weights": the importance
    ratio compares the learner's probability of the sampled token with the one
    recorded at rollout; this is the learner's log pi(y_t | history).
    lse_t = m_t + log sum_v exp(z_tv - m_t) with m_t = max_v z_tv;
    logpi_t = z_{t, target_t} - lse_t.  Returns (logpi [T], lse [T])."""
    m = np.max(z, axis=1)
    lse = m + np.log(np.sum(np.exp(z - m[:, None]), axis=1))
    zt = z[np.arange(z.shape[0]), np.asarray(target, np.int64)]
    return zt - lse, lse


def logprob(x_bits, gamma_bits, eps, W_bits, target, row_chunk: int = 256):
    """End-to-end learner log-probabilities: rmsnorm -> logits ->
    log_softmax_gather, row chunk by row chunk (rows are independent).
    Returns (logpi [T], lse [T])."""
    Wv = _vals(W_bits)
    T = np.asarray(x_bits).shape[0]
    lp = np.empty(T)
    lse = np.empty(T)
    for a in range(0, T, row_chunk):
        b = min(T, a + row_chunk)
        hh, _ = rmsnorm(x_bits[a:b], gamma_bits, eps)
        lp[a:b], lse[a:b] = log_softmax_gather(logits(hh, Wv), target[a:b])
    return lp, lse


# --------------------------------------------------------------------------
# Unclipped token-level IS REINFORCE loss and the D3 diagnostic
# --------------------------------------------------------------------------

def advantages(reward, group_offsets) -> np.ndarray:
    """[P2] "Alignment permits a simpler learning path": the advantage of a
    response is its reward minus the mean reward of its prompt group; no value
    model, no std scaling.  Reading: the group mean includes the response
    itself.  group_offsets[G+1] are response offsets of the groups."""
    r = np.asarray(reward, np.float64)
    go = np.asarray(group_offsets, np.int64)
    A = np.empty_like(r)
    for g in range(len(go) - 1):
        a, b = go[g], go[g + 1]
        A[a:b] = r[a:b] - np.mean(r[a:b])
    return A


def is_weights(logp, mu):
    """Token-level importance weight w = pi / mu = exp(log pi - log mu), with
    no clipping ([P1] lede and "Core insight"; [P2] intro and the
    decomposition of log pi - log mu; [P3] body: the IS coefficient is the
    exponential of the log-probability difference, and no ratio clipping is
    used).  Returns (w, delta)."""
    delta = np.asarray(logp, np.float64) - np.asarray(mu, np.float64)
    return np.exp(delta), delta


def is_loss(logp, mu, resp_offsets, group_offsets, reward):
    """Unclipped token-level IS REINFORCE loss ([P2] "Alignment permits a
    simpler learning path": advantage = reward minus group mean, tokens
    averaged within each response, no value model, no rejection gate).

    Reading of the value form (the pages print no formula): the surrogate
    that is minimised,
        loss = -(1/R) sum_i A_i * (1/L_i) sum_{t in i} w_t,
    whose gradient with respect to log pi_t is
        coef_t = -A_i * w_t / (R * L_i).
    The mean over responses is a plain mean over all R responses.

    Returns a dict with loss, coef [T], advantage [R], w [T]."""
    ro = np.asarray(resp_offsets, np.int64)
    R = len(ro) - 1
    A = advantages(reward, group_offsets)
    w, _ = is_weights(logp, mu)
    coef = np.empty_like(w)
    total = 0.0
    for i in range(R):
        a, b = ro[i], ro[i + 1]
        L = b - a
        total += A[i] * np.mean(w[a:b])
        coef[a:b] = -A[i] * w[a:b] / (R * L)
    return {"loss": -total / R, "coef": coef, "advantage": A, "w": w}


def is_coef_rows(logp_rows, mu_rows, rows, resp_offsets, group_offsets, reward):
    """coef_t = -A_i w_t / (R L_i) for a subset of tokens `rows` (global token
    indices) of a batch, with that batch's structure: the same quantity
    is_loss returns, for when the batch is too large for the oracle's forward
    on every token.  The coefficient of a token needs only its own logpi and
    mu plus the per-response metadata."""
    ro = np.asarray(resp_offsets, np.int64)
    R = len(ro) - 1
    A = advantages(reward, group_offsets)
    rows = np.asarray(rows, np.int64)
    resp = np.searchsorted(ro, rows, side="right") - 1
    L = (ro[resp + 1] - ro[resp]).astype(np.float64)
    w, _ = is_weights(logp_rows, mu_rows)
    return -A[resp] * w / (R * L)


def d3(logp, mu) -> float:
    """D3 diagnostic: the per-update token mean of w - 1 - log w ([P2] "Only
    one probability gap comes from old weights"; [P3] Fig. 2 caption: a batch
    average).  Reading: a flat mean over all tokens of the update.  Since
    log w = delta, w - 1 - log w = expm1(delta) - delta, written that way to
    avoid cancellation when w is near 1."""
    _, delta = is_weights(logp, mu)
    return float(np.mean(np.expm1(delta) - delta))


def kl_estimators(logp, mu):
    """Sample estimates of the rollout-to-learner KL, KL(mu || pi), from the
    tokens of one update, which were drawn from the rollout policy mu ([P3]
    Fig. 1 caption: the KL is estimated from samples; [P2] "Only one
    probability gap comes from old weights" for D3).  The pages name no
    estimator; the reading taken is the three standard ones in the log ratio
    delta = log pi - log mu (so w = e^delta = pi / mu):
        k1 = mean(-delta), k2 = mean(delta^2 / 2), k3 = mean(w - 1 - delta).
    Under tokens drawn from mu, k1 and k3 are unbiased for KL(mu || pi)
    (E_mu[w] = 1), and k3 is the pages' D3 (same expression as d3()).  Flat
    means over all tokens of the update.  Returns (k1, k2, k3)."""
    _, delta = is_weights(logp, mu)
    return (float(np.mean(-delta)), float(np.mean(0.5 * delta * delta)),
            float(np.mean(np.expm1(delta) - delta)))


def peak_median(series):
    """The tracking statistic the pages report for a per-update diagnostic
    over a training run ([P2] "Only one probability gap comes from old
    weights" and [P3] Fig. 2: the peak of the per-update D3 over its median;
    [P2] "Keep throughput, lag and quality conditions separate": the median
    KL of a window of updates).  Returns (median, peak, peak / median) of the
    values, median as numpy defines it (mean of the middle two for an even
    count)."""
    v = np.asarray(series, np.float64)
    med = float(np.median(v))
    peak = float(np.max(v))
    return med, peak, peak / med


def decompose(logp_learner, logp_learner_old, mu):
    """The log-ratio decomposition of [P2] "Only one probability gap comes from
    old weights" for one token history:
        log pi_k - log mu_v = (log pi_k - log pi_v) + (log pi_v - log mu_v),
    pi_k the learner at the current weights, pi_v the learner at the rollout's
    weights, mu_v what the rollout recorded.  The first term is the weight
    lag, the second the kernel mismatch, which batch-invariant kernels with a
    matching forward make exactly 0 ([P3] body).  Inputs are per-token
    log-probabilities; returns (lag, mismatch) in float64."""
    a = np.asarray(logp_learner, np.float64)
    b = np.asarray(logp_learner_old, np.float64)
    m = np.asarray(mu, np.float64)
    return a - b, b - m


# --------------------------------------------------------------------------
# Backward to the hidden states
# --------------------------------------------------------------------------

def logit_grad(z, lse, target, coef):
    """d loss / d z for the loss above: logpi_t = z_t,tgt - lse_t, so
    d logpi_t / d z_tv = onehot(tgt)_v - p_tv with p = exp(z - lse), and the
    chain rule multiplies by coef_t.  Returns dlogits [T, V]."""
    p = np.exp(z - np.asarray(lse, np.float64)[:, None])
    g = -p
    g[np.arange(z.shape[0]), np.asarray(target, np.int64)] += 1.0
    return np.asarray(coef, np.float64)[:, None] * g


def rmsnorm_backward(x_bits, gamma_bits, eps, dhhat):
    """Gradient through y_k = gamma_k x_k r, r = (mean x^2 + eps)^(-1/2):
        dx_j = r gamma_j g_j - x_j r^3 (1/H) sum_k gamma_k g_k x_k,
    with the bf16 rounding of y treated as the identity (straight-through)."""
    x = _vals(x_bits)
    gm = _vals(gamma_bits)
    _, r = rmsnorm(x_bits, gamma_bits, eps, round_output=False)
    H = x.shape[1]
    s = np.sum(gm[None, :] * dhhat * x, axis=1)
    return r[:, None] * gm[None, :] * dhhat - x * (r ** 3 * s / H)[:, None]


def backward(x_bits, gamma_bits, eps, W_bits, target, lse, coef, row_chunk: int = 256,
             round_hhat: bool = True):
    """dhidden = d loss / d x for given per-token lse and coef.
    dhhat_t = sum_v dlogits_tv W_v, then rmsnorm_backward.  Row chunked.
    The logits are formed from the bf16-rounded hhat, as in the forward
    (round_hhat=False drops that rounding, for the finite-difference pins)."""
    Wv = _vals(W_bits)
    T = np.asarray(x_bits).shape[0]
    H = Wv.shape[1]
    out = np.empty((T, H))
    for a in range(0, T, row_chunk):
        b = min(T, a + row_chunk)
        hh, _ = rmsnorm(x_bits[a:b], gamma_bits, eps, round_output=round_hhat)
        z = logits(hh, Wv)
        dh = logit_grad(z, lse[a:b], target[a:b], coef[a:b]) @ Wv
        out[a:b] = rmsnorm_backward(x_bits[a:b], gamma_bits, eps, dh)
    return out


def weight_grads(x_bits, gamma_bits, eps, W_bits, target, lse, coef, row_chunk: int = 256,
                 round_hhat: bool = True):
    """The gradients of the loss with respect to the LM-head weight and the
    RMSNorm weight, for given per-token lse and coef (the rest of the
    learner head's backward; the pages' update step applies the gradient of
    the loss above to all weights, [P2] "Alignment permits a simpler learning
    path").  With dlogits = coef (onehot - p) as in logit_grad:
        dW[v, k] = sum_t dlogits[t, v] hhat[t, k],
        dgamma[k] = sum_t dhhat[t, k] x[t, k] r_t,   dhhat = dlogits W,
    the second because y = gamma x r and the bf16 rounding of y is treated as
    the identity (straight-through), as in rmsnorm_backward.  The logits and
    dW use the rounded hhat, as the forward does (round_hhat=False drops that
    rounding, for the finite-difference pins).  Row chunked; float64.
    Returns (dW [V, H], dgamma [H])."""
    Wv = _vals(W_bits)
    x = _vals(x_bits)
    T = x.shape[0]
    V, H = Wv.shape
    dW = np.zeros((V, H))
    dg = np.zeros(H)
    for a in range(0, T, row_chunk):
        b = min(T, a + row_chunk)
        hh, r = rmsnorm(x_bits[a:b], gamma_bits, eps, round_output=round_hhat)
        g = logit_grad(logits(hh, Wv), lse[a:b], target[a:b], coef[a:b])
        dW += g.T @ hh
        dg += np.sum((g @ Wv) * x[a:b] * r[:, None], axis=0)
    return dW, dg


def learner_step(x_bits, gamma_bits, eps, W_bits, target, mu, resp_offsets, group_offsets, reward):
    """The whole learner head for one update: logprob, IS loss, D3, dhidden."""
    lp, lse = logprob(x_bits, gamma_bits, eps, W_bits, target)
    L = is_loss(lp, mu, resp_offsets, group_offsets, reward)
    return {
        "logprob": lp, "lse": lse, "loss": L["loss"], "coef": L["coef"],
        "advantage": L["advantage"], "w": L["w"], "d3": d3(lp, mu),
        "dhidden": backward(x_bits, gamma_bits, eps, W_bits, target, lse, L["coef"]),
    }
