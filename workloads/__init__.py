"""Seeded synthetic inputs shaped like the workloads the REINFORCE Zero pages
describe (async R1-Distill-Qwen-1.5B with an 8K answer budget, Qwen3-4B at 16K
context and lag 64, the Qwen3-30B-A3B head), plus a tiny case.

This module holds no arithmetic of the method: it draws random numbers, rounds
them to bf16 storage, and lays out ragged batches.  Both the oracle side and
the HIP side consume exactly these arrays.  The rollout log-probabilities are
*not* produced here; the generator returns the lag noise and the caller adds it
to whatever learner log-probability its recipe names.

Every tensor comes from its own child of a ``numpy.random.SeedSequence`` built
from the config's master seed, so adding a tensor never perturbs the others.
Large tensors are drawn in row blocks of ``ROW_BLOCK`` rows, in order, from one
generator; that blocking is part of the recipe.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

ROW_BLOCK = 65536

# Child indices of the master SeedSequence (fixed forever: changing one changes
# the data of every config).
_C_LENGTHS, _C_X, _C_GAMMA, _C_W, _C_TARGET, _C_NOISE, _C_REWARD, _C_TAILS, \
    _C_OUTLIERS, _C_FILLER, _C_PLACEMENT, _C_VERSION = range(12)
_N_CHILDREN = 16


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 storage bits (round to nearest even).

    Storage helper for inputs only: inputs are drawn in float32 and stored as
    bf16, so this one rounding defines the input bits both sides read.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 storage bits to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(master: int, child: int) -> np.random.Generator:
    ss = np.random.SeedSequence(master)
    return np.random.default_rng(ss.spawn(_N_CHILDREN)[child])


def _normal_bf16(rng: np.random.Generator, rows: int, cols: int, std: float,
                 mean: float = 0.0, row_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """rows x cols bf16 bits of N(mean, std), drawn in ROW_BLOCK row blocks."""
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, ROW_BLOCK):
        r1 = min(rows, r0 + ROW_BLOCK)
        blk = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        if mean != 0.0:
            blk += np.float32(mean)
        if row_scale is not None:
            blk *= row_scale[r0:r1, None].astype(np.float32)
        out[r0:r1] = f32_to_bf16_bits(blk)
    return out


@dataclasses.dataclass
class Batch:
    """One ragged learner batch.

    Rows are response tokens; row t pairs the final hidden state that predicts
    ``target[t]`` with that target.  Tokens of a response are contiguous and
    the responses of one prompt group are contiguous.
    """
    name: str
    H: int
    V: int
    x: np.ndarray              # [T, H] uint16 bf16 bits, pre-norm hidden states
                               # ([T, 0] when generated without hidden states)
    gamma: np.ndarray          # [H] uint16 bf16 bits, RMSNorm weight
    W: np.ndarray              # [V, H] uint16 bf16 bits, LM-head weight (row-major)
    target: np.ndarray         # [T] int32
    resp_offsets: np.ndarray   # [R+1] int64 token offsets of responses
    group_offsets: np.ndarray  # [G+1] int64 response offsets of prompt groups
    reward: np.ndarray         # [R] float32
    lag_noise: np.ndarray      # [T] float32, added to a learner logprob to form mu
    eps: float = 1e-6

    @property
    def T(self) -> int:
        return int(self.resp_offsets[-1])

    @property
    def R(self) -> int:
        return int(self.resp_offsets.shape[0] - 1)

    @property
    def G(self) -> int:
        return int(self.group_offsets.shape[0] - 1)


def _offsets(lengths: np.ndarray) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths.astype(np.int64), out=off[1:])
    return off


def _assemble(name: str, master: int, lengths: np.ndarray, group_size: int, H: int, V: int,
              noise_std: float, reward_kind: str, reward_p: float = 0.5,
              tail_frac: float = 0.0, tail_shift: float = 0.0,
              outlier_frac: float = 0.0, outlier_scale: float = 1.0,
              with_W: bool = True, with_x: bool = True) -> Batch:
    T = int(lengths.sum())
    R = len(lengths)
    assert R % group_size == 0
    G = R // group_size
    row_scale = None
    if outlier_frac > 0.0:
        ro = _rng(master, _C_OUTLIERS)
        n_out = max(1, int(round(outlier_frac * T)))
        idx = ro.choice(T, size=n_out, replace=False)
        row_scale = np.ones(T, dtype=np.float32)
        row_scale[idx] = np.float32(outlier_scale)
    x = (_normal_bf16(_rng(master, _C_X), T, H, 1.0, row_scale=row_scale) if with_x
         else np.zeros((T, 0), np.uint16))
    gamma = _normal_bf16(_rng(master, _C_GAMMA), 1, H, 0.1, mean=1.0)[0]
    W = _normal_bf16(_rng(master, _C_W), V, H, 0.02) if with_W else None
    target = _rng(master, _C_TARGET).integers(0, V, size=T, dtype=np.int64).astype(np.int32)
    noise = np.empty(T, dtype=np.float32)
    rn = _rng(master, _C_NOISE)
    for r0 in range(0, T, ROW_BLOCK * 16):
        r1 = min(T, r0 + ROW_BLOCK * 16)
        noise[r0:r1] = rn.standard_normal(r1 - r0, dtype=np.float32) * np.float32(noise_std)
    if tail_frac > 0.0:
        rt = _rng(master, _C_TAILS)
        n_tail = int(round(tail_frac * T))
        idx = rt.choice(T, size=n_tail, replace=False)
        sign = np.where(rt.random(n_tail) < 0.5, -1.0, 1.0).astype(np.float32)
        noise[idx] += sign * np.float32(tail_shift)
    rr = _rng(master, _C_REWARD)
    if reward_kind == "bernoulli":
        reward = (rr.random(R) < reward_p).astype(np.float32)
    elif reward_kind == "uniform":
        reward = rr.random(R).astype(np.float32)
    else:
        raise ValueError(reward_kind)
    return Batch(name=name, H=H, V=V, x=x, gamma=gamma, W=W, target=target,
                 resp_offsets=_offsets(lengths),
                 group_offsets=np.arange(0, R + 1, group_size, dtype=np.int64),
                 reward=reward, lag_noise=noise)


def tiny() -> Batch:
    """4 prompts x 4 responses, lengths uniform on {8..32}; H=128, V=1024.
    Lag noise N(0, 0.01) (added to the oracle logprob); rewards Bernoulli(0.5)."""
    lengths = _rng(0, _C_LENGTHS).integers(8, 33, size=16)
    return _assemble("tiny", 0, lengths, 4, 128, 1024, 0.01, "bernoulli", 0.5)


def qwen15b(with_W: bool = True, with_x: bool = True) -> Batch:
    """1.5B-shaped: H=1536, V=151936, 16 prompts x 8 responses with lengths
    uniform on {1024..8192} (about 590K tokens).  Lag noise N(0, 0.05)
    (lag 2-8); rewards Bernoulli(0.5)."""
    lengths = _rng(1, _C_LENGTHS).integers(1024, 8193, size=128)
    return _assemble("qwen15b", 1, lengths, 8, 1536, 151936, 0.05, "bernoulli", 0.5, with_W=with_W, with_x=with_x)


def qwen4b_lag64(with_W: bool = True, with_x: bool = True) -> Batch:
    """4B-shaped long context, lag 64: H=2560, V=151936, 8 prompts x 8
    responses of 16384 tokens.  Lag noise N(0, 0.2) with 1% of tokens shifted
    by +-3 (fair sign); rewards uniform on [0, 1)."""
    lengths = np.full(64, 16384, dtype=np.int64)
    return _assemble("qwen4b_lag64", 3, lengths, 8, 2560, 151936, 0.2, "uniform",
                     tail_frac=0.01, tail_shift=3.0, with_W=with_W, with_x=with_x)


def a3b30_head(with_W: bool = True, with_x: bool = True) -> Batch:
    """30B-A3B-shaped head: H=2048, V=151936, groups of 16 responses with
    lognormal lengths (median 2048, sigma 1, rounded, clipped to [1, 32768]),
    whole groups added until T >= 2**20; 0.1% of rows scaled by 20 before the
    bf16 rounding; rewards Bernoulli(0.3); lag noise N(0, 0.05)."""
    rl = _rng(4, _C_LENGTHS)
    lengths = []
    while sum(lengths) < (1 << 20):
        grp = np.clip(np.rint(rl.lognormal(math.log(2048.0), 1.0, size=16)), 1, 32768)
        lengths.extend(int(v) for v in grp)
    return _assemble("a3b30_head", 4, np.asarray(lengths, dtype=np.int64), 16, 2048, 151936,
                     0.05, "bernoulli", 0.3, outlier_frac=0.001, outlier_scale=20.0,
                     with_W=with_W, with_x=with_x)


def rows_only(master: int, child: int, T: int, H: int, V: int):
    """Standalone rows (x bits, target) from an independent stream: used as
    filler rows and as the fixed rows of the invariance sweep."""
    x = _normal_bf16(_rng(master, child), T, H, 1.0)
    tgt = _rng(master, child + 1).integers(0, V, size=T, dtype=np.int64).astype(np.int32)
    return x, tgt


@dataclasses.dataclass
class InvarianceSweep:
    """512 fixed rows evaluated inside batches of several sizes at random
    offsets among filler rows (1.5B shapes).  ``batches`` maps a label to a
    list of (row_ids, positions, batch_size): the fixed rows ``row_ids`` sit at
    ``positions`` of a batch of ``batch_size`` rows whose other rows are filler
    rows taken in order from the filler pool."""
    H: int
    V: int
    fixed_x: np.ndarray
    fixed_target: np.ndarray
    filler_x: np.ndarray
    filler_target: np.ndarray
    batches: dict


def invariance_sweep(n_fixed: int = 512, sizes=(1, 7, 64, 100, 200, 1024, 65536),
                     prefill_chunk: int = 2048,
                     H: int = 1536, V: int = 151936, n_filler: int = 65536) -> InvarianceSweep:
    master = 2
    fx, ft = rows_only(master, _C_X, n_fixed, H, V)
    flx, flt = rows_only(master, _C_FILLER, n_filler, H, V)
    rp = _rng(master, _C_PLACEMENT)
    batches = {}
    for B in list(sizes) + [("prefill", prefill_chunk)]:
        label = f"prefill{B[1]}" if isinstance(B, tuple) else f"batch{B}"
        B = B[1] if isinstance(B, tuple) else B
        per = n_fixed if B >= n_fixed else max(1, B // 2)
        plan = []
        for i0 in range(0, n_fixed, per):
            ids = np.arange(i0, min(n_fixed, i0 + per))
            pos = np.sort(rp.choice(B, size=len(ids), replace=False))
            plan.append((ids, pos, B))
        batches[label] = plan
    return InvarianceSweep(H=H, V=V, fixed_x=fx, fixed_target=ft, filler_x=flx,
                           filler_target=flt, batches=batches)


def compose_batch(sweep: InvarianceSweep, ids: np.ndarray, pos: np.ndarray, B: int):
    """Materialise one batch of the sweep: filler rows everywhere except the
    fixed rows ``ids`` at ``pos``."""
    nf = sweep.filler_x.shape[0]
    fill = np.arange(B) % nf
    x = sweep.filler_x[fill].copy()
    t = sweep.filler_target[fill].copy()
    x[pos] = sweep.fixed_x[ids]
    t[pos] = sweep.fixed_target[ids]
    return x, t


def older_version(master: int, x_bits: np.ndarray, gamma_bits: np.ndarray, W_bits: np.ndarray,
                  w_sigma: float, x_sigma: float = 0.0, gamma_sigma: float = 0.0):
    """The head at an older weight version, for the log-ratio decomposition:
    every element of W (and of x, gamma when their sigma is not 0) moved by
    an independent N(0, sigma) draw and rounded to bf16 again.  Draws come
    from the config's own stream (master seed, version child); W is drawn in
    ROW_BLOCK row blocks like the other tensors.  Returns (x, gamma, W) bits."""
    rng = _rng(master, _C_VERSION)

    def moved(bits, sigma):
        if sigma == 0.0:
            return bits
        a = bits.reshape(-1, bits.shape[-1]) if bits.ndim > 1 else bits.reshape(1, -1)
        out = np.empty_like(a)
        for r0 in range(0, a.shape[0], ROW_BLOCK):
            r1 = min(a.shape[0], r0 + ROW_BLOCK)
            d = rng.standard_normal((r1 - r0, a.shape[1]), dtype=np.float32) * np.float32(sigma)
            out[r0:r1] = f32_to_bf16_bits(bf16_bits_to_f32(a[r0:r1]) + d)
        return out.reshape(bits.shape)

    return moved(x_bits, x_sigma), moved(gamma_bits, gamma_sigma), moved(W_bits, w_sigma)


def zipf_targets(master: int, T: int, V: int, exponent: float = 1.1, top_share: float = 0.3,
                 chunk: int = 32768) -> np.ndarray:
    """Target token ids with a Zipfian frequency profile, as natural text has:
    id r (in a seeded random order of the vocabulary) is drawn with weight
    (r + 1)^-exponent, and in every chunk of `chunk` consecutive tokens a
    fraction top_share of the positions (a seeded random subset) holds the
    most frequent id, as end-of-text or newline tokens do.  int32 [T]."""
    rng = _rng(master, _C_TARGET)
    order = rng.permutation(V)
    w = (np.arange(V, dtype=np.float64) + 1.0) ** -exponent
    t = order[rng.choice(V, size=T, p=w / w.sum())].astype(np.int32)
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        k = rng.choice(c1 - c0, size=int(top_share * (c1 - c0)), replace=False)
        t[c0 + k] = order[0]
    return t


CONFIGS = {
    "tiny": tiny,
    "qwen15b": qwen15b,
    "qwen4b_lag64": qwen4b_lag64,
    "a3b30_head": a3b30_head,
}
