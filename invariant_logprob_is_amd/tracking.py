"""Tracking of per-update diagnostics over a run of updates.

The pages judge a run by two statistics of a per-update diagnostic: the
median of the rollout-to-learner KL over a window of updates ([P2] "Keep
throughput, lag and quality conditions separate": the median KL of the first
and the last thousand updates), and the peak of the per-update D3 over its
median ([P3] Fig. 2 caption; [P2] "Only one probability gap comes from old
weights").  The per-update values come from the library (rz_kl, or the kl
output of rz_learner_step) and stay on the device until read; this class only
collects the scalars and reduces them on the host, which is not part of the
hot path.
"""
from __future__ import annotations

import numpy as np

__all__ = ["UpdateTracker"]

_NAMES = ("k1", "k2", "k3")


class UpdateTracker:
    """Collects (k1, k2, k3) per update; k3 is D3.

    add() takes the [3] fp64 tensor (or any 3-sequence) of one update.
    Values are copied to the host lazily, in batches, by summary()."""

    def __init__(self):
        self._pending = []
        self._rows = []

    def add(self, kl3) -> None:
        self._pending.append(kl3)

    def _flush(self) -> None:
        for v in self._pending:
            a = v.detach().to("cpu").numpy() if hasattr(v, "detach") else np.asarray(v)
            self._rows.append(np.asarray(a, np.float64).reshape(3))
        self._pending.clear()

    def values(self) -> np.ndarray:
        """[n_updates, 3] float64: k1, k2, k3 per update, in order."""
        self._flush()
        return np.array(self._rows, np.float64).reshape(-1, 3)

    def summary(self, window: slice | None = None) -> dict:
        """Per estimator over the updates in `window` (all by default):
        median, peak and peak / median (numpy's median: the mean of the
        middle two for an even count)."""
        v = self.values()
        if window is not None:
            v = v[window]
        if v.shape[0] == 0:
            raise ValueError("no updates recorded in the window")
        out = {}
        for q, name in enumerate(_NAMES):
            med = float(np.median(v[:, q]))
            peak = float(np.max(v[:, q]))
            out[name] = {"median": med, "peak": peak, "peak_over_median": peak / med}
        return out
