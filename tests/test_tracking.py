"""Host-side tracking of per-update diagnostics against the oracle's
statistic (no GPU: the per-update values are given)."""
import numpy as np
import pytest

import oracle
from invariant_logprob_is_amd.tracking import UpdateTracker


def test_tracker_summary_matches_oracle_peak_median():
    rng = np.random.default_rng(3)
    rows = np.abs(rng.normal(0, 1e-3, (37, 3))) + 1e-6
    tr = UpdateTracker()
    for r in rows:
        tr.add(r)
    s = tr.summary()
    for q, name in enumerate(("k1", "k2", "k3")):
        med, peak, ratio = oracle.peak_median(rows[:, q])
        assert s[name] == {"median": med, "peak": peak, "peak_over_median": ratio}
    # a window (the last ten updates)
    s10 = tr.summary(slice(-10, None))
    assert s10["k3"]["median"] == oracle.peak_median(rows[-10:, 2])[0]
    np.testing.assert_array_equal(tr.values(), rows)


def test_tracker_empty_window_raises():
    tr = UpdateTracker()
    with pytest.raises(ValueError):
        tr.summary()
