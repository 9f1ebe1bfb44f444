"""Pins of the oracle's exact top-k, prefetch threshold and radix threshold bin."""

import itertools

import numpy as np
import pytest

from oracle import topk_row, sample_threshold, threshold_bin


def _brute_force_topk(s, k):
    """The unique subset of size min(k, n) in which every member beats every
    non-member: higher score, or an equal score and a lower index."""
    n = len(s)
    m = min(k, n)
    found = []
    for sub in itertools.combinations(range(n), m):
        inside = set(sub)
        ok = all(s[a] > s[b] or (s[a] == s[b] and a < b)
                 for a in inside for b in range(n) if b not in inside)
        if ok:
            found.append(sub)
    assert len(found) == 1
    return list(found[0])


@pytest.mark.parametrize("n,k", [(1, 1), (5, 2), (6, 3), (8, 4), (7, 7), (3, 5), (8, 1)])
def test_brute_force_tiny(n, k):
    rng = np.random.default_rng(n * 31 + k)
    for trial in range(30):
        s = rng.integers(-2, 3, n).astype(np.float64)      # many ties
        if trial % 3 == 0:
            s = s * 0.0                                     # includes -0.0 and +0.0
            s[rng.random(n) < 0.5] *= -1
        got = topk_row(s, k)
        want = _brute_force_topk(s, k)
        assert got[:len(want)].tolist() == want
        assert (got[len(want):] == -1).all()


def test_invariants_medium_with_ties():
    rng = np.random.default_rng(11)
    for n, k in [(1000, 100), (4096, 256), (5000, 2048), (300, 2048)]:
        s = np.round(rng.standard_normal(n).astype(np.float32) * 3) / 3
        idx = topk_row(s, k)
        m = min(n, k)
        sel = idx[:m]
        assert (idx[m:] == -1).all()
        assert len(set(sel.tolist())) == m and (np.diff(sel) > 0).all()
        mask = np.zeros(n, bool)
        mask[sel] = True
        if m < n:
            lo, hi = s[mask].min(), s[~mask].max()
            assert lo >= hi
            if lo == hi:   # boundary ties: every selected tied index < every unselected one
                assert np.flatnonzero(mask & (s == lo)).max() < np.flatnonzero(~mask & (s == lo)).min()


def test_signed_zero_equal():
    s = np.array([-0.0, 0.0, -0.0, 0.0], np.float32)
    assert topk_row(s, 2).tolist() == [0, 1]


def test_empty_and_short_rows():
    assert topk_row(np.zeros(0), 4).tolist() == [-1, -1, -1, -1]
    assert topk_row(np.array([3.0, 1.0]), 4).tolist() == [0, 1, -1, -1]


def test_sample_threshold_is_nearest_rank_percentile():
    rng = np.random.default_rng(12)
    for n in [4096, 10000, 131072, 1000]:
        s = rng.standard_normal(n)
        pos = (np.arange(4096) * n) // 4096
        want = np.percentile(s[pos], 95, method="inverted_cdf")
        assert sample_threshold(s, 4096, 95.0) == want
    # the 205th largest of 4096 samples
    s = np.arange(4096, dtype=np.float64)
    assert sample_threshold(s) == 4096 - 205


def test_threshold_bin_inequality():
    # the page's inequality (section 6.2): with j top bins summing to <= k and
    # the next bin S_{255-j} overflowing, their total S satisfies S > k - S_{255-j}
    rng = np.random.default_rng(13)
    for n, k in [(65536, 2048), (20000, 2048), (5000, 256)]:
        s = rng.standard_normal(n).astype(np.float32) * rng.uniform(0.1, 5)
        hist, j, tb = threshold_bin(s, k)
        S = hist[256 - j:].sum()
        assert S <= k and tb >= 0
        assert S > k - hist[tb]
        # every score in the j top bins is in the exact top-k
        top = set(topk_row(s, k).tolist())
        from oracle.topk import f32_order_key
        in_top_bins = np.flatnonzero((f32_order_key(s) >> 24) > tb)
        assert set(in_top_bins.tolist()) <= top
