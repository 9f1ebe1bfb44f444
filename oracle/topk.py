"""Exact top-k, the prefetch threshold, and the radix threshold bin (oracle; test infrastructure only).

ECHO page §2: the indexer's scores feed an exact top-k (k = 2048 in V3.2);
every score must exist before the set is known, which is the global
dependency §3.4 describes.

Readings where the page is silent:

* Ties at the k-th score go to the lower token index, so the selected set is
  unique under the order (score descending, index ascending).
* Scores compare by value: -0.0 equals +0.0.
* Rows shorter than k select all their tokens; the output is padded with -1.
* The output lists the selected token indices in ascending order (the set is
  what matters; ascending order is the library's documented layout).

The top-k is decided in whatever precision the scores arrive in: float64
oracle scores, or the float32 values a test generated for both sides.

Pinned by brute force over all subsets on tiny rows, and by the invariants
(count, every selected >= every unselected, boundary ties to lower index).
"""

import math

import numpy as np


def topk_row(scores, k):
    """Indices of the k highest scores of one row, ascending, -1 padded to k."""
    s = np.asarray(scores)
    n = s.shape[0]
    out = np.full(k, -1, dtype=np.int32)
    m = min(k, n)
    if m == 0:
        return out
    # primary key: score descending; secondary key: index ascending (lexsort
    # sorts by the last key first and is stable)
    order = np.lexsort((np.arange(n), -s))
    out[:m] = np.sort(order[:m])
    return out


def topk_rows(rows, k):
    """topk_row over a list of rows -> int32 [n_rows, k]."""
    return np.stack([topk_row(r, k) for r in rows]) if len(rows) else np.zeros((0, k), np.int32)


def sample_threshold(scores, n_sample=4096, percentile=95.0):
    """Prefetch threshold of one request from a fixed sample of its scores.

    The page (§6.1) predicts the k-th score with an EMA over decode steps; a
    single synthetic decode step has no history, so the stand-in threshold is
    the nearest-rank `percentile` of the scores at positions
    floor(i * L / n_sample), i < n_sample.  Nearest rank: the
    ceil(percentile/100 * n_sample)-th smallest sampled score.  Only which
    rows move early depends on it; the selected set does not (§6.1, the
    guaranteed recall makes prefetch lossless).  Returns +inf for L == 0.
    """
    s = np.asarray(scores)
    n = s.shape[0]
    if n == 0:
        return math.inf
    pos = (np.arange(n_sample, dtype=np.int64) * n) // n_sample
    sample = np.sort(s[pos])
    rank = math.ceil(percentile / 100.0 * n_sample)      # 1-based
    return sample[rank - 1]


def f32_order_key(x):
    """Order-preserving map of float32 values to uint32 (-0.0 folded onto +0.0)."""
    x = np.asarray(x, dtype=np.float32) + np.float32(0.0)   # -0.0 + 0.0 = +0.0
    b = x.view(np.uint32).astype(np.uint64)
    neg = (b >> 31) == 1
    key = np.where(neg, (~b) & 0xFFFFFFFF, b | 0x80000000)
    return key.astype(np.uint32)


def threshold_bin(scores_f32, k):
    """The threshold bin of the page's 8-bit radix histogram (§6.2).

    Scores are mapped by the top 8 bits of their order-preserving key into 256
    bins S_0..S_255.  The j highest bins are the largest group whose total is
    <= k; the next bin down, 255 - j, is the threshold bin.  Returns
    (hist, j, threshold_bin_index or -1 when every bin fits).
    """
    bins = (f32_order_key(scores_f32) >> 24).astype(np.int64)
    hist = np.bincount(bins, minlength=256)
    total = 0
    j = 0
    while j < 256 and total + hist[255 - j] <= k:
        total += hist[255 - j]
        j += 1
    return hist, j, (255 - j if j < 256 else -1)
