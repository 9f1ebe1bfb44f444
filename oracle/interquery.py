"""Inter-query prefetch for a chunked prefill with offloaded KV (oracle; test infrastructure only).

ECHO page §6.2: the indexer scores a prefill's query blocks in order, so the tokens block i
selected can be fetched while block i+1 is scored.  An exact top-k inside the indexer kernel
would slow it badly, so an approximate top-k yields a subset of each row's top-k for the
prefetch.  Every score is mapped by its top 8 bits to one of 256 bins S_0..S_255.  The j
highest bins whose total stays within k are taken whole, and the next bin down, 255 - j, is the
threshold bin, so S = S_{256-j} + ... + S_255 > k - S_{255-j}.  The smaller the threshold bin,
the closer the subset is to the whole top-k.  To shrink it, every score is first shifted by a
prediction of the k-th score: an EMA of the k-th score of the previous chunk's last token.  The
region of interest then sits where the bins are finest.  Whatever the subset misses, the
guaranteed recall fetches after the exact top-k, so the result is lossless.

Readings where the page is silent:

* Bins: the top 8 bits of the order-preserving key (sign-flipped, -0 folded onto +0) of the
  float32 shifted score fl32(s - shift), s the float32 score.  The subset of a row is the
  tokens whose bin is above the threshold bin; all its tokens when every bin fits within k.
* A query block is one prefill chunk (one call over its rows).  Its prefetch set is the union
  of its rows' subsets, and its guaranteed recall covers the union of its rows' exact top-k.
  Both unions are listed in ascending token order, in segments of 4096 consecutive token
  indices (segment s holds the union's tokens in [4096 s, 4096 s + 4096)).
* The shift of chunk 0 is 0 (no prediction yet).  After chunk c the estimate takes the k-th
  score of the chunk's last row, by the same EMA (alpha = 0.5) as the decode loop.  That k-th
  score is the smallest score that row selected.

Pinned by: the page's inequality and the subset's inclusion in the exact top-k (brute force
over random rows, shifts and ties), special cases (k >= L: the whole row; a constant row), the
threshold bin shrinking under the shift on normal scores, and the chunk loop's pool invariants
and losslessness.
"""

import numpy as np

from .multistep import ema_update, kth_scores
from .pool import pool_step
from .scores import index_scores
from .topk import f32_order_key, topk_rows

SEG = 4096


def approx_subset(scores_f32, k, shift):
    """(subset ascending int array, threshold-bin size, S) of one row (§6.2)."""
    s = np.asarray(scores_f32, np.float32)
    shifted = (s - np.float32(shift)).astype(np.float32)
    bins = (f32_order_key(shifted) >> 24).astype(np.int64)
    hist = np.bincount(bins, minlength=256)
    total, j = 0, 0
    while j < 256 and total + hist[255 - j] <= k:
        total += hist[255 - j]
        j += 1
    if j == 256:
        return np.arange(len(s)), 0, total
    thr = 255 - j
    return np.flatnonzero(bins > thr), int(hist[thr]), total


def union_segments(rows, n_keys):
    """The union of the given index lists (entries >= 0), as [ceil(n_keys / 4096), 4096] int32
    (segment s = the union's tokens in [4096 s, 4096 s + 4096), ascending, -1 padded) and the
    per-segment counts."""
    n_seg = max(1, -(-n_keys // SEG))
    mark = np.zeros(n_seg * SEG, bool)
    for r in rows:
        r = np.asarray(r)
        mark[r[r >= 0]] = True
    out = np.full((n_seg, SEG), -1, np.int32)
    cnt = np.zeros(n_seg, np.int32)
    for g in range(n_seg):
        toks = np.flatnonzero(mark[g * SEG:(g + 1) * SEG]) + g * SEG
        out[g, :len(toks)] = toks
        cnt[g] = len(toks)
    return out, cnt


def prefill_chunk_loop(q, w, k, req_to_host, state, host_kv, chunk, topk_k, step0,
                       alpha=0.5):
    """The chunked prefill of one request with its KV offloaded: query rows in chunks of
    `chunk`, row t seeing keys [0, t].  Per chunk: the approximate subsets under the current
    shift, the exact top-k, the guaranteed residency of the union of the exact top-k (pool step,
    stamp step0 + c), then the shift update.  Returns (state, [dict per chunk])."""
    n = q.shape[0]
    shift = 0.0
    theta = np.array([np.nan])
    recs = []
    for c, t0 in enumerate(range(0, n, chunk)):
        t1 = min(n, t0 + chunk)
        rows = [index_scores(q[t:t + 1], w[t:t + 1], k, None, np.array([0]), np.array([t + 1]))[0]
                for t in range(t0, t1)]
        sub = [approx_subset(np.asarray(r, np.float32), topk_k, shift) for r in rows]
        idx = topk_rows(rows, topk_k)
        n_keys = t1
        pre, pre_cnt = union_segments([s[0] for s in sub], n_keys)
        uni, uni_cnt = union_segments(list(idx), n_keys)
        state, res = pool_step(state, host_kv, uni, np.zeros(len(uni), np.int64), req_to_host,
                               step0 + c)
        kth_last = kth_scores([rows[-1]], idx[-1:])
        recs.append(dict(shift=shift, rows=rows, subsets=sub, idx=idx, prefetch=pre,
                         prefetch_cnt=pre_cnt, union=uni, union_cnt=uni_cnt, state=state,
                         result=res, kth_last=kth_last[0]))
        theta = ema_update(theta, kth_last, alpha)
        shift = float(np.float32(theta[0]))
    return state, recs
