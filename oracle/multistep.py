"""Several decode steps in a row: new tokens and the EMA threshold (oracle; test infrastructure only).

ECHO page §2 (offload: a token's latent row is backed up to host memory when it is generated,
which is why eviction never moves data), §5.2 (allocate serves newly generated KV as well as
recalled tokens) and §6.1 (the k-th largest score of a layer is predicted for the next decode
step by an exponential moving average, s_hat(t+1) = alpha * s_hat(t) + (1 - alpha) * s(t) with
alpha = 0.5, and tokens scoring above the prediction are prefetched while the indexer runs; the
guaranteed recall afterwards keeps the selection lossless).

Readings where the page is silent:

* Order inside a step: every request first appends its new token, then its query scores every
  cached token, the new one included.
* Append: the token's indexer key (and its key scale, if keys carry scales) goes to the end of
  the request's key range, its host index (chosen by the caller; not resident) to req_to_host,
  its latent row to that host row (write-through) and into a GPU slot.  The slot comes from the
  canonical allocate of the pool step with the new tokens as the misses, in request order,
  evicting the lowest (priority, slot) when no slot is free; nothing is protected; the slot's
  priority is the step stamp.  The row is placed from the token's own copy (equal to the host
  row just written).  A request whose key range is full appends nothing and the step reports
  ST_CACHE_FULL.
* s(t) of a request is the smallest score among its selected tokens: the k-th largest when the
  request holds at least k tokens, its smallest score otherwise.
* The first step has no estimate.  The estimate is NaN then: no score exceeds it, so nothing is
  prefetched, and the first update sets it to s(0).  A request with no tokens keeps its
  estimate.  The update is computed exactly here (float64 on float32 inputs, alpha = 0.5 makes
  every product exact); the library rounds to float32.
* Prefetch only moves rows earlier.  So the oracle's steps are the ones without prefetch, and a
  loop with prefetch must select the same tokens and hold the same rows for them.

Pinned by: the EMA recursion against its closed form (a geometrically weighted sum of the s(i)),
constant and alternating sequences, the k-th score against a full sort, a hand-worked append on
a tiny pool, the pool invariant checker after every step, and a one-step loop equal to
decode_step after the appends.
"""

from dataclasses import dataclass

import numpy as np

from .pool import pool_step
from .scores import index_scores
from .topk import topk_rows

ST_CACHE_FULL = 8


@dataclass
class KeyCache:
    """The indexer K cache and token -> host map of B requests; request r owns rows
    key_begin[r] .. key_begin[r] + capacity - 1, of which the first key_len[r] are in use."""
    k: np.ndarray            # uint8 [n_k, 128]
    k_scale: object          # float32 [n_k] or None
    key_begin: np.ndarray    # int64 [B]
    key_len: np.ndarray      # int32 [B]
    req_to_host: np.ndarray  # int32 [n_k]
    capacity: int

    def copy(self):
        return KeyCache(self.k.copy(), None if self.k_scale is None else self.k_scale.copy(),
                        self.key_begin.copy(), self.key_len.copy(), self.req_to_host.copy(),
                        self.capacity)


def kth_scores(scores, idx):
    """s(t) per request: the smallest score among the selected tokens (NaN if none).
    scores: list of float64 rows; idx: int [B, k] selected token indices, -1 padded."""
    out = np.full(len(scores), np.nan)
    for r, row in enumerate(scores):
        sel = idx[r][idx[r] >= 0]
        if len(sel):
            out[r] = np.min(np.asarray(row)[sel])
    return out


def ema_update(theta, kth, alpha):
    """Next-step estimate of the k-th score (§6.1); NaN estimate = none yet."""
    theta = np.asarray(theta, np.float64)
    kth = np.asarray(kth, np.float64)
    out = alpha * theta + (1.0 - alpha) * kth
    out = np.where(np.isnan(theta), kth, out)
    return np.where(np.isnan(kth), theta, out)


def append_tokens(cache, state, host_kv, new_k, new_scale, new_kv, new_host, step_id):
    """One new token per request.  Returns (cache, state, host_kv, slot, status), all new
    objects: slot[r] is the GPU slot the new token of request r got (-1 if none)."""
    cache = cache.copy()
    host_kv = host_kv.copy()
    n_rows = len(cache.key_len)
    pos = np.full((n_rows, 1), -1, np.int64)
    status = 0
    for r in range(n_rows):
        p = int(cache.key_len[r])
        if p >= cache.capacity:
            status |= ST_CACHE_FULL
            continue
        row = int(cache.key_begin[r]) + p
        cache.k[row] = new_k[r]
        if cache.k_scale is not None:
            cache.k_scale[row] = new_scale[r]
        cache.req_to_host[row] = new_host[r]
        cache.key_len[r] = p + 1
        pos[r, 0] = p
        h = int(new_host[r])
        if 0 <= h < len(host_kv):
            host_kv[h] = new_kv[r]                       # write-through backup
    new_state, res = pool_step(state, host_kv, pos, cache.key_begin, cache.req_to_host, step_id)
    slot = res.topk_slot[:, 0].copy() if res.status == 0 else np.full(n_rows, -1, np.int32)
    return cache, new_state, host_kv, slot, status | res.status


@dataclass
class StepRecord:
    scores: list             # float64 rows, one per request
    idx: np.ndarray          # int32 [B, k]
    kth: np.ndarray          # float64 [B]
    theta_used: np.ndarray   # float64 [B]: the estimate this step's prefetch compared against
    theta_next: np.ndarray   # float64 [B]
    new_slot: np.ndarray     # int32 [B]
    state: object            # PoolState after the step
    result: object           # PoolStepResult of the guaranteed recall
    append_status: int


def decode_loop(cache, state, host_kv, steps, topk_k, alpha=0.5, theta0=None, reserve=0):
    """Runs the steps in order.  steps: list of dicts with q [B,64,128], w [B,64], new_k [B,128],
    new_scale [B] or None, new_kv [B,576], new_host [B], step_id.  reserve: free slots each
    step's guaranteed recall leaves for the next step's prefetch (pool.pool_step).  Returns
    (cache, state, host_kv, [StepRecord])."""
    n_rows = len(cache.key_len)
    theta = np.full(n_rows, np.nan) if theta0 is None else np.asarray(theta0, np.float64)
    records = []
    for st in steps:
        cache, state, host_kv, slot, ast = append_tokens(
            cache, state, host_kv, st["new_k"], st.get("new_scale"), st["new_kv"], st["new_host"],
            st["step_id"])
        scores = index_scores(st["q"], st["w"], cache.k, cache.k_scale, cache.key_begin,
                              cache.key_len)
        idx = topk_rows(scores, topk_k)
        state, res = pool_step(state, host_kv, idx, cache.key_begin, cache.req_to_host,
                               st["step_id"], reserve)
        kth = kth_scores(scores, idx)
        nxt = ema_update(theta, kth, alpha)
        records.append(StepRecord(scores, idx, kth, theta, nxt, slot, state, res, ast))
        theta = nxt
    return cache, state, host_kv, records
