"""Threshold prefetch over token ranges, as one scoring launch with a copy stage does it
(oracle; test infrastructure only).

ECHO page §6.1: while the indexer is still scoring, tokens whose score is above a threshold
predicted for the request's k-th score are moved from host memory into the GPU pool ahead of
the exact top-k.  How many move is bounded in proportion to the context, so that the copies do
not slow the indexer.  The guaranteed recall afterwards fills whatever is still missing, so the
selection and the rows attention reads are the same with or without prefetch (lossless).
ECHO page §6.3: the indexer kernel does this in a single launch; each part of the key range is
scored, tested against the threshold, and the passing tokens reach a copy stage through a
bounded queue.

Readings (the page fixes none of these; they are the plainest ones that make the result a
function of the inputs alone):

* Ranges.  Request r's tokens [0, L_r) are cut into ranges of R tokens, x = 0, 1, ...
  (one workgroup each on the GPU).  n_ranges_r = ceil(L_r / R).
* Cap.  Request r may move cap_r = min(cap, ceil(L_r / cap_div)) rows (the page's bound in
  proportion to the context), at most max_per_range (128) per range:
  c_r = min(cap_r, 128 * n_ranges_r).  Its ranges split c_r evenly: range x moves at most
  m_x = floor((x + 1) c_r / n_ranges_r) - floor(x c_r / n_ranges_r) rows (the shares differ by
  at most one and add up to c_r; a range's share is 0 when c_r < n_ranges_r).
* Qualifying tokens.  s in the range, ascending, with float32 score > float32 theta_r (strict;
  a NaN threshold passes nothing), whose host index h = req_to_host[key_begin_r + s] lies in
  [0, N_H) and is not resident (HostTokenToGPU[h] = INF) before the prefetch.  The first
  m_x qualifying tokens of each range move; demand_r counts all qualifying tokens.
* Slots.  The pool's free slots before the prefetch, ascending, form a list F.  Request r owns
  c_r entries from O_r = sum over r' < r of c_r'; its range x owns the m_x entries from
  O_r + floor(x c_r / n_ranges_r), and its i-th moved token takes entry i of those if the list
  is that long (otherwise it does not move).
* A moved token: Free = 0, ToHost = h, HostToGPU[h] = slot, priority 0 (below every step
  stamp, so it goes first when space is short and it was not selected), and its row is copied
  from the host backup bit for bit.  Nothing is evicted.

Pinned by a worked example computed by hand (tests/golden/range_prefetch_example.txt), the
special cases that reduce to closed forms (threshold +inf or NaN: nothing moves; threshold
-inf with caps and free slots to spare: every non-resident token moves), the invariant checker
of the pool, and the page's losslessness claim (a whole step with the prefetch selects the same
tokens and makes the same rows resident as a step without it).
"""

import numpy as np

from .pool import INF, PoolState
from .scores import index_scores
from .topk import topk_rows
from .pool import pool_step


def request_cap(L, cap, cap_div, range_len, max_per_range=128):
    """c_r: rows a request of L tokens may move over all its ranges (module notes: Cap)."""
    if L <= 0:
        return 0
    n_ranges = -(-L // range_len)
    return min(cap, -(-L // cap_div), max_per_range * n_ranges)


def range_share(c, n_ranges, x):
    """(first entry, count) of range x's share of a request's c rows (module notes)."""
    first = x * c // n_ranges
    return first, (x + 1) * c // n_ranges - first


def range_prefetch(scores, theta, key_begin, key_len, req_to_host, state, host_kv, cap, cap_div,
                   range_len, max_per_range=128):
    """Moves rows ahead of the top-k as described in the module notes.

    scores: per request, the scores of tokens [0, L_r) (float64, cast to float32 for the test);
    theta: per request threshold (cast to float32).  state is not modified.
    Returns (new_state, moved, demand): moved lists (request, token, host index, slot) in the
    order the slots were taken; demand[r] counts the qualifying tokens of request r."""
    n = len(key_len)
    theta32 = np.asarray(theta, np.float32)
    free_list = np.flatnonzero(state.free == 1)
    new = state.copy()
    moved, demand = [], np.zeros(n, np.int64)
    offset = 0
    for r in range(n):
        L = max(int(key_len[r]), 0)
        c = request_cap(L, cap, cap_div, range_len, max_per_range)
        n_ranges = -(-L // range_len) if L > 0 else 0
        s32 = np.asarray(scores[r][:L], np.float64).astype(np.float32)
        for x in range(n_ranges):
            first, share = range_share(c, n_ranges, x)
            taken = 0
            for s in range(x * range_len, min(L, (x + 1) * range_len)):
                if not s32[s] > theta32[r]:
                    continue
                h = int(req_to_host[int(key_begin[r]) + s])
                if h < 0 or h >= state.n_host or state.host_to_gpu[h] != INF:
                    continue
                demand[r] += 1
                entry = offset + first + taken
                if taken < share and entry < len(free_list):
                    slot = int(free_list[entry])
                    new.free[slot] = 0
                    new.to_host[slot] = h
                    new.host_to_gpu[h] = slot
                    new.priority[slot] = 0
                    new.gpu_kv[slot] = host_kv[h]
                    moved.append((r, s, h, slot))
                    taken += 1
        offset += c
    return new, moved, demand


def decode_step_prefetched(q, w, k, k_scale, key_begin, key_len, req_to_host, state, host_kv,
                           topk_k, step_id, theta, cap, cap_div, range_len, reserve=0):
    """A whole decode step with the range prefetch ahead of the exact top-k and the guaranteed
    recall (§4 with §6.1 / §6.3).  Returns (scores, idx, state after the prefetch, moved,
    demand, final state, PoolStepResult)."""
    scores = index_scores(q, w, k, k_scale, key_begin, key_len)
    mid, moved, demand = range_prefetch(scores, theta, key_begin, key_len, req_to_host, state,
                                        host_kv, cap, cap_div, range_len)
    idx = topk_rows(scores, topk_k)
    final, res = pool_step(mid, host_kv, idx, key_begin, req_to_host, step_id, reserve=reserve)
    return scores, idx, mid, moved, demand, final, res
