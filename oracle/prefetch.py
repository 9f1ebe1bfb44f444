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

Readings (the page fixes these only in part):

* Ranges.  Request r's tokens [0, L_r) are cut into ranges of R tokens, x = 0, 1, ...
  (one workgroup each on the GPU).
* Qualifying tokens.  s, with float32 score > float32 theta_r (strict; a NaN threshold passes
  nothing), whose host index h = req_to_host[key_begin_r + s] lies in [0, N_H) and is not
  resident (HostTokenToGPU[h] = INF) before the prefetch.  demand_r counts them.  A range asks
  for places for its first 128 qualifying tokens in token order (its candidates).
* Cap.  Request r may move c_r = min(cap, ceil(L_r / cap_div), N_G) rows (the page's bound in
  proportion to the context).  When the caps of all requests add up to C > F, the number of
  free slots, each becomes floor(c_r * F / C), so that every request keeps a share of the free
  slots.
* Places.  The free slots before the prefetch, ascending, form a list.  Request r owns the c_r
  entries from O_r = sum over r' < r of c_r'.  Its ranges claim them first come, first served
  (the page's prefetch counter, one per request): a claim takes the next free places of the
  request, in the token order of the claiming range.  So when a request's candidates fit its
  cap, every one of them moves, and otherwise exactly c_r do, each range's moved tokens being a
  token-order prefix of its candidates; the places taken are always the request's first
  entries; which candidate gets which of them depends on timing.  `range_prefetch` returns the
  canonical outcome (candidates in request, then token order, take the places in order) with
  what defines the set of valid outcomes.
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


def request_caps(key_len, cap, cap_div, n_free, n_gpu):
    """(c_r before scaling, c_r after scaling) per request (module notes: Cap)."""
    c = [0 if L <= 0 else min(cap, -(-int(L) // cap_div), n_gpu) for L in key_len]
    total = sum(c)
    if total > n_free:
        return c, [ci * n_free // total for ci in c]
    return c, list(c)


def prefetch_candidates(scores, theta, key_begin, key_len, req_to_host, state, range_len,
                        per_range=128):
    """Per request: the qualifying tokens (all of them) and each range's candidates (its first
    per_range qualifying tokens), as {range: [(token, host index), ...]}, token order."""
    theta32 = np.asarray(theta, np.float32)
    qual, cand = [], []
    for r in range(len(key_len)):
        L = max(int(key_len[r]), 0)
        s32 = np.asarray(scores[r][:L], np.float64).astype(np.float32)
        q, c = [], {}
        for s in range(L):
            if not s32[s] > theta32[r]:
                continue
            h = int(req_to_host[int(key_begin[r]) + s])
            if h < 0 or h >= state.n_host or state.host_to_gpu[h] != INF:
                continue
            q.append((s, h))
            lst = c.setdefault(s // range_len, [])
            if len(lst) < per_range:
                lst.append((s, h))
        qual.append(q)
        cand.append(c)
    return qual, cand


def range_prefetch(scores, theta, key_begin, key_len, req_to_host, state, host_kv, cap, cap_div,
                   range_len, per_range=128):
    """The canonical outcome of the prefetch (module notes) and what defines the valid ones.

    scores: per request, the scores of tokens [0, L_r) (float64, cast to float32 for the test);
    theta: per request threshold (cast to float32).  state is not modified.
    Returns (new_state, moved, demand, info): moved lists (request, token, host index, slot) in
    the canonical order; demand[r] counts the qualifying tokens of request r; info holds
    'free_list', 'cap' (scaled c_r), 'offset' (O_r) and 'cand' (per request, range -> the
    range's candidates)."""
    free_list = np.flatnonzero(state.free == 1)
    qual, cand = prefetch_candidates(scores, theta, key_begin, key_len, req_to_host, state,
                                     range_len, per_range)
    _, caps = request_caps(key_len, cap, cap_div, len(free_list), state.n_gpu)
    offsets = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64) if len(caps) else []
    new = state.copy()
    moved = []
    for r in range(len(key_len)):
        flat = [t for x in sorted(cand[r]) for t in cand[r][x]]
        for i, (s, h) in enumerate(flat[:caps[r]]):
            slot = int(free_list[offsets[r] + i])
            new.free[slot] = 0
            new.to_host[slot] = h
            new.host_to_gpu[h] = slot
            new.priority[slot] = 0
            new.gpu_kv[slot] = host_kv[h]
            moved.append((r, s, h, slot))
    demand = np.array([len(q) for q in qual], np.int64)
    info = dict(free_list=free_list, cap=caps, offset=offsets, cand=cand)
    return new, moved, demand, info


def check_prefetch_outcome(before, after, host_kv, key_begin, req_to_host, info, demand_got=None,
                           demand=None, slot_order=True):
    """Raises AssertionError unless `after` is a valid outcome of the prefetch from `before`
    (module notes: Places): per request, min(#candidates, c_r) rows moved, each range's a
    token-order prefix of its candidates with ascending slots, into exactly the request's first
    places; maps, priority 0 and rows set; nothing else changed.  slot_order=False skips the
    ascending slots within a range (for a reference computed with other ranges than the run's,
    where only the moved set, the places and the rows are comparable)."""
    new_slots = np.flatnonzero((before.free == 1) & (after.free == 0))
    assert not np.flatnonzero((before.free == 0) & (after.free == 1)).size, "a slot was freed"
    where = {}
    for r, c in enumerate(info["cand"]):
        for x, lst in c.items():
            for s, h in lst:
                where[h] = (r, x, s)
    got = {}
    for sl in new_slots:
        h = int(after.to_host[sl])
        assert h in where, "slot %d holds a host index that is no candidate" % sl
        assert after.host_to_gpu[h] == sl and after.priority[sl] == 0, "maps of slot %d" % sl
        assert np.array_equal(after.gpu_kv[sl], host_kv[h]), "row of slot %d" % sl
        r, x, s = where[h]
        got.setdefault(r, {}).setdefault(x, []).append((s, int(sl)))
    fl = info["free_list"]
    for r, c in enumerate(info["cand"]):
        n_cand = sum(len(v) for v in c.values())
        rows = got.get(r, {})
        n_moved = sum(len(v) for v in rows.values())
        assert n_moved == min(n_cand, info["cap"][r]), "request %d moved %d" % (r, n_moved)
        slots = sorted(sl for v in rows.values() for _, sl in v)
        o = int(info["offset"][r]) if n_moved else 0
        assert slots == sorted(int(v) for v in fl[o:o + n_moved]), "request %d places" % r
        for x, v in rows.items():
            v.sort()
            assert [s for s, _ in v] == [s for s, _ in c[x][:len(v)]], "range %d/%d prefix" % (r, x)
            assert not slot_order or [sl for _, sl in v] == sorted(sl for _, sl in v), \
                "range %d/%d slot order" % (r, x)
    keep = np.ones(before.n_gpu, bool)
    keep[new_slots] = False
    for name in ("free", "priority", "to_host", "indices_buf"):
        assert np.array_equal(getattr(after, name)[keep], getattr(before, name)[keep]), name
    assert np.array_equal(after.gpu_kv[keep], before.gpu_kv[keep]), "gpu_kv outside the new slots"
    moved_h = after.to_host[new_slots]
    hk = np.ones(before.n_host, bool)
    hk[moved_h] = False
    assert np.array_equal(after.host_to_gpu[hk], before.host_to_gpu[hk]), "host_to_gpu"
    if demand is not None:
        assert np.array_equal(np.asarray(demand_got), np.asarray(demand)), "demand"


def decode_step_prefetched(q, w, k, k_scale, key_begin, key_len, req_to_host, state, host_kv,
                           topk_k, step_id, theta, cap, cap_div, range_len, reserve=0):
    """A whole decode step with the range prefetch ahead of the exact top-k and the guaranteed
    recall (§4 with §6.1 / §6.3), with the canonical prefetch outcome.  Returns (scores, idx,
    state after the prefetch, moved, demand, info, final state, PoolStepResult)."""
    scores = index_scores(q, w, k, k_scale, key_begin, key_len)
    mid, moved, demand, info = range_prefetch(scores, theta, key_begin, key_len, req_to_host,
                                              state, host_kv, cap, cap_div, range_len)
    idx = topk_rows(scores, topk_k)
    final, res = pool_step(mid, host_kv, idx, key_begin, req_to_host, step_id, reserve=reserve)
    return scores, idx, mid, moved, demand, info, final, res
