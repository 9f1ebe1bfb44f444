"""Threshold prefetch: what the ECHO page fixes about it (oracle; test infrastructure only).

ECHO page §6.1 (intra-query prefetching): while the indexer is still scoring, tokens whose
score is above a per-layer prediction of the k-th largest score are moved from host memory into
the GPU pool ahead of the exact top-k.  Only tokens that are not already resident need a
transfer.  The number of prefetches is bounded by a counter whose limit grows in proportion to
the context length, so that the copies do not slow the indexer down.  The guaranteed recall
after the top-k fills whatever is still missing, so the prefetch never changes the result
(lossless).  ECHO page §6.3: the indexer kernel does this in one launch, the tokens passing the
threshold test reach a copy stage through a bounded queue; the page leaves open which passing
tokens win when the bound is reached (first come, first served).

The page therefore fixes a contract, not one outcome.  This module states that contract and
nothing more:

* Eligible tokens (§6.1): token s of request r with float32 score > float32 theta_r (strict;
  "scores above the estimate"; a NaN threshold passes nothing), whose host index
  h = req_to_host[key_begin_r + s] is a valid host row ([0, N_H)) that is not resident
  (HostTokenToGPU[h] = INF) when the prefetch starts.
* Bound (§6.1, the counter in proportion to the context): request r moves at most
  c_r = min(cap, ceil(L_r / cap_div), N_G) rows.  Reading: cap and cap_div are the two
  constants of that proportion; N_G because no request can use more slots than the pool has.
* Where rows go.  Reading (the page does not say where a prefetched row lands when space is
  short): a prefetch takes only slots that are free when it starts and never evicts; eviction
  belongs to the guaranteed recall's free operation (§5.2).
* A moved row (§5.1 metadata, §5.2 allocate): Free = 0, ToHost = h, HostToGPU[h] = slot, its row
  copied bit for bit from the host backup, priority 0.  Reading of the priority: below every
  step stamp, so a prefetched row that the step does not select is the first to go when space
  is short (§6.1 notes that wrongly prefetched rows only cost transfer time).
* Lossless (§6.1): after the same top-k and guaranteed recall, a step with any valid prefetch
  selects the same tokens, and every selected token's row is resident bit for bit.

`prefetch_eligible`, `prefetch_bound` and `check_prefetch_contract` state the contract;
`apply_prefetch` applies a list of (host index, slot) moves; `greedy_prefetch` gives one valid
outcome, the plainest: requests in order, each request's eligible tokens in token order up to
its bound, into the lowest free slots while any are left.  Which outcome a GPU run produces
depends on timing, so GPU results are checked against the contract, never against this one
outcome.

Pinned (tests/test_oracle_prefetch.py) by a worked example derived by hand, the thresholds that
reduce to closed forms (+inf and NaN move nothing; -inf with room to spare makes every token
resident), planted mistakes the contract checker must reject, and the page's losslessness over
random pools and random valid outcomes.
"""

import numpy as np

from .pool import INF


def prefetch_eligible(scores, theta, key_begin, key_len, req_to_host, state):
    """Per request, the eligible tokens as [(token, host index), ...] in token order.
    scores: per request the scores of tokens [0, L_r) (compared in float32, as the page's
    kernel compares its float scores); theta: per request threshold (float32)."""
    theta32 = np.asarray(theta, np.float32)
    out = []
    for r in range(len(key_len)):
        L = max(int(key_len[r]), 0)
        s32 = np.asarray(scores[r][:L], np.float64).astype(np.float32)
        lst = []
        for s in range(L):
            if not s32[s] > theta32[r]:
                continue
            h = int(req_to_host[int(key_begin[r]) + s])
            if 0 <= h < state.n_host and state.host_to_gpu[h] == INF:
                lst.append((s, h))
        out.append(lst)
    return out


def prefetch_bound(key_len, cap, cap_div, n_gpu):
    """c_r = min(cap, ceil(L_r / cap_div), N_G) per request (0 for an empty request)."""
    return [0 if L <= 0 else min(int(cap), -(-int(L) // int(cap_div)), int(n_gpu))
            for L in key_len]


def apply_prefetch(state, host_kv, moves):
    """The state after moving host rows h into slots (h, slot) as a prefetch does (module notes:
    a moved row).  state is not modified."""
    new = state.copy()
    for h, slot in moves:
        new.free[slot] = 0
        new.to_host[slot] = h
        new.host_to_gpu[h] = slot
        new.priority[slot] = 0
        new.gpu_kv[slot] = host_kv[h]
    return new


def greedy_prefetch(scores, theta, key_begin, key_len, req_to_host, state, host_kv, cap, cap_div):
    """One valid outcome (module notes).  Returns (new_state, moves [(request, token, host,
    slot)], eligible, bounds)."""
    elig = prefetch_eligible(scores, theta, key_begin, key_len, req_to_host, state)
    bound = prefetch_bound(key_len, cap, cap_div, state.n_gpu)
    free = list(np.flatnonzero(state.free == 1))
    moves = []
    for r, lst in enumerate(elig):
        for s, h in lst[:bound[r]]:
            if not free:
                break
            moves.append((r, s, h, int(free.pop(0))))
    new = apply_prefetch(state, host_kv, [(h, sl) for _, _, h, sl in moves])
    return new, moves, elig, bound


def check_prefetch_contract(before, after, host_kv, eligible, bound):
    """Raises AssertionError unless `after` follows from `before` by a prefetch the page allows
    (module notes).  eligible: prefetch_eligible(...) against `before`; bound: prefetch_bound(...).
    Returns the number of rows moved per request."""
    assert not np.flatnonzero((before.free == 0) & (after.free == 1)).size, "a slot was freed"
    new_slots = np.flatnonzero((before.free == 1) & (after.free == 0))
    owner = {h: r for r, lst in enumerate(eligible) for _, h in lst}
    per_req = np.zeros(len(eligible), np.int64)
    for sl in new_slots:
        h = int(after.to_host[sl])
        assert h in owner, "slot %d holds host row %d, which was not eligible" % (sl, h)
        assert after.host_to_gpu[h] == sl, "HostTokenToGPU of host row %d" % h
        assert after.priority[sl] == 0, "priority of prefetched slot %d" % sl
        assert np.array_equal(after.gpu_kv[sl], host_kv[h]), "row of slot %d" % sl
        per_req[owner[h]] += 1
    for r, n in enumerate(per_req):
        assert n <= bound[r], "request %d moved %d rows, above its bound %d" % (r, n, bound[r])
    keep = np.ones(before.n_gpu, bool)
    keep[new_slots] = False
    for name in ("free", "priority", "to_host", "gpu_kv"):
        assert np.array_equal(getattr(after, name)[keep], getattr(before, name)[keep]), \
            "%s changed outside the prefetched slots" % name
    assert np.array_equal(after.indices_buf, before.indices_buf), "indices_buf changed"
    hk = np.ones(before.n_host, bool)
    hk[after.to_host[new_slots]] = False
    assert np.array_equal(after.host_to_gpu[hk], before.host_to_gpu[hk]), \
        "HostTokenToGPU changed for a row that was not prefetched"
    return per_req
