"""The fused prefetch kernel's documented policy, as a CPU model for its tests.

This is NOT the oracle.  The ECHO page (§6.1, §6.3) fixes only the contract that
oracle/prefetch.py checks: moved rows are non-resident tokens scoring strictly above the
threshold, at most a bound in proportion to the context per request, into free slots, with
priority 0 and rows equal to the host backup, nothing evicted, and a step with prefetch selecting
and keeping resident what a step without it does.  Which of the eligible tokens move, and into
which free slots, is left open there.  The library's fused scoring launch
(echo_index_scores_fused, and echo_decode_select with ECHO_PREFETCH_FUSED) makes these choices,
and echo.h documents them; this module writes that documented choice out so the tests can check
the kernel against what it promises, on top of the page's contract:

* Ranges.  Request r's tokens [0, L_r) are cut into ranges of R tokens (one workgroup each).
* Candidates.  A range asks for places for its first 128 eligible tokens in token order.
* Cap.  c_r = min(cap, ceil(L_r / cap_div), N_G); when the caps add up to C > F (the free
  slots), each becomes floor(c_r * F / C).
* Places.  The free slots before the prefetch, ascending, form a list; request r owns the c_r
  entries from O_r = sum over r' < r of c_r', and its ranges claim them first come, first
  served.  When a request's candidates fit its cap all of them move; otherwise exactly c_r do,
  each range's moved tokens a token-order prefix of its candidates; the places taken are the
  request's first entries.

`policy_prefetch` returns the canonical outcome (candidates in request, then token order, take
the places in order) and what defines the valid ones; `check_policy_outcome` accepts every
valid one.  Pinned by a worked example derived by hand
(tests/golden/range_prefetch_policy_example.txt) and planted mistakes
(tests/test_prefetch_policy.py).
"""

import numpy as np

import oracle
from oracle.pool import INF


def request_caps(key_len, cap, cap_div, n_free, n_gpu):
    """(c_r before scaling, c_r after scaling) per request (module notes: Cap)."""
    c = [0 if L <= 0 else min(cap, -(-int(L) // cap_div), n_gpu) for L in key_len]
    total = sum(c)
    if total > n_free:
        return c, [ci * n_free // total for ci in c]
    return c, list(c)


def policy_candidates(scores, theta, key_begin, key_len, req_to_host, state, range_len,
                      per_range=128):
    """Per request: the eligible tokens (oracle.prefetch_eligible) and each range's candidates
    (its first per_range eligible tokens), as {range: [(token, host index), ...]}."""
    elig = oracle.prefetch_eligible(scores, theta, key_begin, key_len, req_to_host, state)
    cand = []
    for q in elig:
        c = {}
        for s, h in q:
            lst = c.setdefault(s // range_len, [])
            if len(lst) < per_range:
                lst.append((s, h))
        cand.append(c)
    return elig, cand


def policy_prefetch(scores, theta, key_begin, key_len, req_to_host, state, host_kv, cap, cap_div,
                    range_len, per_range=128):
    """Canonical outcome of the policy and what defines the valid ones.  Returns (new_state,
    moved [(request, token, host, slot)], demand [per request eligible count], info with
    'free_list', 'cap' (scaled c_r), 'offset' (O_r), 'cand' and 'eligible')."""
    free_list = np.flatnonzero(state.free == 1)
    elig, cand = policy_candidates(scores, theta, key_begin, key_len, req_to_host, state,
                                   range_len, per_range)
    _, caps = request_caps(key_len, cap, cap_div, len(free_list), state.n_gpu)
    offsets = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64) if len(caps) else []
    moves = []
    moved = []
    for r in range(len(key_len)):
        flat = [t for x in sorted(cand[r]) for t in cand[r][x]]
        for i, (s, h) in enumerate(flat[:caps[r]]):
            slot = int(free_list[offsets[r] + i])
            moves.append((h, slot))
            moved.append((r, s, h, slot))
    new = oracle.apply_prefetch(state, host_kv, moves)
    demand = np.array([len(q) for q in elig], np.int64)
    info = dict(free_list=free_list, cap=caps, offset=offsets, cand=cand, eligible=elig)
    return new, moved, demand, info


def check_policy_outcome(before, after, host_kv, info, slot_order=True):
    """Raises AssertionError unless `after` is a valid outcome of the policy from `before`:
    per request min(#candidates, c_r) rows moved, each range's a token-order prefix of its
    candidates with ascending slots, into exactly the request's first places; maps, priority 0
    and rows set; nothing else changed.  slot_order=False skips the ascending slots within a
    range (for a reference computed with other ranges than the run's)."""
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
    hk = np.ones(before.n_host, bool)
    hk[after.to_host[new_slots]] = False
    assert np.array_equal(after.host_to_gpu[hk], before.host_to_gpu[hk]), "host_to_gpu"


def decode_step_policy(q, w, k, k_scale, key_begin, key_len, req_to_host, state, host_kv, topk_k,
                       step_id, theta, cap, cap_div, range_len, reserve=0):
    """A whole decode step with the policy's canonical prefetch ahead of the exact top-k and the
    guaranteed recall.  Returns (scores, idx, state after the prefetch, moved, demand, info, final
    state, PoolStepResult)."""
    scores = oracle.index_scores(q, w, k, k_scale, key_begin, key_len)
    mid, moved, demand, info = policy_prefetch(scores, theta, key_begin, key_len, req_to_host,
                                               state, host_kv, cap, cap_div, range_len)
    idx = oracle.topk_rows(scores, topk_k)
    final, res = oracle.pool_step(mid, host_kv, idx, key_begin, req_to_host, step_id,
                                  reserve=reserve)
    return scores, idx, mid, moved, demand, info, final, res
