"""Pins of the oracle's pool step: the page's worked example, the footprint formula,
brute-force eviction, invariants, error paths, and planted mistakes."""

import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import (INF, ST_EXHAUSTED, ST_BAD_HOST, ST_DUP_HOST, PoolState, pool_step,
                    allocate_with_ranks, metadata_bytes, check_pool_invariants,
                    PoolInvariantError)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _random_pool(rng, n_gpu, n_host, n_occ):
    st = PoolState.empty(n_gpu, n_host)
    slots = rng.permutation(n_gpu)[:n_occ]
    hosts = rng.permutation(n_host)[:n_occ]
    st.free[slots] = 0
    st.to_host[slots] = hosts
    st.host_to_gpu[hosts] = slots
    st.priority[slots] = rng.integers(0, max(2, n_occ // 2), n_occ)   # ties on purpose
    host_kv = rng.integers(0, 0xBFFF, (n_host, 576)).astype(np.uint16)
    st.gpu_kv[slots] = host_kv[hosts]
    return st, host_kv


def _one_request(rng, n_host, n_sel, L=None):
    L = n_host if L is None else L
    req_to_host = rng.permutation(n_host).astype(np.int32)[:L]
    sel = np.sort(rng.permutation(L)[:n_sel]).astype(np.int32)[None, :]
    return sel, np.array([0]), req_to_host


def test_allocate_worked_example():
    ex = _load("allocate_example.json")
    slots = allocate_with_ranks(ex["free"], ex["ranks"], ex["host_indices"])
    assert slots == ex["expected_slots"]
    # the canonical rule on the same all-free bitmap: ascending free slots
    st = PoolState.empty(ex["n_slots"], 8)
    req_to_host = np.array(ex["host_indices"], np.int32)
    sel = np.array([[0, 1]], np.int32)
    host_kv = np.arange(8 * 576, dtype=np.uint16).reshape(8, 576)
    new, res = pool_step(st, host_kv, sel, np.array([0]), req_to_host, step_id=7)
    assert res.status == 0 and res.n_miss == 2
    assert res.miss_slot[:2].tolist() == [0, 1]
    assert new.to_host[:2].tolist() == [3, 4] and new.host_to_gpu[[3, 4]].tolist() == [0, 1]
    assert new.priority[:2].tolist() == [7, 7] and new.priority[2:].tolist() == [-1] * 4
    assert new.indices_buf.tolist() == [0, 1, -1, -1, -1, -1]
    check_pool_invariants(new, host_kv, [3, 4], [0, 1])


def test_footprint_formula():
    ex = _load("footprint.json")
    for nh, ng in [(2_000_000, 200_000), (1, 1), (8_388_608, 1_048_576)]:
        assert metadata_bytes(nh, ng) == 4 * nh + 13 * ng
    per_layer = metadata_bytes(ex["n_host"], ex["n_gpu"]) / 1e6
    assert abs(per_layer - ex["per_layer_mb_approx"]) / ex["per_layer_mb_approx"] < 0.1
    total = per_layer * ex["layers"]
    assert abs(total - ex["total_mb_approx"]) / ex["total_mb_approx"] < 0.1


def _brute_force_evicted(st, protected, need):
    """The unique set of `need` unprotected occupied slots each of which precedes
    every kept unprotected occupied slot in (priority, slot) order."""
    cand = [e for e in range(st.n_gpu) if st.free[e] == 0 and e not in protected]
    found = []
    for sub in itertools.combinations(cand, need):
        kept = [u for u in cand if u not in sub]
        if all((st.priority[e], e) < (st.priority[u], u) for e in sub for u in kept):
            found.append(set(sub))
    assert len(found) == 1
    return found[0]


def test_eviction_brute_force_tiny():
    rng = np.random.default_rng(21)
    for trial in range(60):
        n_gpu, n_host = 8, 24
        st, host_kv = _random_pool(rng, n_gpu, n_host, n_occ=int(rng.integers(5, 9)))
        sel, kb, r2h = _one_request(rng, n_host, n_sel=int(rng.integers(1, 6)))
        hosts = r2h[sel[0]]
        protected = {int(st.host_to_gpu[h]) for h in hosts if st.host_to_gpu[h] != INF}
        n_miss = sum(1 for h in hosts if st.host_to_gpu[h] == INF)
        need = max(0, n_miss - int(st.free.sum()))
        n_cand = sum(1 for e in range(n_gpu) if st.free[e] == 0 and e not in protected)
        new, res = pool_step(st, host_kv, sel, kb, r2h, step_id=100)
        if need > n_cand:
            assert res.status == ST_EXHAUSTED
            continue
        assert res.status == 0 and res.n_evicted == need
        want = _brute_force_evicted(st, protected, need)
        # evicted = slots that held an unselected host before and no longer hold it
        evicted = {e for e in range(n_gpu) if st.free[e] == 0 and e not in protected
                   and new.to_host[e] != st.to_host[e]}
        assert evicted == want
        check_pool_invariants(new, host_kv, hosts, res.topk_slot[0][res.topk_slot[0] >= 0],
                              protected_before=sorted(protected))


@pytest.mark.parametrize("reserve", [1, 3, 8])
def test_eviction_reserve_brute_force_tiny(reserve):
    # with room kept for prefetch, the step evicts further down the same (priority, slot)
    # order until `reserve` slots stay free after the allocation, as far as unprotected slots go
    rng = np.random.default_rng(40 + reserve)
    for trial in range(60):
        n_gpu, n_host = 8, 24
        st, host_kv = _random_pool(rng, n_gpu, n_host, n_occ=int(rng.integers(5, 9)))
        sel, kb, r2h = _one_request(rng, n_host, n_sel=int(rng.integers(1, 6)))
        hosts = r2h[sel[0]]
        protected = {int(st.host_to_gpu[h]) for h in hosts if st.host_to_gpu[h] != INF}
        n_miss = sum(1 for h in hosts if st.host_to_gpu[h] == INF)
        n_free = int(st.free.sum())
        n_cand = sum(1 for e in range(n_gpu) if st.free[e] == 0 and e not in protected)
        new, res = pool_step(st, host_kv, sel, kb, r2h, step_id=100, reserve=reserve)
        if n_miss - n_free > n_cand:
            assert res.status == ST_EXHAUSTED
            continue
        need = min(max(0, n_miss + reserve - n_free), n_cand)
        assert res.status == 0 and res.n_evicted == need
        evicted = {e for e in range(n_gpu) if st.free[e] == 0 and e not in protected
                   and new.to_host[e] != st.to_host[e]}
        assert evicted == _brute_force_evicted(st, protected, need)
        # free slots afterwards: at least the reserve, or every unprotected slot gone
        left = int(new.free.sum())
        assert left == max(reserve, n_free - n_miss) or (left < reserve and need == n_cand)
        check_pool_invariants(new, host_kv, hosts, res.topk_slot[0][res.topk_slot[0] >= 0],
                              protected_before=sorted(protected))
        # reserve 0 reduces to the plain step
        if reserve == 1:
            plain, r0 = pool_step(st, host_kv, sel, kb, r2h, step_id=100)
            assert r0.n_evicted == max(0, n_miss - n_free)


def test_step_postconditions_random():
    rng = np.random.default_rng(22)
    for trial in range(20):
        n_gpu, n_host = 64, 400
        st, host_kv = _random_pool(rng, n_gpu, n_host, n_occ=int(rng.integers(30, 65)))
        B, k = 3, 12
        L = [100, 150, 150]
        r2h = rng.permutation(n_host).astype(np.int32)[:sum(L)]
        kb = np.array([0, 100, 250])
        sel = np.full((B, k), -1, np.int32)
        for r in range(B):
            m = int(rng.integers(0, k + 1))
            sel[r, :m] = np.sort(rng.permutation(L[r])[:m])
        before = st.copy()
        new, res = pool_step(st, host_kv, sel, kb, r2h, step_id=999)
        assert np.array_equal(st.free, before.free)          # input not modified
        if res.status:
            continue
        rows, cols = np.nonzero(sel >= 0)
        hosts = r2h[kb[rows] + sel[rows, cols]]
        slots = res.topk_slot[rows, cols]
        check_pool_invariants(new, host_kv, hosts, slots)
        assert (new.priority[slots] == 999).all()
        assert (res.topk_slot[sel < 0] == -1).all()
        # rows change only where a recall landed: eviction moves no data
        untouched = np.setdiff1d(np.arange(n_gpu), res.miss_slot[:res.n_miss])
        assert np.array_equal(new.gpu_kv[untouched], before.gpu_kv[untouched])
        # misses listed in (request, token) order and given ascending slots
        ms = res.miss_slot[:res.n_miss]
        assert (np.diff(ms) > 0).all()
        assert (res.miss_slot[res.n_miss:] == -1).all()
        # a second identical step finds everything resident
        new2, res2 = pool_step(new, host_kv, sel, kb, r2h, step_id=1000)
        assert res2.n_miss == 0 and res2.n_evicted == 0
        assert np.array_equal(new2.to_host, new.to_host)


def test_error_paths():
    rng = np.random.default_rng(23)
    st, host_kv = _random_pool(rng, 4, 20, n_occ=4)
    r2h = rng.permutation(20).astype(np.int32)
    # exhaustion: 4 slots, select 5 non-resident tokens
    nonres = [i for i in range(20) if st.host_to_gpu[r2h[i]] == INF][:5]
    sel = np.array([sorted(nonres)], np.int32)
    new, res = pool_step(st, host_kv, sel, np.array([0]), r2h, 5)
    assert res.status == ST_EXHAUSTED and new is st
    # bad host index
    bad = r2h.copy()
    bad[sel[0, 0]] = 20
    new, res = pool_step(st, host_kv, sel[:, :1], np.array([0]), bad, 5)
    assert res.status == ST_BAD_HOST and new is st
    # duplicate host index among misses
    dup = r2h.copy()
    dup[sel[0, 1]] = dup[sel[0, 0]]
    new, res = pool_step(st, host_kv, sel[:, :2], np.array([0]), dup, 5)
    assert res.status == ST_DUP_HOST


@pytest.mark.parametrize("corrupt", ["dup_slot", "broken_inverse", "free_mismatch",
                                     "missed_row", "evicted_protected", "orphan_host",
                                     "moved_row"])
def test_checker_catches_corruption(corrupt):
    for seed in range(24, 100):      # first draw with a protected (resident, selected) slot
        rng = np.random.default_rng(seed)
        st, host_kv = _random_pool(rng, 16, 64, n_occ=12)
        sel, kb, r2h = _one_request(rng, 64, n_sel=6)
        protected = [int(st.host_to_gpu[h]) for h in r2h[sel[0]] if st.host_to_gpu[h] != INF]
        if protected:
            break
    before = st.copy()
    new, res = pool_step(st, host_kv, sel, kb, r2h, 50)
    hosts, slots = r2h[sel[0]], res.topk_slot[0]
    untouched = np.setdiff1d(np.arange(16), res.miss_slot[:res.n_miss])
    check_pool_invariants(new, host_kv, hosts, slots, protected,
                          (untouched, before.gpu_kv[untouched]))
    bad = new.copy()
    occ = np.flatnonzero(bad.free == 0)
    kw = {}
    if corrupt == "dup_slot":
        bad.to_host[occ[1]] = bad.to_host[occ[0]]
    elif corrupt == "broken_inverse":
        bad.host_to_gpu[bad.to_host[occ[0]]] = occ[1]
    elif corrupt == "free_mismatch":
        bad.free[occ[0]] = 1
    elif corrupt == "missed_row":
        bad.gpu_kv[slots[0]] = 0xFFFF
    elif corrupt == "evicted_protected":
        p = protected[0]
        bad.host_to_gpu[bad.to_host[p]] = INF
        bad.to_host[p], bad.free[p], bad.priority[p] = INF, 1, -1
        kw["protected_before"] = protected
    elif corrupt == "orphan_host":
        spare = [h for h in range(64) if bad.host_to_gpu[h] == INF][0]
        bad.host_to_gpu[spare] = occ[0]
    elif corrupt == "moved_row":
        # rows change only in slots that received a recall; corrupt another one
        untouched = np.setdiff1d(np.arange(16), res.miss_slot[:res.n_miss])
        kw["evicted_rows_before"] = (untouched, before.gpu_kv[untouched])
        bad.gpu_kv[untouched[0]] ^= 1
    with pytest.raises(PoolInvariantError):
        if corrupt in ("evicted_protected", "moved_row"):
            check_pool_invariants(bad, **kw)
        else:
            check_pool_invariants(bad, host_kv, hosts, slots)


def test_planted_oracle_mistakes_are_caught(monkeypatch):
    """Mistakes planted in the oracle (on the CPU) must fail the pins above."""
    rng = np.random.default_rng(25)
    st, host_kv = _random_pool(rng, 8, 24, n_occ=8)
    sel, kb, r2h = _one_request(rng, 24, n_sel=4)
    hosts = r2h[sel[0]]
    protected = {int(st.host_to_gpu[h]) for h in hosts if st.host_to_gpu[h] != INF}
    n_miss = sum(1 for h in hosts if st.host_to_gpu[h] == INF)
    need = max(0, n_miss - int(st.free.sum()))
    want = _brute_force_evicted(st, protected, need)
    assert need > 0
    # planted mistake 1: evict the highest priorities instead of the lowest
    real_lexsort = np.lexsort
    monkeypatch.setattr(oracle.pool.np, "lexsort",
                        lambda keys: real_lexsort(keys)[::-1])
    new, res = pool_step(st, host_kv, sel, kb, r2h, 77)
    monkeypatch.undo()
    evicted = {e for e in range(8) if st.free[e] == 0 and e not in protected
               and new.to_host[e] != st.to_host[e]}
    assert evicted != want
    # planted mistake 2: recall copies the wrong row (off by one host index)
    new, res = pool_step(st, host_kv, sel, kb, r2h, 77)
    shifted = new.copy()
    ms = res.miss_slot[:res.n_miss]
    shifted.gpu_kv[ms] = host_kv[(res.miss_host[:res.n_miss] + 1) % 24]
    with pytest.raises(PoolInvariantError):
        check_pool_invariants(shifted, host_kv, hosts, res.topk_slot[0])
