"""GPU parity of the scoring kernel with the host-gather wave (ECHO page §6.3; the threshold
prefetch of §6.1 done inside the scoring launch).  Two checks on what moves: the page's
contract (oracle.check_prefetch_contract: only eligible tokens, at most the bound per request,
free slots, priority 0, rows equal to the host, nothing else touched) and, on top of it, the
kernel's own documented policy (tests/prefetch_policy.py, check_policy_outcome).  On
integer-grid inputs the scores are bit-exact and the pool after the prefetch is a valid outcome
of that policy: the same demand, per request
min(#candidates, cap) rows moved, each range's a token-order prefix of its candidates, into
exactly the request's first places, maps, priorities and rows set, nothing else touched; when a
request's candidates fit its cap, its moved set is the oracle's exactly.  Cases cover several
range lengths, caps, thresholds (NaN and infinities), caps scaled to a short free list, a full
pool and 300 requests; a failed pool (status set) moves nothing.  General FP8 with scales: the
scores within tolerance and the same properties against the GPU's own scores.  The whole
decode step with the fused prefetch, eager and as one replayed hipGraph, against the oracle's
step: selection, misses, counters, and every pool array equal up to which of the prefetched
slots holds which prefetched row."""

import numpy as np
import pytest
import torch

import oracle
import prefetch_policy as pol
from dsa_indexer_top_amd import binding as B, inputs as gen
from dsa_indexer_top_amd.runner import DecodeRunner
from gpu_util import announce, dev, host, DevPool, assert_pool_equal

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _pool_case(inp, seed, n_gpu, free_frac, resident_frac):
    """A pool with a share of the requests' tokens resident and free_frac of the slots free."""
    rng = np.random.default_rng(seed)
    host_kv = gen.fill_latent_rows(seed, np.empty((inp.n_host, 576), np.uint16))
    st = oracle.PoolState.empty(n_gpu, inp.n_host)
    n_occ = int(round(n_gpu * (1 - free_frac)))
    tok_hosts = inp.req_to_host[rng.random(len(inp.req_to_host)) < resident_frac]
    others = np.setdiff1d(np.arange(inp.n_host), tok_hosts)
    hosts = np.concatenate([rng.permutation(tok_hosts), rng.permutation(others)])[:n_occ]
    slots = rng.permutation(n_gpu)[:n_occ]
    st.free[slots] = 0
    st.to_host[slots] = hosts
    st.host_to_gpu[hosts] = slots
    st.priority[slots] = rng.permutation(n_occ) + 1
    st.gpu_kv[slots] = host_kv[hosts]
    return st, host_kv


def _thetas(scores, q, specials):
    th = np.array([np.quantile(s, q) if len(s) else np.nan for s in scores], np.float32)
    for r, v in specials.items():
        th[r] = v
    return th


def _run_standalone(inp, st, host_kv, theta, cap, cap_div, rng_len, status=0):
    n, L = len(inp.key_len), max(int(inp.key_len.max()), 1)
    P = DevPool(st.free, st.priority, st.to_host, st.host_to_gpu, st.indices_buf, st.gpu_kv, host_kv)
    P.status.fill_(status)
    sc = torch.full((n, L), -7.0, dtype=torch.float32, device="cuda")
    npf = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    dem = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.fused_workspace_bytes(n, P.n_gpu), dtype=torch.uint8, device="cuda")
    B.index_scores_fused(dev(inp.q), dev(inp.w), dev(inp.k),
                         None if inp.k_scale is None else dev(inp.k_scale), dev(inp.key_begin),
                         dev(inp.key_len), L, sc, dev(theta), dev(inp.req_to_host), P.pool, cap,
                         cap_div, rng_len, npf, dem, ws)
    return host(sc), P.state(), int(host(npf)[0]), int(host(dem)[0]), P


def _lens_many(n, seed):
    return np.random.default_rng(seed).integers(0, 260, n).astype(np.int32).tolist()


CASES = [
    # lens, range, cap, cap_div, free share, threshold quantile, special thresholds, n_gpu
    ([0, 1, 127, 128, 129, 700, 3000], 128, 2048, 4, 0.5, 0.8, {}, None),
    ([0, 1, 127, 128, 129, 700, 3000], 256, 50, 1, 0.5, 0.6,
     {1: -np.inf, 4: np.nan, 5: np.inf}, None),
    ([5000, 2000, 3], 384, 4096, 1, 0.03, 0.5, {}, None),            # the free list runs short
    ([8192 + 130, 64], 8192, 4096, 1, 0.6, 0.0, {0: -np.inf}, None),  # 128 per range at most
    ([300, 129, 1000], 128, 64, 1, 0.0, 0.5, {}, 1003),               # a full pool: nothing moves
    (_lens_many(300, 9), 128, 40, 3, 0.7, 0.4, {}, 4096 + 77),        # offsets over 300 requests
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_prefetch_exact(case):
    lens, R, cap, cap_div, free_frac, qt, specials, n_gpu = CASES[case]
    announce("fused prefetch standalone", len(lens), "requests", R, cap, cap_div, free_frac)
    cfg = gen.DecodeConfig("fz", len(lens), 0, 64, "int", False, 0.5, 1, seed=300 + case)
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    n_gpu = n_gpu or max(256, inp.n_host // 2)
    st, host_kv = _pool_case(inp, 300 + case, n_gpu, free_frac, 0.3)
    scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
    theta = _thetas(scores, qt, specials)
    want, moved, demand, info = pol.policy_prefetch(scores, theta, inp.key_begin, inp.key_len,
                                                    inp.req_to_host, st, host_kv, cap, cap_div, R)
    got_sc, got_st, npf, dem, P = _run_standalone(inp, st, host_kv, theta, cap, cap_div, R)
    try:
        for r, s in enumerate(scores):
            assert np.array_equal(got_sc[r, :len(s)].astype(np.float64), s), "scores row %d" % r
        assert npf == len(moved) and dem == int(demand.sum())
        oracle.check_prefetch_contract(st, got_st, host_kv, info["eligible"],
                                       oracle.prefetch_bound(lens, cap, cap_div, n_gpu))
        pol.check_policy_outcome(st, got_st, host_kv, info)
        assert (len(moved) > 0) == (free_frac > 0) and demand.sum() > 0
    finally:
        P.hostbuf.close()


def test_fused_prefetch_automatic_range():
    # range = 0 lets the library pick the ranges; with at most 128 qualifying tokens per request
    # no range can have more than 128 candidates, so the outcome does not depend on the ranges
    # and the oracle's with one range per request is the reference
    lens = [3000, 5000, 129, 0]
    announce("fused prefetch, automatic range", lens)
    cfg = gen.DecodeConfig("fza", len(lens), 0, 64, "int", False, 0.5, 1, seed=340)
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    st, host_kv = _pool_case(inp, 340, 4000, 0.5, 0.3)
    scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
    theta = _thetas(scores, 0.98, {})
    want, moved, demand, info = pol.policy_prefetch(scores, theta, inp.key_begin, inp.key_len,
                                                    inp.req_to_host, st, host_kv, 200, 16,
                                                    max(lens))
    # the precondition: at most 128 eligible tokens per request, so no range of any length
    # holds more than 128 candidates
    assert int(demand.max()) <= 128
    got_sc, got_st, npf, dem, P = _run_standalone(inp, st, host_kv, theta, 200, 16, 0)
    try:
        for r, s_ in enumerate(scores):
            assert np.array_equal(got_sc[r, :len(s_)].astype(np.float64), s_), "scores row %d" % r
        assert npf == len(moved) > 0 and dem == int(demand.sum())
        # every candidate fits its cap: the moved set is the oracle's; the slots within the
        # request's places follow the library's own ranges
        assert all(sum(map(len, c.values())) <= cr for c, cr in zip(info["cand"], info["cap"]))
        oracle.check_prefetch_contract(st, got_st, host_kv, info["eligible"],
                                       oracle.prefetch_bound(lens, 200, 16, 4000))
        pol.check_policy_outcome(st, got_st, host_kv, info, slot_order=False)
    finally:
        P.hostbuf.close()


def test_fused_prefetch_failed_pool_moves_nothing():
    announce("fused prefetch with the status set")
    cfg = gen.DecodeConfig("fz", 3, 0, 64, "int", False, 0.5, 1, seed=310)
    inp = gen.make_decode_inputs(cfg, lengths=[900, 300, 1500])
    st, host_kv = _pool_case(inp, 310, 1500, 0.5, 0.2)
    scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
    theta = _thetas(scores, 0.5, {})
    got_sc, got_st, npf, dem, P = _run_standalone(inp, st, host_kv, theta, 100, 1, 256, status=1)
    try:
        assert npf == 0
        assert_pool_equal(got_st, st, "failed pool")
        for r, s in enumerate(scores):
            assert np.array_equal(got_sc[r, :len(s)].astype(np.float64), s)
    finally:
        P.hostbuf.close()


def test_fused_prefetch_general_fp8_properties():
    # general FP8 with per-token scales: the scores within 1e-4 T; what moved is, per request,
    # min(#candidates, cap) rows (candidates: each range's first 128 tokens whose GPU score is
    # above the threshold and that were not resident), each range's a token-order prefix in
    # ascending slots, in exactly the request's first places; every moved row equals its host
    # row
    announce("fused prefetch general fp8")
    lens, R, cap, cap_div = [3000, 1, 129, 2500], 256, 300, 2
    cfg = gen.DecodeConfig("fzg", len(lens), 0, 64, "general", True, 0.5, 1, seed=320)
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    st, host_kv = _pool_case(inp, 320, 3000, 0.4, 0.3)
    scores = oracle.index_scores(inp.q, inp.w, inp.k, inp.k_scale, inp.key_begin, inp.key_len)
    theta = _thetas(scores, 0.7, {})
    got_sc, got_st, npf, dem, P = _run_standalone(inp, st, host_kv, theta, cap, cap_div, R)
    try:
        T = oracle.error_scale(inp.q, inp.w, inp.k, inp.k_scale, inp.key_begin, inp.key_len)
        for r, s in enumerate(scores):
            g = got_sc[r, :len(s)].astype(np.float64)
            assert (np.abs(g - s) <= TOL * T[r]).all(), "scores row %d" % r
        oracle.check_pool_invariants(got_st, host_kv)
        new = np.flatnonzero((st.free == 1) & (got_st.free == 0))
        assert len(new) == npf > 0
        free_list = np.flatnonzero(st.free == 1)
        tok_of_host = {int(inp.req_to_host[inp.key_begin[r] + s]): (r, s)
                       for r in range(len(lens)) for s in range(lens[r])}
        by_req = {}
        for sl in new:
            r, s = tok_of_host[int(got_st.to_host[sl])]
            assert got_st.priority[sl] == 0 and np.array_equal(got_st.gpu_kv[sl], host_kv[got_st.to_host[sl]])
            by_req.setdefault(r, []).append((s, int(sl)))
        gpu_scores = [got_sc[r, :lens[r]].astype(np.float64) for r in range(len(lens))]
        oracle.check_prefetch_contract(
            st, got_st, host_kv,
            oracle.prefetch_eligible(gpu_scores, theta, inp.key_begin, inp.key_len,
                                     inp.req_to_host, st),
            oracle.prefetch_bound(lens, cap, cap_div, len(st.free)))
        caps = pol.request_caps(lens, cap, cap_div, len(free_list), len(st.free))[1]
        offset, n_dem = 0, 0
        for r in range(len(lens)):
            L = lens[r]
            # candidates from the GPU's own scores: per range the first 128 qualifying tokens
            qual = [s for s in range(L) if got_sc[r, s] > theta[r]
                    and st.host_to_gpu[inp.req_to_host[inp.key_begin[r] + s]] == oracle.INF]
            n_dem += len(qual)
            cand = {}
            for s_ in qual:
                if len(cand.setdefault(s_ // R, [])) < 128:
                    cand[s_ // R].append(s_)
            got = sorted(by_req.get(r, []))
            assert len(got) == min(sum(map(len, cand.values())), caps[r]), "request %d count" % r
            assert sorted(sl for _, sl in got) == list(free_list[offset:offset + len(got)])
            for x, cx in cand.items():
                gx = [(s_, sl) for s_, sl in got if s_ // R == x]
                assert [s_ for s_, _ in gx] == cx[:len(gx)], "request %d range %d prefix" % (r, x)
                assert [sl for _, sl in gx] == sorted(sl for _, sl in gx)
            offset += caps[r]
        assert dem == n_dem
    finally:
        P.hostbuf.close()


def _oracle_state(pool):
    return oracle.PoolState(pool.free.copy(), pool.priority.copy(), pool.to_host.copy(),
                            pool.host_to_gpu.copy(), pool.indices_buf.copy(), pool.gpu_kv.copy())


def _as_state(d):
    return oracle.PoolState(d["free"], d["priority"], d["to_host"], d["host_to_gpu"],
                            d["indices_buf"], d["gpu_kv"])


def _assert_equal_up_to_prefetched(got, want, pf_slots, what):
    """Every pool array equal, except that the prefetched rows may sit in any of the prefetched
    slots (which one gets which depends on timing): there, the (host index, priority, row)
    triples must agree as multisets and the maps must stay inverse."""
    keep = np.ones(len(want.free), bool)
    keep[pf_slots] = False
    for name in ("free", "priority", "to_host", "indices_buf", "gpu_kv"):
        a, b = getattr(got, name), getattr(want, name)
        assert np.array_equal(a[keep], b[keep]), "%s: %s outside the prefetched slots" % (what, name)
    trip = lambda st: sorted((int(st.to_host[s]), int(st.priority[s]), st.gpu_kv[s].tobytes())
                             for s in pf_slots)
    assert trip(got) == trip(want), "%s: the prefetched rows" % what
    hk = np.ones(len(want.host_to_gpu), bool)
    hk[want.to_host[pf_slots][want.to_host[pf_slots] != oracle.INF]] = False
    assert np.array_equal(got.host_to_gpu[hk], want.host_to_gpu[hk]), "%s: host_to_gpu" % what
    for s_ in pf_slots:
        h = got.to_host[s_]
        assert h == oracle.INF or got.host_to_gpu[h] == s_, "%s: maps of slot %d" % (what, s_)


@pytest.mark.parametrize("given_theta", [True, False])
@pytest.mark.parametrize("lens,k,R,div,reserve", [([3000, 700, 1, 0], 64, 256, 1, 1500),
                                                  ([5000, 4096], 256, 128, 1, 3000),
                                                  ([2000, 900], 128, 256, 4, 0)])   # a full pool
def test_decode_step_fused(lens, k, R, div, reserve, given_theta):
    # the whole step with the fused prefetch: the threshold given (the EMA estimate) or the
    # sample percentile; every request's candidates fit its cap and the misses fit the free
    # room, so what moves and what the step does afterwards are unique; selection, misses,
    # counters and the pool after the step against the oracle's step, up to which prefetched
    # slot holds which prefetched row; then replayed as one graph from the same start
    announce("decode step fused", lens, k, R, reserve, "given theta" if given_theta else "sample theta")
    cfg = gen.DecodeConfig("fzd", len(lens), 0, k, "int", False, 0.5, div, seed=330 + k,
                           reserve=reserve)
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    host_kv = gen.fill_latent_rows(cfg.seed, np.empty((inp.n_host, 576), np.uint16))
    scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
    idx = oracle.topk_rows(scores, k)
    pool = gen.make_pool_state(inp, idx, host_kv)
    if given_theta:
        theta = _thetas(scores, 0.9, {len(lens) - 1: np.nan})
    else:
        theta = np.array([oracle.sample_threshold(s, 4096, 95.0) for s in scores], np.float32)
    cap, cap_div = 2048, 8
    st0 = _oracle_state(pool)
    _, want_idx, mid, moved, demand, info, want_state, res = pol.decode_step_policy(
        inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len, inp.req_to_host, st0, host_kv, k,
        pool.step_id, theta, cap, cap_div, R)
    assert (len(moved) > 0) == (reserve > 0) and res.status == 0
    for r, c in enumerate(info["cand"]):                # the preconditions of a unique result
        assert sum(map(len, c.values())) <= info["cap"][r] or info["cap"][r] == 0
    assert reserve == 0 or res.n_evicted == 0
    pf_slots = np.array(sorted(m[3] for m in moved), np.int64)
    pf = dict(cap=cap, cap_div=cap_div, range=R)
    rn = DecodeRunner(inp, pool, host_kv, prefetch="fused", pf=pf,
                      theta=theta if given_theta else None)
    try:
        for mode in ("eager", "graph", "graph again"):
            if mode == "eager":
                rn.run_eager()
            else:
                if rn.graph is None:
                    rn.capture()
                rn.restore()
                rn.replay()
            got = rn.results()
            assert got["status"] == 0, mode
            assert np.array_equal(got["topk_idx"], want_idx), mode
            assert np.array_equal(got["miss_host"], res.miss_host), mode
            assert np.array_equal(got["miss_slot"], res.miss_slot), mode
            assert list(got["counters"][:3]) == [res.n_miss, int(demand.sum()), len(moved)], mode
            pf_sel = np.isin(res.topk_slot, pf_slots)
            assert np.array_equal(got["topk_slot"][~pf_sel], res.topk_slot[~pf_sel]), mode
            assert np.isin(got["topk_slot"][pf_sel], pf_slots).all(), mode
            _assert_equal_up_to_prefetched(_as_state(got["pool"]), want_state, pf_slots, mode)
            idx_ = got["topk_idx"]
            rows, cols = np.nonzero(idx_ >= 0)
            hosts = inp.req_to_host[inp.key_begin[rows] + idx_[rows, cols]]
            oracle.check_pool_invariants(_as_state(got["pool"]), host_kv, hosts,
                                         got["topk_slot"][rows, cols])
    finally:
        rn.close()


@pytest.mark.parametrize("mode", ["fused", "ranged"])
def test_decode_step_prefetch_then_evict(mode):
    # the prefetch fills the few free slots with candidates; the guaranteed recall then has
    # more misses than free slots left and evicts, the prefetched rows (priority 0) first.
    # Which rows stay resident then depends on timing; the selection, the scores, every selected
    # row resident bit for bit and the pool invariants must not, eager and over graph replays,
    # and they must equal the step without prefetch
    announce("decode step, %s prefetch, then eviction" % mode)
    lens, k, reserve = [6000, 3000, 5000], 256, 400
    cfg = gen.DecodeConfig("pfe", len(lens), 0, k, "int", False, 0.3, 4, seed=77, reserve=reserve)
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    host_kv = gen.fill_latent_rows(cfg.seed, np.empty((inp.n_host, 576), np.uint16))
    scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
    idx = oracle.topk_rows(scores, k)
    pool = gen.make_pool_state(inp, idx, host_kv)
    assert int(pool.free.sum()) == reserve
    theta = _thetas(scores, 0.9, {})
    off = DecodeRunner(inp, pool, host_kv)
    try:
        off.run_eager()
        base = off.results()
    finally:
        off.close()
    assert base["status"] == 0 and np.array_equal(base["topk_idx"], idx)
    rn = DecodeRunner(inp, pool, host_kv, prefetch=mode, theta=theta,
                      pf=dict(n_chunks=3, cap=2048, cap_div=4, range=256))
    try:
        for run in ("eager", "graph", "graph again"):
            if run == "eager":
                rn.run_eager()
            else:
                if rn.graph is None:
                    rn.capture()
                rn.restore()
                rn.replay()
            got = rn.results()
            assert got["status"] == 0, run
            assert np.array_equal(got["topk_idx"], idx), run
            for r, L in enumerate(lens):
                assert np.array_equal(got["scores"][r, :L].astype(np.float64), scores[r]), (run, r)
            n_miss, moved = int(got["counters"][0]), int(got["counters"][2])
            assert moved > 0, run
            assert n_miss > reserve - moved, run            # the recall had to evict
            rows, cols = np.nonzero(idx >= 0)
            hosts = inp.req_to_host[inp.key_begin[rows] + idx[rows, cols]]
            oracle.check_pool_invariants(_as_state(got["pool"]), host_kv, hosts,
                                         got["topk_slot"][rows, cols])
            sel = got["pool"]["gpu_kv"][got["topk_slot"][rows, cols]]
            assert np.array_equal(sel, base["pool"]["gpu_kv"][base["topk_slot"][rows, cols]]), run
    finally:
        rn.close()
