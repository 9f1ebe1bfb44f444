"""GPU parity of the whole decode step (echo_decode_select, eager and as one captured hipGraph)
against the oracle's decode step; the prefetch threshold, the fused prefetch scoring, and the
losslessness of prefetch (same selection and resident rows with prefetch on and off)."""

import numpy as np
import pytest
import torch

import oracle
from dsa_indexer_top_amd import binding as B, inputs as gen
from dsa_indexer_top_amd.runner import DecodeRunner
from gpu_util import announce, dev, host, assert_pool_equal

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _setup(cfg, lengths=None, hit_rate=None, reserve=None):
    inp = gen.make_decode_inputs(cfg, lengths=lengths)
    host_kv = gen.fill_latent_rows(cfg.seed, np.empty((inp.n_host, 576), np.uint16))
    scores = oracle.index_scores(inp.q, inp.w, inp.k, inp.k_scale, inp.key_begin, inp.key_len)
    idx = oracle.topk_rows(scores, cfg.topk)
    pool = gen.make_pool_state(inp, idx, host_kv, hit_rate=hit_rate, reserve=reserve)
    return inp, host_kv, scores, idx, pool


def _oracle_state(pool):
    return oracle.PoolState(pool.free.copy(), pool.priority.copy(), pool.to_host.copy(),
                            pool.host_to_gpu.copy(), pool.indices_buf.copy(), pool.gpu_kv.copy())


def _as_state(d):
    return oracle.PoolState(d["free"], d["priority"], d["to_host"], d["host_to_gpu"],
                            d["indices_buf"], d["gpu_kv"])


def _check_exact(inp, host_kv, scores, idx, pool, got):
    for r in range(len(inp.key_len)):
        L = int(inp.key_len[r])
        assert np.array_equal(got["scores"][r, :L].astype(np.float64), scores[r]), "scores row %d" % r
    _check_pool_exact(inp, host_kv, idx, pool, got)


def _check_pool_exact(inp, host_kv, idx, pool, got, reserve=0):
    st0 = _oracle_state(pool)
    want_state, want = oracle.pool_step(st0, host_kv, idx, inp.key_begin, inp.req_to_host, pool.step_id,
                                        reserve)
    assert np.array_equal(got["topk_idx"], idx)
    assert got["status"] == want.status
    if want.status:
        assert_pool_equal(_as_state(got["pool"]), st0, "untouched")
        return
    assert int(got["counters"][0]) == want.n_miss
    assert np.array_equal(got["topk_slot"], want.topk_slot)
    assert np.array_equal(got["miss_host"], want.miss_host)
    assert np.array_equal(got["miss_slot"], want.miss_slot)
    assert_pool_equal(_as_state(got["pool"]), want_state)


def _check_invariants(inp, host_kv, got):
    idx = got["topk_idx"]
    rows, cols = np.nonzero(idx >= 0)
    hosts = inp.req_to_host[inp.key_begin[rows] + idx[rows, cols]]
    oracle.check_pool_invariants(_as_state(got["pool"]), host_kv, hosts, got["topk_slot"][rows, cols])


def _check_topk_tolerance(inp, scores, got, rows):
    """General FP8: GPU and oracle sets may differ only by tokens whose oracle score is within
    the tolerance of the oracle's k-th score."""
    k = inp.cfg.topk
    for r in rows:
        sl = slice(r, r + 1)
        T = oracle.error_scale(inp.q[sl], inp.w[sl], inp.k, inp.k_scale, inp.key_begin[sl], inp.key_len[sl])[0]
        s = scores[r]
        g = got["scores"][r, :len(s)].astype(np.float64)
        assert (np.abs(g - s) <= TOL * T).all(), "score tolerance row %d" % r
        want = oracle.topk_row(s, k)
        mine = got["topk_idx"][r]
        assert (np.diff(mine[mine >= 0]) > 0).all()
        m = min(k, len(s))
        if m == 0:
            continue
        kth = want[:m][np.argmin(s[want[:m]])]
        diff = np.setxor1d(mine[:m], want[:m])
        for t in diff:
            assert abs(s[t] - s[kth]) <= TOL * (T[t] + T[kth]), "row %d token %d outside tolerance" % (r, t)


def test_decode_tiny_eager_exact():
    announce("decode tiny eager")
    cfg = gen.CONFIGS["tiny"]
    inp, host_kv, scores, idx, pool = _setup(cfg)
    rn = DecodeRunner(inp, pool, host_kv)
    rn.run_eager()
    _check_exact(inp, host_kv, scores, idx, pool, rn.results())
    rn.close()


@pytest.mark.parametrize("one_stream", [False, True])
@pytest.mark.parametrize("lens,k,hit,div", [([1, 300, 5000], 256, 0.6, 4),
                                            ([2048, 2047, 2049], 2048, 0.25, 1),
                                            ([0, 70, 4097], 64, 0.6, 4),
                                            ([0, 1, 0], 64, 0.6, 4)])
def test_decode_small_ragged_exact(lens, k, hit, div, one_stream):
    announce("decode small ragged", lens, k, "one stream" if one_stream else "two streams")
    cfg = gen.DecodeConfig("s", len(lens), 0, k, "int", False, hit, div, seed=31 + k)
    inp, host_kv, scores, idx, pool = _setup(cfg, lengths=lens)
    rn = DecodeRunner(inp, pool, host_kv)
    if one_stream:
        rn.side = rn.main
    rn.run_eager()
    _check_exact(inp, host_kv, scores, idx, pool, rn.results())
    rn.close()


@pytest.mark.parametrize("reserve", [1, 500, 5000, 100000])
def test_decode_reserve_exact(reserve):
    # the guaranteed recall leaves `reserve` slots free (as far as unprotected slots allow):
    # the same canonical pool step as the oracle's with that reserve, bit for bit; 100000 is
    # more than the evictable slots, so everything unprotected goes
    announce("decode reserve", reserve)
    lens = [3000, 700, 9000]
    cfg = gen.DecodeConfig("r", 3, 0, 256, "int", False, 0.5, 4, seed=39)
    inp, host_kv, scores, idx, pool = _setup(cfg, lengths=lens)
    rn = DecodeRunner(inp, pool, host_kv, reserve=min(reserve, inp.n_gpu))
    rn.capture()
    rn.replay()
    got = rn.results()
    assert got["status"] == 0
    _check_pool_exact(inp, host_kv, idx, pool, got, reserve=min(reserve, inp.n_gpu))
    rn.close()


def test_decode_exhausted_pool_untouched():
    announce("decode exhausted")
    lens = [2048, 2047, 2049]
    cfg = gen.DecodeConfig("x", 3, 0, 2048, "int", False, 0.25, 2, seed=37)
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    host_kv = gen.fill_latent_rows(cfg.seed, np.empty((inp.n_host, 576), np.uint16))
    scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
    idx = oracle.topk_rows(scores, cfg.topk)
    pool = gen.make_pool_state(inp, idx, host_kv)
    rn = DecodeRunner(inp, pool, host_kv)
    rn.run_eager()
    got = rn.results()
    assert got["status"] == oracle.ST_EXHAUSTED      # 6143 selected rows cannot fit 3072 slots
    _check_exact(inp, host_kv, scores, idx, pool, got)
    rn.close()


def test_decode_b8_64k_graph_replays_exact():
    announce("decode b8_64k graph")
    cfg = gen.CONFIGS["b8_64k"]
    inp, host_kv, scores, idx, pool = _setup(cfg)
    rn = DecodeRunner(inp, pool, host_kv)
    rn.run_eager()
    eager = rn.results()
    _check_exact(inp, host_kv, scores, idx, pool, eager)
    rn.capture()
    for rep in range(3):
        rn.restore()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum().item()   # eager work between replays
        rn.replay()
        got = rn.results()
        assert got["status"] == 0
        for key in ("topk_idx", "topk_slot", "miss_host", "miss_slot", "counters"):
            assert np.array_equal(got[key], eager[key]), (rep, key)
        for n in got["pool"]:
            assert np.array_equal(got["pool"][n], eager["pool"][n]), (rep, n)
    rn.close()


def test_decode_b32_ragged_general_tolerance():
    announce("decode b32_ragged full")
    cfg = gen.CONFIGS["b32_ragged"]
    inp, host_kv, scores, idx, pool = _setup(cfg)
    rn = DecodeRunner(inp, pool, host_kv)
    rn.capture()
    rn.replay()
    got = rn.results()
    assert got["status"] == 0
    _check_topk_tolerance(inp, scores, got, rows=range(len(inp.key_len)))   # all 32 requests
    _check_invariants(inp, host_kv, got)
    if np.array_equal(got["topk_idx"], idx):           # same set: the pool must match exactly
        _check_pool_exact(inp, host_kv, idx, pool, got)
    rn.close()


def test_prefetch_threshold_matches_sample_percentile():
    announce("prefetch threshold")
    for grid in ("int", "general"):
        cfg = gen.DecodeConfig("t", 4, 0, 64, grid, grid == "general", 0.5, 4, seed=41)
        lens = [5000, 100, 0, 70000]
        inp = gen.make_decode_inputs(cfg, lengths=lens)
        theta = torch.empty(4, dtype=torch.float32, device="cuda")
        B.prefetch_threshold(dev(inp.q), dev(inp.w), dev(inp.k),
                             None if inp.k_scale is None else dev(inp.k_scale),
                             dev(inp.key_begin), dev(inp.key_len), max(lens), 4096, 95.0, theta)
        got = host(theta)
        scores = oracle.index_scores(inp.q, inp.w, inp.k, inp.k_scale, inp.key_begin, inp.key_len)
        for r in range(4):
            want = oracle.sample_threshold(scores[r], 4096, 95.0)
            if lens[r] == 0:
                assert np.isinf(got[r])
            elif grid == "int":
                assert got[r] == want, (r, got[r], want)
            else:
                assert abs(got[r] - want) <= 1e-3 * (abs(want) + 1), (r, got[r], want)
        # lengths above max_key_len are clamped: the sample covers the first max_key_len keys
        clamp = 3000
        B.prefetch_threshold(dev(inp.q), dev(inp.w), dev(inp.k),
                             None if inp.k_scale is None else dev(inp.k_scale),
                             dev(inp.key_begin), dev(inp.key_len), clamp, 4096, 95.0, theta)
        got = host(theta)
        for r in range(4):
            L = min(lens[r], clamp)
            if L == 0:
                assert np.isinf(got[r])
                continue
            want = oracle.sample_threshold(scores[r][:L], 4096, 95.0)
            if grid == "int":
                assert got[r] == want, ("clamped", r, got[r], want)
            else:
                assert abs(got[r] - want) <= 1e-3 * (abs(want) + 1), ("clamped", r, got[r], want)


def _prefetch_scoring_case(lens, quantile, cap, cap_div, seed):
    # the scoring launch lists over-threshold non-resident tokens up to the cap and counts all
    # of them as demand
    cfg = gen.DecodeConfig("p", len(lens), 0, 64, "int", False, 0.5, 4, seed=seed)
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    rng = np.random.default_rng(5)
    h2g = np.full(inp.n_host, gen.INF, np.int32)
    res = rng.permutation(inp.n_host)[: inp.n_host // 3]
    h2g[res] = np.arange(len(res))                      # a third of the tokens resident
    scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
    theta = np.array([np.quantile(s, quantile) for s in scores], np.float32)
    d = {n: dev(getattr(inp, n)) for n in ("q", "w", "k", "key_begin", "key_len", "req_to_host")}
    n = len(lens)
    sc = torch.empty((n, max(lens)), dtype=torch.float32, device="cuda")
    cand = torch.full((n, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(n, dtype=torch.int32, device="cuda")
    tot = torch.zeros(n, dtype=torch.int32, device="cuda")
    B.index_scores_prefetch(d["q"], d["w"], d["k"], None, d["key_begin"], d["key_len"], max(lens),
                            0, max(lens), sc, dev(theta), d["req_to_host"], dev(h2g), cand, cnt,
                            tot, cap, cap_div)
    got_s, got_c, got_n, got_t = host(sc), host(cand), host(cnt), host(tot)
    for r in range(n):
        L = lens[r]
        s = scores[r]
        assert np.array_equal(got_s[r, :L].astype(np.float64), s)
        hosts = inp.req_to_host[inp.key_begin[r]:inp.key_begin[r] + L]
        eligible = np.flatnonzero((s > theta[r]) & (h2g[hosts] == gen.INF))
        cap_r = min(cap, -(-L // cap_div))
        assert got_t[r] == len(eligible)
        # a workgroup lists at least the eligible ones among its first 1024 over-threshold
        # tokens; here that is more than the cap wherever the eligible tokens are
        assert got_n[r] == min(cap_r, len(eligible))
        listed = got_c[r, :got_n[r]]
        assert len(set(listed.tolist())) == len(listed)
        assert set(listed.tolist()) <= set(eligible.tolist())


def test_fused_prefetch_scoring_candidates():
    announce("prefetch scoring candidates")
    _prefetch_scoring_case([9000, 300, 20000], 0.9, 4096, 8, 43)


def test_prefetch_scoring_list_overflow_b8_64k():
    # 2048 tokens per workgroup at this size; at the 0.2 quantile about 1600 of them are over
    # the threshold, more than a workgroup's list holds: the ones past it are looked up in the
    # streaming loop and only counted towards the demand, which stays exact
    announce("prefetch scoring, list overflow, 8 x 65536")
    _prefetch_scoring_case([65536] * 8, 0.2, 4096, 64, 44)


@pytest.mark.parametrize("side_stream", [True, False])
def test_prefetch_is_lossless(side_stream):
    announce("prefetch lossless side=%s" % side_stream)
    cfg = gen.DecodeConfig("l", 6, 24000, 512, "general", True, 0.5, 8, reserve=4000,
                           prefetch=True, seed=47)
    inp, host_kv, scores, idx, pool = _setup(cfg)
    off = DecodeRunner(inp, pool, host_kv)
    off.capture()
    off.replay()
    a = off.results()
    off.close()
    pf = dict(n_chunks=3, n_sample=1024, percentile=90.0, cap=400, cap_div=64)
    on = DecodeRunner(inp, pool, host_kv, prefetch=True, pf=pf)
    if not side_stream:
        on.side = on.main
    on.capture()
    on.replay()
    b = on.results()
    on.close()
    assert a["status"] == 0 and b["status"] == 0
    assert np.array_equal(a["scores"], b["scores"])
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    assert b["counters"][2] > 0                          # prefetch moved rows
    assert b["counters"][0] < a["counters"][0]           # and the guaranteed recall had less to do
    for got in (a, b):
        _check_invariants(inp, host_kv, got)
    # the selected rows are the same bits either way
    rows, cols = np.nonzero(a["topk_idx"] >= 0)
    ra = a["pool"]["gpu_kv"][a["topk_slot"][rows, cols]]
    rb = b["pool"]["gpu_kv"][b["topk_slot"][rows, cols]]
    assert np.array_equal(ra, rb)
    _check_topk_tolerance(inp, scores, b, rows=[0, 5])


def test_prefetch_lossless_over_chunk_counts():
    # the prefetch races the scoring of later ranges and the other requests' gathers; whatever
    # the number of ranges, the selection and the selected rows must not change
    announce("prefetch lossless, chunk counts 1..8")
    cfg = gen.DecodeConfig("c", 4, 9000, 256, "int", False, 0.5, 6, reserve=1500,
                           prefetch=True, seed=53)
    inp, host_kv, scores, idx, pool = _setup(cfg)
    moved = 0
    for n_chunks in range(1, 9):
        pf = dict(n_chunks=n_chunks, n_sample=1024, percentile=96.0, cap=512, cap_div=16)
        rn = DecodeRunner(inp, pool, host_kv, prefetch=True, pf=pf)
        rn.run_eager()
        got = rn.results()
        rn.close()
        assert got["status"] == 0, n_chunks
        assert np.array_equal(got["topk_idx"], idx), n_chunks
        for r in range(len(inp.key_len)):
            L = int(inp.key_len[r])
            assert np.array_equal(got["scores"][r, :L].astype(np.float64), scores[r]), (n_chunks, r)
        _check_invariants(inp, host_kv, got)
        moved += int(got["counters"][2])
    assert moved > 0


def test_ranged_prefetch_share_passes_on():
    # the ranged prefetch's launches share a request's cap cumulatively: ranges 0..c list at
    # most floor(cap_r (c+1) / n) rows.  Request 0 and 2 have their first half resident, so
    # their first ranges have no demand and pass their share on; request 1 has its second half
    # resident, so its demand sits in the first ranges and is held to their shares.
    announce("ranged prefetch: cumulative share of the cap")
    n_req, L, n_chunks, cap = 3, 8192, 4, 100
    cfg = gen.DecodeConfig("share", n_req, L, 256, "int", False, 0.5, 1, seed=59)
    inp = gen.make_decode_inputs(cfg)
    host_kv = gen.fill_latent_rows(cfg.seed, np.empty((inp.n_host, 576), np.uint16))
    scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
    idx = oracle.topk_rows(scores, cfg.topk)
    half = L // 2
    resident = [np.arange(half), np.arange(half, L), np.arange(half)]
    n_res = n_req * half
    n_gpu = n_res + 6000
    rng = np.random.default_rng(59)
    hosts = np.concatenate([inp.req_to_host[inp.key_begin[r] + resident[r]] for r in range(n_req)])
    slots = rng.permutation(n_gpu)[:n_res]
    free = np.ones(n_gpu, np.uint8)
    priority = np.full(n_gpu, -1, np.int32)
    to_host = np.full(n_gpu, gen.INF, np.int32)
    h2g = np.full(inp.n_host, gen.INF, np.int32)
    free[slots], to_host[slots], h2g[hosts] = 0, hosts, slots
    priority[slots] = rng.permutation(n_res).astype(np.int32)
    gpu_kv = np.full((n_gpu, 576), gen.POISON, np.uint16)
    gpu_kv[slots] = host_kv[hosts]
    pool = gen.PoolArrays(free, priority, to_host, h2g, np.full(n_gpu, -1, np.int32), gpu_kv,
                          step_id=n_res + 1)
    theta = np.array([np.quantile(s, 0.97) for s in scores], np.float32)
    span = -(-L // n_chunks)
    want_demand = want_moved = 0
    for r in range(n_req):
        hosts_r = inp.req_to_host[inp.key_begin[r] + np.arange(L)]
        elig = (scores[r] > theta[r]) & (h2g[hosts_r] == gen.INF)
        per_range = [int(elig[c * span:(c + 1) * span].sum()) for c in range(n_chunks)]
        over = [int((scores[r][c * span:(c + 1) * span] > theta[r]).sum()) for c in range(n_chunks)]
        assert max(over) <= 1024                # every workgroup lists all of its own
        cap_r, listed = min(cap, L), 0
        for c, e in enumerate(per_range):
            listed += min(e, cap_r * (c + 1) // n_chunks - listed)
        want_demand += sum(per_range)
        want_moved += listed
    pf = dict(n_chunks=n_chunks, cap=cap, cap_div=1)
    rn = DecodeRunner(inp, pool, host_kv, prefetch="ranged", pf=pf, theta=theta)
    try:
        rn.run_eager()
        got = rn.results()
    finally:
        rn.close()
    assert got["status"] == 0
    assert np.array_equal(got["topk_idx"], idx)
    assert int(got["counters"][1]) == want_demand
    assert int(got["counters"][2]) == want_moved
    assert want_moved > n_req * cap // 2         # more than fixed halves would have moved
    _check_invariants(inp, host_kv, got)


@pytest.mark.parametrize("prefetch", [False, "ranged"])
def test_decode_step_paged_keys_matches_contiguous(prefetch):
    # the decode step over a paged indexer-K cache (128-token pages in a random order, general
    # FP8 keys with scales, the threshold sampled from the pages too): scores, selection, misses
    # and every pool array bit for bit those of the step over the contiguous cache, and the
    # selection the oracle's up to the tolerance
    announce("decode step paged keys, prefetch", prefetch)
    cfg = gen.DecodeConfig("pg", 5, 0, 256, "general", True, 0.5, 4, reserve=800,
                           prefetch=bool(prefetch), seed=61)
    inp = gen.make_decode_inputs(cfg, lengths=[9000, 1, 4500, 128, 3333])
    host_kv = gen.fill_latent_rows(cfg.seed, np.empty((inp.n_host, 576), np.uint16))
    scores = oracle.index_scores(inp.q, inp.w, inp.k, inp.k_scale, inp.key_begin, inp.key_len)
    idx = oracle.topk_rows(scores, cfg.topk)
    pool = gen.make_pool_state(inp, idx, host_kv)
    pk = gen.page_key_cache(inp.k, inp.k_scale, inp.key_begin, inp.key_len, 128, seed=3)
    pf = dict(n_chunks=3, n_sample=1024, percentile=90.0, cap=400, cap_div=16)
    got = []
    for pages in (None, pk):
        rn = DecodeRunner(inp, pool, host_kv, prefetch=prefetch, pf=pf, pages=pages)
        try:
            rn.capture()
            rn.replay()
            got.append(rn.results())
        finally:
            rn.close()
    a, b = got
    assert a["status"] == b["status"] == 0
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    for r, L in enumerate(inp.key_len):                 # entries past a request's length are unset
        assert np.array_equal(a["scores"][r, :L], b["scores"][r, :L]), r
    if not prefetch:                       # which candidates win the prefetch depends on timing
        for key in ("topk_slot", "miss_host", "miss_slot", "counters"):
            assert np.array_equal(a[key], b[key]), key
        for n in a["pool"]:
            assert np.array_equal(a["pool"][n], b["pool"][n]), n
    else:
        assert b["counters"][2] > 0
    _check_topk_tolerance(inp, scores, b, rows=range(len(inp.key_len)))
    _check_invariants(inp, host_kv, b)
