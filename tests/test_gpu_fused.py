"""GPU parity of the scoring kernel with the host-gather wave (ECHO page §6.3; the threshold
prefetch of §6.1 done inside the scoring launch) against the oracle's range prefetch
(oracle/prefetch.py): the scores and the pool after the prefetch bit-exact on integer-grid
inputs, for several range lengths, caps, thresholds (including NaN and infinities) and free
lists that run short; a failed pool (status set) moves nothing.  General FP8 with scales: the
scores within tolerance and what moved checked through the properties that define it.  The
whole decode step with the fused prefetch, eager and as one replayed hipGraph, bit-exact against
the oracle's step (the EMA estimate and the sample percentile as thresholds)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import prefetch as pfo
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
    want, moved, demand = oracle.range_prefetch(scores, theta, inp.key_begin, inp.key_len,
                                                inp.req_to_host, st, host_kv, cap, cap_div, R)
    got_sc, got_st, npf, dem, P = _run_standalone(inp, st, host_kv, theta, cap, cap_div, R)
    try:
        for r, s in enumerate(scores):
            assert np.array_equal(got_sc[r, :len(s)].astype(np.float64), s), "scores row %d" % r
        assert npf == len(moved) and dem == int(demand.sum())
        assert_pool_equal(got_st, want, "after the fused prefetch")
        assert (len(moved) > 0) == (free_frac > 0) and demand.sum() > 0
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
    # general FP8 with per-token scales: the scores within 1e-4 T; what moved is, per range, a
    # token-order prefix of the tokens whose GPU score is above the threshold and that were not
    # resident, within the range's share, in distinct slots that were free, taken from the
    # ascending free list in (request, range, rank) order; every moved row equals its host row
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
        tok_of_host = {int(h): (r, s) for r in range(len(lens)) for s in range(lens[r])
                       for h in [inp.req_to_host[inp.key_begin[r] + s]]}
        moved = sorted((tok_of_host[int(got_st.to_host[sl])], int(sl)) for sl in new)
        assert [sl for _, sl in moved] == sorted(sl for _, sl in moved)   # list order
        assert all(got_st.priority[sl] == 0 for _, sl in moved)
        offset, n_dem = 0, 0
        for r in range(len(lens)):
            L = lens[r]
            c, n_rng = pfo.request_cap(L, cap, cap_div, R), -(-L // R)
            qual = [s for s in range(L) if got_sc[r, s] > theta[r]
                    and st.host_to_gpu[inp.req_to_host[inp.key_begin[r] + s]] == oracle.INF]
            n_dem += len(qual)
            for x in range(n_rng):
                first, share = pfo.range_share(c, n_rng, x)
                qx = [s for s in qual if s // R == x]
                gx = [(s, sl) for (rr, s), sl in moved if rr == r and s // R == x]
                assert [s for s, _ in gx] == qx[:len(gx)] and len(gx) <= share
                # each range's rows sit in its own entries of the free list, in rank order
                for i, (_, sl) in enumerate(gx):
                    assert free_list[offset + first + i] == sl
                if len(gx) < min(len(qx), share):
                    assert offset + first + len(gx) >= len(free_list)   # the list ran out
            offset += c
        assert dem == n_dem
    finally:
        P.hostbuf.close()


def _oracle_state(pool):
    return oracle.PoolState(pool.free.copy(), pool.priority.copy(), pool.to_host.copy(),
                            pool.host_to_gpu.copy(), pool.indices_buf.copy(), pool.gpu_kv.copy())


def _as_state(d):
    return oracle.PoolState(d["free"], d["priority"], d["to_host"], d["host_to_gpu"],
                            d["indices_buf"], d["gpu_kv"])


@pytest.mark.parametrize("given_theta", [True, False])
@pytest.mark.parametrize("lens,k,R,reserve", [([3000, 700, 1, 0], 64, 256, 300),
                                              ([5000, 4096], 256, 128, 1500),
                                              ([2000, 900], 128, 256, 0)])     # a full pool
def test_decode_step_fused_exact(lens, k, R, reserve, given_theta):
    # the whole step with the fused prefetch: the threshold given (the EMA estimate) or the
    # sample percentile; selection, slots, miss lists, counters and the pool after the step
    # bit-exact against the oracle's step; then replayed as one graph from the same start
    announce("decode step fused", lens, k, R, reserve, "given theta" if given_theta else "sample theta")
    cfg = gen.DecodeConfig("fzd", len(lens), 0, k, "int", False, 0.5, 4, seed=330 + k,
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
    cap, cap_div = 200, 8
    st0 = _oracle_state(pool)
    _, want_idx, mid, moved, demand, want_state, res = oracle.decode_step_prefetched(
        inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len, inp.req_to_host, st0, host_kv, k,
        pool.step_id, theta, cap, cap_div, R, reserve=reserve)
    assert (len(moved) > 0) == (reserve > 0) and res.status == 0
    pf = dict(cap=cap, cap_div=cap_div, range=R)
    rn = DecodeRunner(inp, pool, host_kv, prefetch="fused", pf=pf, reserve=reserve,
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
            assert np.array_equal(got["topk_slot"], res.topk_slot), mode
            assert np.array_equal(got["miss_host"], res.miss_host), mode
            assert np.array_equal(got["miss_slot"], res.miss_slot), mode
            assert list(got["counters"][:3]) == [res.n_miss, int(demand.sum()), len(moved)], mode
            assert_pool_equal(_as_state(got["pool"]), want_state, mode)
    finally:
        rn.close()
