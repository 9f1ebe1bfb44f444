"""Pins of the oracle's range prefetch (oracle/prefetch.py) against what the ECHO page and the
mathematics fix: a worked example derived by hand (tests/golden/range_prefetch_example.txt),
the thresholds that reduce to closed forms (+inf and NaN move nothing; -inf with room to spare
moves every non-resident token), the structure of what moves (a token-order prefix of each
range's qualifying tokens, into distinct slots that were free), the pool invariants, and the
page's losslessness (§6.1): a whole step with the prefetch selects the same tokens and ends
with the same selected rows resident as a step without it."""

import os

import numpy as np
import pytest

import oracle
from oracle import prefetch as pfo
from dsa_indexer_top_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "range_prefetch_example.txt")


def _parse_int(v):
    return int(oracle.INF) if v == "inf" else int(v)


def _load_example():
    f = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            key, _, val = line.partition(" ")
            f[key] = val
    n_gpu, n_host = int(f["n_gpu"]), int(f["n_host"])
    st = oracle.PoolState.empty(n_gpu, n_host)
    st.free[:] = [int(v) for v in f["free"].split()]
    st.to_host[:] = [_parse_int(v) for v in f["to_host"].split()]
    st.priority[:] = [int(v) for v in f["priority"].split()]
    for s, h in enumerate(st.to_host):
        if h != oracle.INF:
            st.host_to_gpu[h] = s
    ex = dict(state=st,
              key_begin=np.array(f["key_begin"].split(), np.int64),
              key_len=np.array(f["key_len"].split(), np.int32),
              req_to_host=np.array(f["req_to_host"].split(), np.int32),
              scores=[np.array(p.split(), np.float64) for p in f["scores"].split("|")],
              theta=np.array([float(v) for v in f["theta"].split()], np.float32),
              cap=int(f["cap"]), cap_div=int(f["cap_div"]), range=int(f["range"]),
              moved=[tuple(int(v) for v in m.split(",")) for m in f["moved"].split()],
              demand=np.array(f["demand"].split(), np.int64),
              free_after=np.array(f["free_after"].split(), np.uint8))
    return ex


def _host_rows(n_host, seed=3):
    return gen.fill_latent_rows(seed, np.empty((n_host, 576), np.uint16))


def test_worked_example():
    ex = _load_example()
    st = ex["state"]
    host_kv = _host_rows(st.n_host)
    new, moved, demand = oracle.range_prefetch(ex["scores"], ex["theta"], ex["key_begin"],
                                               ex["key_len"], ex["req_to_host"], st, host_kv,
                                               ex["cap"], ex["cap_div"], ex["range"])
    assert moved == ex["moved"]
    assert np.array_equal(demand, ex["demand"])
    assert np.array_equal(new.free, ex["free_after"])
    for r, s, h, slot in moved:
        assert new.priority[slot] == 0 and new.to_host[slot] == h and new.host_to_gpu[h] == slot
        assert np.array_equal(new.gpu_kv[slot], host_kv[h])
    # the slots that held tokens before are untouched, and the input state is not modified
    assert new.to_host[0] == 2 and new.to_host[3] == 9 and new.priority[3] == 7
    assert st.free.sum() == 12
    oracle.check_pool_invariants(new, host_kv)


def test_request_cap_and_shares():
    assert pfo.request_cap(0, 10, 1, 128) == 0
    assert pfo.request_cap(65536, 2048, 64, 512) == 1024        # ceil(65536 / 64)
    assert pfo.request_cap(131072, 2048, 64, 8192) == 2048      # the cap
    assert pfo.request_cap(1000, 10 ** 6, 1, 8192) == 128       # 128 in its one range
    assert pfo.request_cap(1, 5, 1000, 128) == 1                # ceil(1 / 1000) = 1
    # shares: consecutive, differing by at most one, adding up to c, for any c and n
    for c in (0, 1, 3, 7, 64, 127, 128, 1000):
        for n in (1, 2, 3, 4, 7, 128):
            if c > 128 * n:
                continue
            sh = [pfo.range_share(c, n, x) for x in range(n)]
            assert sum(m for _, m in sh) == c
            assert all(sh[x][0] + sh[x][1] == sh[x + 1][0] for x in range(n - 1))
            assert max(m for _, m in sh) - min(m for _, m in sh) <= 1
            assert max(m for _, m in sh) <= 128


def _random_case(seed, n_rows=5, n_gpu=400, resident=0.3, free=0.5):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 300, n_rows).astype(np.int32)
    lens[0] = 0
    kb = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    n_k = int(lens.sum())
    n_host = n_k + 50
    r2h = rng.permutation(n_host)[:n_k].astype(np.int32)
    st = oracle.PoolState.empty(n_gpu, n_host)
    occ = rng.permutation(n_gpu)[: int(n_gpu * (1 - free))]
    hosts = rng.permutation(n_host)[: len(occ)]
    # a share of the requests' tokens resident, the rest of the occupied slots other rows
    tok_hosts = r2h[rng.random(n_k) < resident]
    hosts = np.concatenate([tok_hosts, np.setdiff1d(hosts, tok_hosts)])[: len(occ)]
    st.free[occ] = 0
    st.to_host[occ] = hosts
    st.host_to_gpu[hosts] = occ
    st.priority[occ] = rng.permutation(len(occ)) + 1
    host_kv = _host_rows(n_host, seed)
    st.gpu_kv[occ] = host_kv[hosts]
    scores = [np.round(rng.standard_normal(L) * 4) / 4 for L in lens]     # ties on purpose
    theta = rng.standard_normal(n_rows).astype(np.float32)
    return st, kb, lens, r2h, scores, theta, host_kv


@pytest.mark.parametrize("seed", range(6))
def test_structure_of_what_moves(seed):
    st, kb, lens, r2h, scores, theta, host_kv = _random_case(seed)
    cap, cap_div, R = 40, 7, 64
    new, moved, demand = oracle.range_prefetch(scores, theta, kb, lens, r2h, st, host_kv, cap,
                                               cap_div, R)
    oracle.check_pool_invariants(new, host_kv)
    free_before = set(np.flatnonzero(st.free == 1).tolist())
    slots = [m[3] for m in moved]
    assert len(set(slots)) == len(slots) and set(slots) <= free_before
    # the free slots are taken in ascending order along (request, range, rank)
    assert slots == sorted(slots)
    by_range = {}
    for r, s, h, slot in moved:
        by_range.setdefault((r, s // R), []).append(s)
    for r in range(len(lens)):
        L = int(lens[r])
        qual_all = [s for s in range(L) if np.float32(scores[r][s]) > theta[r]
                    and st.host_to_gpu[r2h[kb[r] + s]] == oracle.INF]
        assert demand[r] == len(qual_all)
        c = pfo.request_cap(L, cap, cap_div, R)
        n_rng = -(-L // R)
        assert sum(len(v) for (rr, _), v in by_range.items() if rr == r) <= c
        for x in range(n_rng):
            qual = [s for s in qual_all if s // R == x]
            got = by_range.get((r, x), [])
            # a prefix of the range's qualifying tokens in token order, within its share
            assert got == qual[: len(got)] and len(got) <= pfo.range_share(c, n_rng, x)[1]
    # nothing resident before changed
    occ = np.flatnonzero(st.free == 0)
    assert np.array_equal(new.to_host[occ], st.to_host[occ])
    assert np.array_equal(new.priority[occ], st.priority[occ])


def test_infinite_and_nan_thresholds_move_nothing():
    st, kb, lens, r2h, scores, _, host_kv = _random_case(11)
    for t in (np.inf, np.nan):
        theta = np.full(len(lens), t, np.float32)
        new, moved, demand = oracle.range_prefetch(scores, theta, kb, lens, r2h, st, host_kv,
                                                   10 ** 6, 1, 128)
        assert moved == [] and demand.sum() == 0
        for a, b in zip((new.free, new.priority, new.to_host, new.host_to_gpu, new.gpu_kv),
                        (st.free, st.priority, st.to_host, st.host_to_gpu, st.gpu_kv)):
            assert np.array_equal(a, b)


def test_minus_infinity_with_room_moves_every_non_resident_token():
    # one range per request (R >= L <= 128) and caps above L: every token that is not resident
    # moves, and afterwards every token of every request is resident with its row
    st, kb, lens, r2h, scores, _, host_kv = _random_case(12, n_gpu=2000, free=0.8)
    lens = np.minimum(lens, 128).astype(np.int32)
    theta = np.full(len(lens), -np.inf, np.float32)
    new, moved, demand = oracle.range_prefetch(scores, theta, kb, lens, r2h, st, host_kv,
                                               10 ** 6, 1, 128)
    hosts = np.concatenate([r2h[kb[r]: kb[r] + lens[r]] for r in range(len(lens))]).astype(np.int64)
    non_res = int((st.host_to_gpu[hosts] == oracle.INF).sum())
    assert len(moved) == non_res == demand.sum()
    oracle.check_pool_invariants(new, host_kv, hosts, new.host_to_gpu[hosts])


@pytest.mark.parametrize("seed", [21, 22])
def test_whole_step_is_lossless(seed):
    # a full pool with a reserve of free slots; the EMA-like threshold from a percentile
    cfg = gen.DecodeConfig("t", 3, 0, 32, "int", False, 0.5, 4, seed=seed, reserve=200)
    inp = gen.make_decode_inputs(cfg, lengths=[700, 300, 1])
    host_kv = gen.fill_latent_rows(seed, np.empty((inp.n_host, 576), np.uint16))
    scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
    idx = oracle.topk_rows(scores, 32)
    pool = gen.make_pool_state(inp, idx, host_kv)
    st = oracle.PoolState(pool.free, pool.priority, pool.to_host, pool.host_to_gpu,
                          pool.indices_buf, pool.gpu_kv)
    theta = np.array([np.quantile(s, 0.9) if len(s) else np.nan for s in scores], np.float32)
    _, idx0, final0, res0 = oracle.decode_step(inp.q, inp.w, inp.k, None, inp.key_begin,
                                               inp.key_len, inp.req_to_host, st, host_kv, 32,
                                               pool.step_id)
    _, idx1, mid, moved, demand, final1, res1 = oracle.decode_step_prefetched(
        inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len, inp.req_to_host, st, host_kv, 32,
        pool.step_id, theta, 64, 4, 128)
    assert len(moved) > 0
    assert np.array_equal(idx0, idx1)
    for fin, res in ((final0, res0), (final1, res1)):
        assert res.status == 0
        rows, cols = np.nonzero(idx1 >= 0)
        hosts = inp.req_to_host[inp.key_begin[rows] + idx1[rows, cols]]
        oracle.check_pool_invariants(fin, host_kv, hosts, res.topk_slot[rows, cols])
    # prefetched rows the step selected are hits: fewer misses with the prefetch
    assert res1.n_miss <= res0.n_miss
    sel = set(map(int, inp.req_to_host[inp.key_begin[rows] + idx1[rows, cols]]))
    hit_pf = sum(1 for m in moved if m[2] in sel)
    assert res1.n_miss == res0.n_miss - hit_pf
