"""Pins of the oracle's range prefetch (oracle/prefetch.py) against what the ECHO page and the
mathematics fix: a worked example derived by hand (tests/golden/range_prefetch_example.txt),
the caps scaled to the free slots by hand, the thresholds that reduce to closed forms (+inf
and NaN move nothing; -inf with room to spare moves every non-resident token), the structure of
what moves, the outcome checker accepting the canonical outcome and other valid ones and
rejecting planted mistakes, the pool invariants, and the page's losslessness (§6.1): a whole
step with the prefetch selects the same tokens and ends with the same selected rows resident
as a step without it."""

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
              caps=[int(v) for v in f["caps"].split()], offsets=[int(v) for v in f["offsets"].split()],
              demand=np.array(f["demand"].split(), np.int64),
              free_after=np.array(f["free_after"].split(), np.uint8))
    return ex


def _host_rows(n_host, seed=3):
    return gen.fill_latent_rows(seed, np.empty((n_host, 576), np.uint16))


def test_worked_example():
    ex = _load_example()
    st = ex["state"]
    host_kv = _host_rows(st.n_host)
    new, moved, demand, info = oracle.range_prefetch(ex["scores"], ex["theta"], ex["key_begin"],
                                                     ex["key_len"], ex["req_to_host"], st, host_kv,
                                                     ex["cap"], ex["cap_div"], ex["range"])
    assert moved == ex["moved"]
    assert list(info["cap"]) == ex["caps"] and list(info["offset"]) == ex["offsets"]
    assert np.array_equal(demand, ex["demand"])
    assert np.array_equal(new.free, ex["free_after"])
    for r, s, h, slot in moved:
        assert new.priority[slot] == 0 and new.to_host[slot] == h and new.host_to_gpu[h] == slot
        assert np.array_equal(new.gpu_kv[slot], host_kv[h])
    # the slots that held tokens before are untouched, and the input state is not modified
    assert new.to_host[0] == 2 and new.to_host[3] == 9 and new.priority[3] == 7
    assert st.free.sum() == 12
    oracle.check_pool_invariants(new, host_kv)
    oracle.check_prefetch_outcome(st, new, host_kv, ex["key_begin"], ex["req_to_host"], info)
    # another valid outcome: r0's range 1 stops after s2 and range 2 moves s4; places permuted
    # between ranges
    alt = _apply(st, host_kv, [(4, 1), (7, 4), (11, 2), (3, 6), (8, 5), (13, 12), (14, 10),
                               (16, 11)])
    oracle.check_prefetch_outcome(st, alt, host_kv, ex["key_begin"], ex["req_to_host"], info)
    canon = [(4, 1), (7, 2), (0, 4), (3, 5), (8, 6), (13, 10), (14, 11), (16, 12)]
    planted = {
        "not a prefix of range 1": [(4, 1), (0, 2), (11, 4)] + canon[3:],
        "range 1's slots out of token order": [(4, 1), (7, 4), (0, 2)] + canon[3:],
        "a place that is not among r1's first": canon[:3] + [(3, 5), (8, 7)] + canon[5:],
        "r3 moved too few": canon[:6],
        "a candidate of r3 moved twice": canon + [(13, 13)],
    }
    for what, moves in planted.items():
        b = _apply(st, host_kv, moves)
        with pytest.raises(AssertionError):
            oracle.check_prefetch_outcome(st, b, host_kv, ex["key_begin"], ex["req_to_host"], info)
            raise RuntimeError("not caught: " + what)
    b = _apply(st, host_kv, canon)
    b.gpu_kv[10, 0] ^= 1
    with pytest.raises(AssertionError):
        oracle.check_prefetch_outcome(st, b, host_kv, ex["key_begin"], ex["req_to_host"], info)


def _apply(st, host_kv, moves):
    """st with host rows h placed in slots (h, slot)."""
    b = st.copy()
    for h, slot in moves:
        b.free[slot], b.to_host[slot], b.host_to_gpu[h], b.priority[slot] = 0, h, slot, 0
        b.gpu_kv[slot] = host_kv[h]
    return b


def test_caps_scaled_to_the_free_slots():
    # c_r = min(cap, ceil(L / cap_div), n_gpu); scaled by F / C when they add up to C > F
    assert oracle.request_caps([5, 3, 0, 8], 3, 1, 12, 14) == ([3, 3, 0, 3], [3, 3, 0, 3])
    assert oracle.request_caps([5, 3, 0, 8], 3, 1, 5, 14) == ([3, 3, 0, 3], [1, 1, 0, 1])
    assert oracle.request_caps([65536] * 8, 2048, 64, 16384, 65536)[1] == [1024] * 8
    assert oracle.request_caps([65536] * 8, 2048, 64, 4000, 65536)[1] == [500] * 8
    assert oracle.request_caps([10 ** 6], 10 ** 7, 1, 10 ** 6, 2048)[0] == [2048]   # at most N_G
    assert oracle.request_caps([1], 5, 1000, 10, 10)[0] == [1]                       # ceil(1/1000)


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
    new, moved, demand, info = oracle.range_prefetch(scores, theta, kb, lens, r2h, st, host_kv,
                                                     cap, cap_div, R, per_range=5)
    oracle.check_pool_invariants(new, host_kv)
    oracle.check_prefetch_outcome(st, new, host_kv, kb, r2h, info)
    free_before = np.flatnonzero(st.free == 1)
    assert sum(info["cap"]) <= len(free_before)
    for r in range(len(lens)):
        L = int(lens[r])
        qual = [s for s in range(L) if np.float32(scores[r][s]) > theta[r]
                and st.host_to_gpu[r2h[kb[r] + s]] == oracle.INF]
        assert demand[r] == len(qual)
        # candidates: each range's first 5 qualifying tokens
        for x in range(-(-L // R)):
            qx = [s for s in qual if s // R == x][:5]
            assert [s for s, _ in info["cand"][r].get(x, [])] == qx
        mr = [m for m in moved if m[0] == r]
        n_cand = sum(len(v) for v in info["cand"][r].values())
        assert len(mr) == min(n_cand, info["cap"][r])


def test_infinite_and_nan_thresholds_move_nothing():
    st, kb, lens, r2h, scores, _, host_kv = _random_case(11)
    for t in (np.inf, np.nan):
        theta = np.full(len(lens), t, np.float32)
        new, moved, demand, _ = oracle.range_prefetch(scores, theta, kb, lens, r2h, st, host_kv,
                                                      10 ** 6, 1, 128)
        assert moved == [] and demand.sum() == 0
        for a, b in zip((new.free, new.priority, new.to_host, new.host_to_gpu, new.gpu_kv),
                        (st.free, st.priority, st.to_host, st.host_to_gpu, st.gpu_kv)):
            assert np.array_equal(a, b)


def test_minus_infinity_with_room_moves_every_non_resident_token():
    # caps above L and room to spare: every token that is not resident moves, and afterwards
    # every token of every request is resident with its row
    st, kb, lens, r2h, scores, _, host_kv = _random_case(12, n_gpu=2000, free=0.8)
    lens = np.minimum(lens, 128).astype(np.int32)
    theta = np.full(len(lens), -np.inf, np.float32)
    new, moved, demand, _ = oracle.range_prefetch(scores, theta, kb, lens, r2h, st, host_kv,
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
    _, idx1, mid, moved, demand, _, final1, res1 = oracle.decode_step_prefetched(
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
