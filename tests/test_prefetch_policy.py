"""Pins of the CPU model of the fused prefetch kernel's documented policy
(tests/prefetch_policy.py; ranges, 128 candidates per range, caps scaled to the free slots,
per-request places claimed first come), which the GPU tests of that kernel use on top of the
page's contract (oracle/prefetch.py): a worked example derived by hand
(tests/golden/range_prefetch_policy_example.txt), the caps scaled by hand, the structure of what
moves on random pools, every canonical outcome satisfying the page's contract, and the outcome
checker accepting another valid outcome and rejecting planted mistakes."""

import os

import numpy as np
import pytest

import oracle
import prefetch_policy as pol
from dsa_indexer_top_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "range_prefetch_policy_example.txt")


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
    return dict(state=st,
                key_begin=np.array(f["key_begin"].split(), np.int64),
                key_len=np.array(f["key_len"].split(), np.int32),
                req_to_host=np.array(f["req_to_host"].split(), np.int32),
                scores=[np.array(p.split(), np.float64) for p in f["scores"].split("|")],
                theta=np.array([float(v) for v in f["theta"].split()], np.float32),
                cap=int(f["cap"]), cap_div=int(f["cap_div"]), range=int(f["range"]),
                moved=[tuple(int(v) for v in m.split(",")) for m in f["moved"].split()],
                caps=[int(v) for v in f["caps"].split()],
                offsets=[int(v) for v in f["offsets"].split()],
                demand=np.array(f["demand"].split(), np.int64),
                free_after=np.array(f["free_after"].split(), np.uint8))


def _host_rows(n_host, seed=3):
    return gen.fill_latent_rows(seed, np.empty((n_host, 576), np.uint16))


def _apply(st, host_kv, moves):
    return oracle.apply_prefetch(st, host_kv, moves)


def test_worked_example():
    ex = _load_example()
    st = ex["state"]
    host_kv = _host_rows(st.n_host)
    new, moved, demand, info = pol.policy_prefetch(ex["scores"], ex["theta"], ex["key_begin"],
                                                   ex["key_len"], ex["req_to_host"], st, host_kv,
                                                   ex["cap"], ex["cap_div"], ex["range"])
    assert moved == ex["moved"]
    assert list(info["cap"]) == ex["caps"] and list(info["offset"]) == ex["offsets"]
    assert np.array_equal(demand, ex["demand"])
    assert np.array_equal(new.free, ex["free_after"])
    assert st.free.sum() == 12                       # the input state is not modified
    oracle.check_pool_invariants(new, host_kv)
    pol.check_policy_outcome(st, new, host_kv, info)
    # the policy's outcome is one the page allows
    bound = oracle.prefetch_bound(ex["key_len"], ex["cap"], ex["cap_div"], st.n_gpu)
    oracle.check_prefetch_contract(st, new, host_kv, info["eligible"], bound)
    # another valid outcome: r0's range 1 stops after s2 and range 2 moves s4; places permuted
    # between ranges
    alt = _apply(st, host_kv, [(4, 1), (7, 4), (11, 2), (3, 6), (8, 5), (13, 12), (14, 10),
                               (16, 11)])
    pol.check_policy_outcome(st, alt, host_kv, info)
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
            pol.check_policy_outcome(st, b, host_kv, info)
            raise RuntimeError("not caught: " + what)
    b = _apply(st, host_kv, canon)
    b.gpu_kv[10, 0] ^= 1
    with pytest.raises(AssertionError):
        pol.check_policy_outcome(st, b, host_kv, info)


def test_caps_scaled_to_the_free_slots():
    # c_r = min(cap, ceil(L / cap_div), n_gpu); scaled by F / C when they add up to C > F
    assert pol.request_caps([5, 3, 0, 8], 3, 1, 12, 14) == ([3, 3, 0, 3], [3, 3, 0, 3])
    assert pol.request_caps([5, 3, 0, 8], 3, 1, 5, 14) == ([3, 3, 0, 3], [1, 1, 0, 1])
    assert pol.request_caps([65536] * 8, 2048, 64, 16384, 65536)[1] == [1024] * 8
    assert pol.request_caps([65536] * 8, 2048, 64, 4000, 65536)[1] == [500] * 8
    assert pol.request_caps([10 ** 6], 10 ** 7, 1, 10 ** 6, 2048)[0] == [2048]   # at most N_G
    assert pol.request_caps([1], 5, 1000, 10, 10)[0] == [1]                       # ceil(1/1000)


def random_case(seed, n_rows=5, n_gpu=400, resident=0.3, free=0.5):
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
    st, kb, lens, r2h, scores, theta, host_kv = random_case(seed)
    cap, cap_div, R = 40, 7, 64
    new, moved, demand, info = pol.policy_prefetch(scores, theta, kb, lens, r2h, st, host_kv,
                                                   cap, cap_div, R, per_range=5)
    oracle.check_pool_invariants(new, host_kv)
    pol.check_policy_outcome(st, new, host_kv, info)
    oracle.check_prefetch_contract(st, new, host_kv, info["eligible"],
                                   oracle.prefetch_bound(lens, cap, cap_div, st.n_gpu))
    assert sum(info["cap"]) <= int(st.free.sum())
    for r in range(len(lens)):
        L = int(lens[r])
        qual = [s for s in range(L) if np.float32(scores[r][s]) > theta[r]
                and st.host_to_gpu[r2h[kb[r] + s]] == oracle.INF]
        assert demand[r] == len(qual)
        for x in range(-(-L // R)):                   # each range's first 5 eligible tokens
            qx = [s for s in qual if s // R == x][:5]
            assert [s for s, _ in info["cand"][r].get(x, [])] == qx
        n_cand = sum(len(v) for v in info["cand"][r].values())
        assert len([m for m in moved if m[0] == r]) == min(n_cand, info["cap"][r])
