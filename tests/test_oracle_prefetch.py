"""Pins of the oracle's threshold-prefetch contract (oracle/prefetch.py) against what the ECHO
page fixes (§6.1: tokens scoring strictly above the predicted k-th score that are not resident,
at most a bound in proportion to the context, lossless thanks to the guaranteed recall; §6.3: a
copy stage fed by the scoring): a worked example derived by hand
(tests/golden/prefetch_contract_example.txt), the thresholds that reduce to closed forms (+inf
and NaN move nothing; -inf with room to spare makes every token resident), planted mistakes the
contract checker must reject, and losslessness of a whole step after the greedy outcome and
after random valid outcomes (any eligible subset within the bounds, in any free slots)."""

import os

import numpy as np
import pytest

import oracle
from dsa_indexer_top_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefetch_contract_example.txt")


def _load_example():
    f = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            key, _, val = line.partition(" ")
            f[key] = val
    st = oracle.PoolState.empty(int(f["n_gpu"]), int(f["n_host"]))
    st.free[:] = [int(v) for v in f["free"].split()]
    st.to_host[:] = [int(oracle.INF) if v == "inf" else int(v) for v in f["to_host"].split()]
    st.priority[:] = [int(v) for v in f["priority"].split()]
    for s, h in enumerate(st.to_host):
        if h != oracle.INF:
            st.host_to_gpu[h] = s
    elig = [[tuple(int(v) for v in p.split(",")) for p in part.split()]
            for part in f["eligible"].split("|")]
    return dict(state=st,
                key_begin=np.array(f["key_begin"].split(), np.int64),
                key_len=np.array(f["key_len"].split(), np.int32),
                req_to_host=np.array(f["req_to_host"].split(), np.int32),
                scores=[np.array(p.split(), np.float64) for p in f["scores"].split("|")],
                theta=np.array([float(v) for v in f["theta"].split()], np.float32),
                cap=int(f["cap"]), cap_div=int(f["cap_div"]), eligible=elig,
                bound=[int(v) for v in f["bound"].split()],
                greedy=[tuple(int(v) for v in m.split(",")) for m in f["greedy"].split()])


def _host_rows(n_host, seed=3):
    return gen.fill_latent_rows(seed, np.empty((n_host, 576), np.uint16))


def test_worked_example():
    ex = _load_example()
    st = ex["state"]
    host_kv = _host_rows(st.n_host)
    elig = oracle.prefetch_eligible(ex["scores"], ex["theta"], ex["key_begin"], ex["key_len"],
                                    ex["req_to_host"], st)
    assert elig == ex["eligible"]
    bound = oracle.prefetch_bound(ex["key_len"], ex["cap"], ex["cap_div"], st.n_gpu)
    assert bound == ex["bound"]
    new, moves, elig2, bound2 = oracle.greedy_prefetch(
        ex["scores"], ex["theta"], ex["key_begin"], ex["key_len"], ex["req_to_host"], st, host_kv,
        ex["cap"], ex["cap_div"])
    assert moves == ex["greedy"] and elig2 == elig and bound2 == bound
    assert st.free.sum() == 12                       # the input state is not modified
    for r, s, h, slot in moves:
        assert new.free[slot] == 0 and new.to_host[slot] == h and new.host_to_gpu[h] == slot
        assert new.priority[slot] == 0 and np.array_equal(new.gpu_kv[slot], host_kv[h])
    assert list(np.flatnonzero(new.free == 1)) == [10, 11, 12, 13]
    per = oracle.check_prefetch_contract(st, new, host_kv, elig, bound)
    assert list(per) == [3, 2, 0, 3]
    oracle.check_pool_invariants(new, host_kv)


def test_contract_accepts_other_valid_outcomes_and_rejects_planted_mistakes():
    ex = _load_example()
    st = ex["state"]
    host_kv = _host_rows(st.n_host)
    elig, bound = ex["eligible"], ex["bound"]
    ok = {
        "nothing moved": [],
        "other eligible tokens, other free slots": [(11, 13), (0, 2), (8, 12), (19, 1), (18, 4),
                                                    (17, 5)],
        "bounds reached exactly": [(4, 1), (7, 2), (0, 4), (3, 5), (8, 6), (13, 7), (14, 8),
                                   (19, 9)],
    }
    for what, moves in ok.items():
        oracle.check_prefetch_contract(st, oracle.apply_prefetch(st, host_kv, moves), host_kv,
                                       elig, bound)
    planted = {
        "a token below the threshold (r3 s0, host 12)": [(12, 1)],
        "a token at the threshold (r1 s0 scores 2.0 = theta; its host 9 is also resident)": [(9, 1)],
        "a resident row moved again (host 2)": [(2, 1)],
        "above r3's bound": [(13, 1), (14, 2), (16, 4), (17, 5)],
        "into an occupied slot": [(4, 0)],
    }
    for what, moves in planted.items():
        with pytest.raises(AssertionError):
            oracle.check_prefetch_contract(st, oracle.apply_prefetch(st, host_kv, moves), host_kv,
                                           elig, bound)
            raise RuntimeError("not caught: " + what)
    base = oracle.apply_prefetch(st, host_kv, [(4, 1), (3, 5)])
    mutations = {
        "an eviction": lambda b: (b.free.__setitem__(3, 1), b.to_host.__setitem__(3, oracle.INF),
                                  b.host_to_gpu.__setitem__(9, oracle.INF)),
        "priority not 0": lambda b: b.priority.__setitem__(1, 1),
        "a row byte": lambda b: b.gpu_kv.__setitem__((5, 7), b.gpu_kv[5, 7] ^ 1),
        "HostTokenToGPU not set": lambda b: b.host_to_gpu.__setitem__(4, oracle.INF),
        "indices_buf written": lambda b: b.indices_buf.__setitem__(0, 1),
        "a row outside the prefetched slots": lambda b: b.gpu_kv.__setitem__((12, 0), 0),
    }
    for what, mut in mutations.items():
        b = base.copy()
        mut(b)
        with pytest.raises(AssertionError):
            oracle.check_prefetch_contract(st, b, host_kv, elig, bound)
            raise RuntimeError("not caught: " + what)


def test_bound_in_proportion_to_the_context():
    assert oracle.prefetch_bound([0, 1, 1024, 1025, 131072], 2048, 1024, 10 ** 6) == [0, 1, 1, 2, 128]
    assert oracle.prefetch_bound([131072], 2048, 32, 10 ** 6) == [2048]        # the cap binds
    assert oracle.prefetch_bound([10 ** 6], 10 ** 7, 1, 2048) == [2048]        # at most N_G


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


@pytest.mark.parametrize("seed", range(4))
def test_eligible_by_definition_on_random_pools(seed):
    st, kb, lens, r2h, scores, theta, host_kv = _random_case(seed)
    elig = oracle.prefetch_eligible(scores, theta, kb, lens, r2h, st)
    for r in range(len(lens)):
        want = [(s, int(r2h[kb[r] + s])) for s in range(int(lens[r]))
                if np.float32(scores[r][s]) > theta[r] and st.host_to_gpu[r2h[kb[r] + s]] == oracle.INF]
        assert elig[r] == want
    new, moves, _, bound = oracle.greedy_prefetch(scores, theta, kb, lens, r2h, st, host_kv, 40, 7)
    oracle.check_prefetch_contract(st, new, host_kv, elig, bound)
    oracle.check_pool_invariants(new, host_kv)


def test_infinite_and_nan_thresholds_move_nothing():
    st, kb, lens, r2h, scores, _, host_kv = _random_case(11)
    for t in (np.inf, np.nan):
        theta = np.full(len(lens), t, np.float32)
        new, moves, elig, _ = oracle.greedy_prefetch(scores, theta, kb, lens, r2h, st, host_kv,
                                                     10 ** 6, 1)
        assert moves == [] and all(e == [] for e in elig)
        for a, b in zip((new.free, new.priority, new.to_host, new.host_to_gpu, new.gpu_kv),
                        (st.free, st.priority, st.to_host, st.host_to_gpu, st.gpu_kv)):
            assert np.array_equal(a, b)


def test_minus_infinity_with_room_makes_every_token_resident():
    st, kb, lens, r2h, scores, _, host_kv = _random_case(12, n_gpu=2000, free=0.8)
    theta = np.full(len(lens), -np.inf, np.float32)
    new, moves, elig, _ = oracle.greedy_prefetch(scores, theta, kb, lens, r2h, st, host_kv,
                                                 10 ** 6, 1)
    hosts = np.concatenate([r2h[kb[r]: kb[r] + lens[r]] for r in range(len(lens))]).astype(np.int64)
    assert len(moves) == int((st.host_to_gpu[hosts] == oracle.INF).sum()) > 0
    assert (new.host_to_gpu[hosts] != oracle.INF).all()
    oracle.check_pool_invariants(new, host_kv, hosts, new.host_to_gpu[hosts])


def _random_valid_moves(rng, st, elig, bound):
    """Any eligible subset within the bounds, in random free slots: the space of outcomes a
    first-come-first-served GPU prefetch may produce."""
    free = list(rng.permutation(np.flatnonzero(st.free == 1)))
    moves = []
    for r, lst in enumerate(elig):
        n = int(rng.integers(0, min(len(lst), bound[r]) + 1))
        for i in rng.permutation(len(lst))[:n]:
            if free:
                moves.append((lst[i][1], int(free.pop())))
    return moves


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_whole_step_is_lossless(seed):
    # a full pool with a reserve of free slots; any valid prefetch ahead of the step leaves the
    # selection unchanged, every selected row resident bit for bit, and exactly the prefetched
    # selected tokens fewer misses
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
    assert res0.status == 0
    rows, cols = np.nonzero(idx0 >= 0)
    sel = set(map(int, inp.req_to_host[inp.key_begin[rows] + idx0[rows, cols]]))
    rng = np.random.default_rng(seed)
    greedy, gmoves, elig, bound = oracle.greedy_prefetch(scores, theta, inp.key_begin, inp.key_len,
                                                         inp.req_to_host, st, host_kv, 64, 4)
    outcomes = [(greedy, [(h, sl) for _, _, h, sl in gmoves])]
    for _ in range(4):
        mv = _random_valid_moves(rng, st, elig, bound)
        outcomes.append((oracle.apply_prefetch(st, host_kv, mv), mv))
    assert len(outcomes[0][1]) > 0
    for mid, mv in outcomes:
        oracle.check_prefetch_contract(st, mid, host_kv, elig, bound)
        _, idx1, final1, res1 = oracle.decode_step(inp.q, inp.w, inp.k, None, inp.key_begin,
                                                   inp.key_len, inp.req_to_host, mid, host_kv, 32,
                                                   pool.step_id)
        assert res1.status == 0
        assert np.array_equal(idx0, idx1)
        hosts = inp.req_to_host[inp.key_begin[rows] + idx1[rows, cols]]
        oracle.check_pool_invariants(final1, host_kv, hosts, res1.topk_slot[rows, cols])
        assert res1.n_miss == res0.n_miss - sum(1 for h, _ in mv if h in sel)
