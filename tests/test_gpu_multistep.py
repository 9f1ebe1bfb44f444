"""GPU parity of several decode steps in a row against the oracle's loop (oracle/multistep.py):
every step appends one token per request (echo_decode_append: key, host index, length, the
latent row written through to the pinned host backup, a GPU slot by the canonical
allocation), then runs the decode step with the EMA estimate of the k-th score
(echo_decode_select with theta_ema).  Integer-grid inputs: bit-exact scores, selections,
k-th scores, pool contents, K cache and host rows after every step; the estimate within
float32 rounding of the exact recursion.  With prefetch against the EMA estimate, ranged or
fused into the scoring launch: the same selections and resident rows (lossless), nothing
prefetched before the first estimate."""

import numpy as np
import pytest

import oracle
from oracle import multistep as ms
from dsa_indexer_top_amd import binding as B, inputs as gen
from dsa_indexer_top_amd.runner import LoopRunner
from gpu_util import announce, assert_pool_equal

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _oracle_start(m):
    cache = ms.KeyCache(m.k.copy(), None if m.k_scale is None else m.k_scale.copy(),
                        m.key_begin.copy(), m.key_len.copy(), m.req_to_host.copy(), m.capacity)
    st = oracle.PoolState(m.pool.free.copy(), m.pool.priority.copy(), m.pool.to_host.copy(),
                          m.pool.host_to_gpu.copy(), m.pool.indices_buf.copy(),
                          m.pool.gpu_kv.copy())
    return cache, st


def _as_state(d):
    return oracle.PoolState(d["free"], d["priority"], d["to_host"], d["host_to_gpu"],
                            d["indices_buf"], d["gpu_kv"])


def _theta_close(got, want, kth_hist):
    # the library rounds every update to float32; the oracle keeps the exact value
    scale = np.max(np.abs(np.array(kth_hist)), axis=0) + 1e-30
    assert (np.abs(got.astype(np.float64) - want) <= 2.0 ** -20 * scale).all(), (got, want)


@pytest.mark.parametrize("B_,L,T,k,n_gpu,mode", [
    (3, 300, 5, 32, 120, "eager"), (2, 1100, 4, 256, 600, "eager"),
    (3, 300, 5, 32, 120, "graph"), (2, 1100, 4, 256, 600, "graph")])
def test_multistep_exact(B_, L, T, k, n_gpu, mode):
    # graph: the stamp on the device, advance + append + step captured once and replayed for
    # every step, with the step's uploads and the checks (eager work) between replays
    announce("multistep exact", B_, L, T, k, n_gpu, mode)
    m, host_kv = gen.make_multistep_inputs(B_, L, T, n_gpu, seed=31 + L)
    cache, st = _oracle_start(m)
    _, _, hk_want, recs = ms.decode_loop(cache, st, host_kv, m.steps, k)
    rn = LoopRunner(m, host_kv, k, device_step=mode == "graph")
    try:
        if mode == "graph":
            rn.capture()
        kth_hist = []
        for t, s in enumerate(m.steps):
            if mode == "graph":
                rn.replay_step(s)
            else:
                rn.run_step(s)
            got = rn.results()
            rec = recs[t]
            assert got["status"] == 0, "step %d status %d" % (t, got["status"])
            assert list(got["key_len"]) == [L + t + 1] * B_
            assert np.array_equal(got["new_slot"], rec.new_slot), "step %d new slots" % t
            for r in range(B_):
                n = L + t + 1
                assert np.array_equal(got["scores"][r, :n].astype(np.float64), rec.scores[r]), \
                    "step %d scores row %d" % (t, r)
            assert np.array_equal(got["topk_idx"], rec.idx), "step %d selection" % t
            assert np.array_equal(got["kth"].astype(np.float64), rec.kth), "step %d k-th" % t
            kth_hist.append(rec.kth)
            _theta_close(got["theta"], rec.theta_next, kth_hist)
            assert int(got["counters"][0]) == rec.result.n_miss
            assert np.array_equal(got["topk_slot"], rec.result.topk_slot)
            assert np.array_equal(got["miss_host"], rec.result.miss_host)
            assert np.array_equal(got["miss_slot"], rec.result.miss_slot)
            assert_pool_equal(_as_state(got["pool"]), rec.state, "step %d" % t)
        cache_T, _, _, _ = ms.decode_loop(*_oracle_start(m), host_kv, m.steps, k)
        assert np.array_equal(got["k"], cache_T.k)
        assert np.array_equal(got["req_to_host"], cache_T.req_to_host)
        assert np.array_equal(got["host_kv"], hk_want)           # write-through of every token
    finally:
        rn.close()


def test_multistep_general_fp8_with_scales():
    announce("multistep general fp8")
    B_, L, T, k = 3, 500, 4, 64
    m, host_kv = gen.make_multistep_inputs(B_, L, T, 240, grid="general", k_scale=True, seed=41)
    cache, st = _oracle_start(m)
    cache_T, _, hk_want, recs = ms.decode_loop(cache, st, host_kv, m.steps, k)
    rn = LoopRunner(m, host_kv, k)
    try:
        for t, s in enumerate(m.steps):
            rn.run_step(s)
            got = rn.results()
            assert got["status"] == 0
            n = L + t + 1
            kb = m.key_begin
            for r in range(B_):
                sl = slice(r, r + 1)
                T_ = oracle.error_scale(s["q"][sl], s["w"][sl], cache_T.k, cache_T.k_scale,
                                        kb[sl], np.array([n], np.int32))[0]
                err = np.abs(got["scores"][r, :n].astype(np.float64) - recs[t].scores[r])
                assert (err <= TOL * T_).all(), "step %d row %d" % (t, r)
            # the step's own selection is resident with the host rows
            idx = got["topk_idx"]
            rows, cols = np.nonzero(idx >= 0)
            hosts = got["req_to_host"][kb[rows] + idx[rows, cols]]
            oracle.check_pool_invariants(_as_state(got["pool"]), got["host_kv"], hosts,
                                         got["topk_slot"][rows, cols])
        assert np.array_equal(got["k_scale"], cache_T.k_scale)
        assert np.array_equal(got["host_kv"], hk_want)
    finally:
        rn.close()


@pytest.mark.parametrize("mode", ["ranged", "fused"])
def test_multistep_prefetch_against_ema_is_lossless(mode):
    announce("multistep %s prefetch with EMA threshold" % mode)
    B_, L, T, k = 3, 2000, 5, 64
    # free room for prefetch: prefetch never evicts
    m, host_kv = gen.make_multistep_inputs(B_, L, T, 2400, seed=43, reserve=1200)
    cache, st = _oracle_start(m)
    _, _, _, recs = ms.decode_loop(cache, st, host_kv, m.steps, k)
    rn = LoopRunner(m, host_kv, k, prefetch=mode, pf=dict(n_chunks=2, cap=256, cap_div=8))
    moved = 0
    try:
        for t, s in enumerate(m.steps):
            rn.run_step(s)
            got = rn.results()
            assert got["status"] == 0
            assert np.array_equal(got["topk_idx"], recs[t].idx), "step %d selection" % t
            assert np.array_equal(got["kth"].astype(np.float64), recs[t].kth)
            if t == 0:
                assert int(got["counters"][2]) == 0, "prefetched before any estimate"
            moved += int(got["counters"][2])
            idx = got["topk_idx"]
            rows, cols = np.nonzero(idx >= 0)
            hosts = got["req_to_host"][m.key_begin[rows] + idx[rows, cols]]
            oracle.check_pool_invariants(_as_state(got["pool"]), got["host_kv"], hosts,
                                         got["topk_slot"][rows, cols])
        assert moved > 0, "the estimate never triggered a prefetch"
    finally:
        rn.close()


@pytest.mark.parametrize("mode", ["ranged", "fused"])
def test_multistep_full_pool_prefetch_with_reserve(mode):
    # the pool starts full; each step's guaranteed recall leaves free room for the next
    # step's prefetch: the loop without prefetch equals the oracle's loop with that reserve
    # bit for bit, and with prefetch rows move in steady state while the selections stay
    announce("multistep full pool, reserve for %s prefetch" % mode)
    B_, L, T, k, R = 3, 2000, 5, 64, 300
    m, host_kv = gen.make_multistep_inputs(B_, L, T, 900, seed=47, drift=0.05)
    cache, st = _oracle_start(m)
    _, _, _, recs = ms.decode_loop(cache, st, host_kv, m.steps, k, reserve=R)
    plain = LoopRunner(m, host_kv, k, device_step=True, reserve=R)
    try:
        plain.capture()
        for t, s in enumerate(m.steps):
            plain.replay_step(s)
            got = plain.results()
            assert got["status"] == 0
            assert np.array_equal(got["topk_idx"], recs[t].idx)
            assert_pool_equal(_as_state(got["pool"]), recs[t].state, "step %d" % t)
            assert int(got["pool"]["free"].sum()) >= min(R, 900 - B_ * (k + 1))
    finally:
        plain.close()
    pf = LoopRunner(m, host_kv, k, prefetch=mode, pf=dict(n_chunks=2, cap=256, cap_div=8),
                    device_step=True, reserve=R)
    moved = 0
    try:
        pf.capture()
        for t, s in enumerate(m.steps):
            pf.replay_step(s)
            got = pf.results()
            assert got["status"] == 0
            assert np.array_equal(got["topk_idx"], recs[t].idx), "step %d selection" % t
            if t >= 1:
                moved += int(got["counters"][2])
            idx = got["topk_idx"]
            rows, cols = np.nonzero(idx >= 0)
            hosts = got["req_to_host"][m.key_begin[rows] + idx[rows, cols]]
            oracle.check_pool_invariants(_as_state(got["pool"]), got["host_kv"], hosts,
                                         got["topk_slot"][rows, cols])
        assert moved > 0, "no prefetch in a full pool despite the reserve"
    finally:
        pf.close()


def test_append_cache_full_and_bad_host():
    announce("append errors")
    B_, L, T, k = 2, 100, 2, 16
    m, host_kv = gen.make_multistep_inputs(B_, L, T, 64, seed=45)
    rn = LoopRunner(m, host_kv, k)
    try:
        # fill request 1 to capacity: the next append sets the sticky cache-full bit
        rn.key_len[1] = m.capacity
        rn.torch.cuda.synchronize()
        s = dict(m.steps[0])
        rn.load_step(s)
        rn.app.step_id = s["step_id"]
        B.decode_append(rn.app, rn.pool, rn.new_slot, rn.ws_app, rn.main)
        got = rn.results()
        assert got["status"] & B.ST_CACHE_FULL
        assert list(got["key_len"]) == [L + 1, m.capacity]
        # a host index outside the host pool: reported, the pool left untouched
        rn.status.zero_()
        rn.key_len[1] = L
        before = {n: t.clone() for n, t in rn.live.items()}
        rn.torch.cuda.synchronize()
        s2 = dict(m.steps[1])
        s2["new_host"] = np.array([s2["new_host"][0], m.n_host + 5], np.int32)
        rn.load_step(s2)
        B.decode_append(rn.app, rn.pool, rn.new_slot, rn.ws_app, rn.main)
        got = rn.results()
        assert got["status"] & B.ST_BAD_HOST
        for n, t in before.items():
            assert np.array_equal(got["pool"][n], t.cpu().numpy()), n
    finally:
        rn.close()
