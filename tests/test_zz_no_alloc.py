"""The no-allocation pool step (echo_pool_lookup_alloc_static, its workspace a fixed device array
inside the library) against the pool step with a caller workspace (echo_pool_lookup_alloc),
through the C ABI: two calls in a row on one GPU, the second smaller than the first, so that what
the first call left in the shared array must not leak into the second.  Both are also checked
against the oracle's pool step."""

import numpy as np
import pytest
import torch

import oracle
from dsa_indexer_top_amd import binding as B
from gpu_util import announce, dev, host, DevPool, assert_pool_equal

pytestmark = pytest.mark.gpu


def _case(seed, n_gpu, n_host, n_occ, rows, k, L):
    rng = np.random.default_rng(seed)
    st = oracle.PoolState.empty(n_gpu, n_host)
    slots = rng.permutation(n_gpu)[:n_occ]
    hosts = rng.permutation(n_host)[:n_occ]
    st.free[slots] = 0
    st.to_host[slots] = hosts
    st.host_to_gpu[hosts] = slots
    st.priority[slots] = rng.integers(0, 50, n_occ)
    host_kv = rng.integers(0, 1 << 16, (n_host, 576), dtype=np.uint16) & np.uint16(0xBFFF)
    st.gpu_kv[slots] = host_kv[hosts]
    req_to_host = rng.permutation(n_host)[:rows * L].astype(np.int32)
    key_begin = (np.arange(rows) * L).astype(np.int64)
    sel = np.full((rows, k), -1, np.int32)
    for r in range(rows):
        m = min(k if r % 3 else int(rng.integers(0, k + 1)), L)
        sel[r, :m] = np.sort(rng.permutation(L)[:m])
    # a share of the selection resident, so that hits are protected and misses evict
    flat = req_to_host[(key_begin[:, None] + np.maximum(sel, 0))[sel >= 0]]
    return st, host_kv, sel, key_begin, req_to_host, flat


def _run(st, host_kv, sel, kb, r2h, step_id, static):
    dp = DevPool(st.free, st.priority, st.to_host, st.host_to_gpu, st.indices_buf, st.gpu_kv, host_kv)
    n_rows, k = sel.shape
    topk_slot = torch.full((n_rows, k), -9, dtype=torch.int32, device="cuda")
    miss_host = torch.full((n_rows * k,), -9, dtype=torch.int32, device="cuda")
    miss_slot = torch.full((n_rows * k,), -9, dtype=torch.int32, device="cuda")
    n_miss = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    try:
        if static:
            B.pool_lookup_alloc_static(dp.pool, dev(sel), dev(kb), dev(r2h), step_id, topk_slot,
                                       miss_host, miss_slot, n_miss)
        else:
            ws = torch.empty(B.pool_workspace_bytes(n_rows, k, dp.n_gpu), dtype=torch.uint8,
                             device="cuda")
            B.pool_lookup_alloc(dp.pool, dev(sel), dev(kb), dev(r2h), step_id, topk_slot,
                                miss_host, miss_slot, n_miss, ws)
        B.recall(dp.pool, miss_host, miss_slot, n_miss, n_rows * k)
        torch.cuda.synchronize()
        return dict(state=dp.state(), topk_slot=host(topk_slot), miss_host=host(miss_host),
                    miss_slot=host(miss_slot), n_miss=int(host(n_miss)[0]),
                    status=int(host(dp.status)[0]))
    finally:
        dp.close()


def test_static_scratch_pool_step_matches_workspace_entry_point():
    cases = [dict(seed=71, n_gpu=20000, n_host=90000, n_occ=20000, rows=6, k=700, L=12000),
             dict(seed=72, n_gpu=3000, n_host=9000, n_occ=2500, rows=2, k=300, L=2000)]
    for i, c in enumerate(cases):
        announce("no-alloc pool step, call %d" % (i + 1), c)
        st, host_kv, sel, kb, r2h, _ = _case(**c)
        step_id = 1000 + i
        a = _run(st, host_kv, sel, kb, r2h, step_id, static=False)
        b = _run(st, host_kv, sel, kb, r2h, step_id, static=True)
        want_state, want = oracle.pool_step(st, host_kv, sel, kb, r2h, step_id)
        assert a["status"] == b["status"] == want.status == 0
        for key in ("topk_slot", "miss_host", "miss_slot", "n_miss"):
            assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), (i, key)
        assert_pool_equal(b["state"], a["state"], "static vs workspace, call %d" % (i + 1))
        assert b["n_miss"] == want.n_miss > 0
        assert np.array_equal(b["topk_slot"], want.topk_slot)
        assert_pool_equal(b["state"], want_state, "static vs oracle, call %d" % (i + 1))
