"""GPU parity of echo_pool_lookup_alloc + echo_recall against the oracle's pool step: every
metadata array, every row, per-entry slots, miss lists and status are equal."""

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as hs, HealthCheck

import oracle
from oracle import INF
from dsa_indexer_top_amd import binding as B
from gpu_util import announce, dev, host, DevPool, assert_pool_equal

pytestmark = pytest.mark.gpu


def _random_case(seed, n_gpu, n_host, n_occ, B_rows, k, L, prio_levels=None):
    rng = np.random.default_rng(seed)
    st = oracle.PoolState.empty(n_gpu, n_host)
    slots = rng.permutation(n_gpu)[:n_occ]
    hosts = rng.permutation(n_host)[:n_occ]
    st.free[slots] = 0
    st.to_host[slots] = hosts
    st.host_to_gpu[hosts] = slots
    levels = prio_levels or max(2, n_occ)
    st.priority[slots] = rng.integers(0, levels, n_occ)
    host_kv = (rng.integers(0, 1 << 16, (n_host, 576), dtype=np.uint16) & np.uint16(0xBFFF))
    st.gpu_kv[slots] = host_kv[hosts]
    total = B_rows * L
    req_to_host = rng.permutation(n_host)[:total].astype(np.int32)
    key_begin = (np.arange(B_rows) * L).astype(np.int64)
    sel = np.full((B_rows, k), -1, np.int32)
    for r in range(B_rows):
        m = int(rng.integers(0, k + 1)) if r % 3 == 2 else k
        m = min(m, L)
        sel[r, :m] = np.sort(rng.permutation(L)[:m])
    return st, host_kv, sel, key_begin, req_to_host


def _run_gpu(st, host_kv, sel, key_begin, req_to_host, step_id, mode=B.RECALL_GATHER):
    dp = DevPool(st.free, st.priority, st.to_host, st.host_to_gpu, st.indices_buf, st.gpu_kv, host_kv)
    n_rows, k = sel.shape
    idx = dev(sel)
    kb = dev(key_begin)
    r2h = dev(req_to_host)
    topk_slot = torch.full((n_rows, k), -9, dtype=torch.int32, device="cuda")
    miss_host = torch.full((n_rows * k,), -9, dtype=torch.int32, device="cuda")
    miss_slot = torch.full((n_rows * k,), -9, dtype=torch.int32, device="cuda")
    n_miss = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.pool_workspace_bytes(n_rows, k, dp.n_gpu), dtype=torch.uint8, device="cuda")
    B.pool_lookup_alloc(dp.pool, idx, kb, r2h, step_id, topk_slot, miss_host, miss_slot, n_miss, ws)
    B.recall(dp.pool, miss_host, miss_slot, n_miss, n_rows * k, mode=mode)
    torch.cuda.synchronize()
    out = dict(state=dp.state(), topk_slot=host(topk_slot), miss_host=host(miss_host),
               miss_slot=host(miss_slot), n_miss=int(host(n_miss)[0]), status=int(host(dp.status)[0]))
    dp.close()
    return out


def _compare(case, step_id=10**6, mode=B.RECALL_GATHER):
    st, host_kv, sel, kb, r2h = case
    want_state, want = oracle.pool_step(st, host_kv, sel, kb, r2h, step_id)
    got = _run_gpu(st, host_kv, sel, kb, r2h, step_id, mode)
    assert got["status"] == want.status
    if want.status:
        assert_pool_equal(got["state"], st, "untouched")
        return got, want
    assert got["n_miss"] == want.n_miss
    assert np.array_equal(got["topk_slot"], want.topk_slot)
    assert np.array_equal(got["miss_host"], want.miss_host)
    assert np.array_equal(got["miss_slot"], want.miss_slot)
    assert_pool_equal(got["state"], want_state)
    return got, want


@pytest.mark.parametrize("seed,n_gpu,n_host,n_occ,rows,k,L,levels", [
    (1, 64, 400, 64, 3, 12, 100, None),       # full pool, evictions
    (2, 64, 400, 30, 3, 12, 100, None),       # enough free slots, no eviction
    (3, 5000, 40000, 5000, 4, 300, 9000, 7),  # many priority ties, several chunks
    (4, 9000, 60000, 8000, 5, 512, 10000, 50),
    (5, 20000, 100000, 19990, 8, 1024, 12000, None),
    (6, 16, 64, 16, 1, 1, 64, 1),             # single selection, all priorities equal
    (11, 65536, 300000, 65536, 8, 2048, 30000, None),   # largest single-workgroup pool
    (12, 65537, 300000, 65537, 4, 2048, 30000, 100),    # smallest multi-kernel pool
    (13, 150000, 600000, 149000, 6, 2048, 50000, 3000), # ties, several slot batches
    (14, 150000, 600000, 150000, 6, 2048, 50000, 3),    # threshold bin overflows the LDS list
    (15, 300000, 1200000, 299000, 4, 2048, 300000, 5000),  # multi-kernel path
])
def test_pool_step_random(seed, n_gpu, n_host, n_occ, rows, k, L, levels):
    announce("pool", seed, n_gpu, n_host, rows, k)
    _compare(_random_case(seed, n_gpu, n_host, n_occ, rows, k, L, levels))


def test_pool_step_memcpy_recall_mode():
    announce("pool memcpy mode")
    _compare(_random_case(7, 3000, 20000, 3000, 4, 256, 4000), mode=B.RECALL_MEMCPY)


def test_pool_exhausted_leaves_pool_untouched():
    announce("pool exhausted")
    rng = np.random.default_rng(8)
    st, host_kv, sel, kb, r2h = _random_case(8, 32, 400, 32, 2, 40, 150)
    got, want = _compare((st, host_kv, sel, kb, r2h))
    assert want.status == oracle.ST_EXHAUSTED


def test_pool_bad_host_index():
    announce("pool bad host")
    st, host_kv, sel, kb, r2h = _random_case(9, 64, 400, 40, 2, 8, 100)
    r2h = r2h.copy()
    r2h[kb[1] + sel[1, 3]] = 400          # outside the host pool
    got, want = _compare((st, host_kv, sel, kb, r2h))
    assert want.status == oracle.ST_BAD_HOST


def test_pool_second_step_all_hits():
    announce("pool repeat step")
    case = _random_case(10, 2000, 9000, 2000, 3, 256, 3000)
    st, host_kv, sel, kb, r2h = case
    s1, _ = oracle.pool_step(st, host_kv, sel, kb, r2h, 10**6)
    got, want = _compare((s1, host_kv, sel, kb, r2h), step_id=10**6 + 1)
    assert want.n_miss == 0


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(hs.data())
def test_pool_step_properties(data):
    # random small pools (every fill level, heavy priority ties, k from 1), against the oracle:
    # bit-exact state or the same status with the pool untouched
    n_gpu = data.draw(hs.integers(1, 96), label="n_gpu")
    n_occ = data.draw(hs.integers(0, n_gpu), label="n_occ")
    rows = data.draw(hs.integers(1, 4), label="rows")
    k = data.draw(hs.integers(1, 40), label="k")
    L = data.draw(hs.integers(1, 60), label="L")
    n_host = max(rows * L, n_occ) + data.draw(hs.integers(0, 50), label="extra_host")
    levels = data.draw(hs.integers(1, 8), label="levels")
    seed = data.draw(hs.integers(0, 2**31 - 1), label="seed")
    announce("pool property", n_gpu, n_occ, rows, k, L, levels)
    _compare(_random_case(seed, n_gpu, n_host, n_occ, rows, k, L, levels))
