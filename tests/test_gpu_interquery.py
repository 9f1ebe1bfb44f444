"""GPU parity of the inter-query prefetch of a chunked prefill (ECHO page §6.2) against the oracle
(oracle/interquery.py): the approximate top-k subsets under a shift (echo_topk_subset), the
segment unions (echo_union_rows) and the k-th score EMA (echo_threshold_ema) bit-exact on the
same float32 inputs; the chunked prefill with its guaranteed residency bit-exact against the
oracle's loop (pool contents after every chunk); with the prefetch on, the same selections and
resident rows."""

import numpy as np
import pytest
import torch

import oracle
from oracle import interquery as iq
from dsa_indexer_top_amd import binding as B, inputs as gen
from dsa_indexer_top_amd.runner import PrefillChunkRunner
from gpu_util import announce, dev, host, assert_pool_equal

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k", [1, 64, 2048])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_subset_exact(k, ties):
    announce("topk subset", k, ties)
    lens = np.array([0, 1, 5, 300, 2047, 2048, 2049, 5000], np.int32)
    ld = 5003
    s = gen.random_scores(70 + k + ties, len(lens), 5000, tie_frac=0.5 if ties else 0.0, ld=ld)
    s = (s * 2.5 + 1.0).astype(np.float32)
    for shift in (float("nan"), 0.0, 1.75, -2.0):
        sh = torch.tensor([shift], dtype=torch.float32, device="cuda")
        sub = torch.empty((len(lens), k), dtype=torch.int32, device="cuda")
        cnt = torch.empty(len(lens), dtype=torch.int32, device="cuda")
        thr = torch.empty(len(lens), dtype=torch.int32, device="cuda")
        B.topk_subset(dev(s), dev(lens), 5000, k, sh, sub, cnt, thr)
        g_sub, g_cnt, g_thr = host(sub), host(cnt), host(thr)
        for r, L in enumerate(lens):
            want, want_thr, S = iq.approx_subset(s[r, :L], k, 0.0 if np.isnan(shift) else shift)
            assert g_cnt[r] == len(want) == S, (shift, r)
            assert np.array_equal(g_sub[r, :S], want), (shift, r)
            assert (g_sub[r, S:] == -1).all()
            assert g_thr[r] == want_thr, (shift, r)


def test_topk_subset_clamps_and_ld():
    # lengths above max_len are clamped; ld wider than the rows; a shift of +inf and -inf
    announce("topk subset clamps")
    s = gen.random_scores(76, 3, 600, ld=640)
    lens = np.array([10000, 600, -5], np.int32)
    for shift in (float("inf"), float("-inf"), 0.5):
        sh = torch.tensor([shift], dtype=torch.float32, device="cuda")
        sub = torch.empty((3, 32), dtype=torch.int32, device="cuda")
        cnt = torch.empty(3, dtype=torch.int32, device="cuda")
        B.topk_subset(dev(s), dev(lens), 600, 32, sh, sub, cnt)
        g_sub, g_cnt = host(sub), host(cnt)
        for r, L in enumerate([600, 600, 0]):
            want, _, S = iq.approx_subset(s[r, :L], 32, shift)
            assert g_cnt[r] == S and np.array_equal(g_sub[r, :S], want), (shift, r)


def test_union_rows_exact():
    announce("union rows")
    rng = np.random.default_rng(72)
    for n_keys, n_rows, k in [(0, 2, 4), (1, 3, 4), (4096, 5, 300), (4097, 7, 700),
                              (20000, 40, 512), (9000, 0, 8)]:
        idx = rng.integers(-3, n_keys + 5, (n_rows, k)).astype(np.int32)
        n_seg = max(1, -(-n_keys // 4096))
        out = torch.empty((n_seg, 4096), dtype=torch.int32, device="cuda")
        cnt = torch.empty(n_seg, dtype=torch.int32, device="cuda")
        ws = torch.empty(max(B.union_workspace_bytes(n_keys), 256), dtype=torch.uint8, device="cuda")
        for rep in range(2):                              # the bitmap is cleared by every call
            B.union_rows(dev(idx), n_keys, out, cnt, ws)
            rows = [r[(r >= 0) & (r < n_keys)] for r in idx]
            want, want_cnt = iq.union_segments(rows, n_keys)
            assert np.array_equal(host(cnt), want_cnt), n_keys
            assert np.array_equal(host(out), want), n_keys


def test_threshold_ema_exact():
    announce("threshold ema")
    s = gen.random_scores(73, 5, 700)
    idx = oracle.topk_rows([r[:L] for r, L in zip(s.astype(np.float64), [700, 3, 0, 64, 65])], 64)
    theta = torch.tensor([np.nan, 1.0, 2.0, -1.0, 0.25], dtype=torch.float32, device="cuda")
    kth = torch.empty(5, dtype=torch.float32, device="cuda")
    B.threshold_ema(dev(s), dev(idx), 0.5, theta, kth)
    want_k = oracle.kth_scores(list(s.astype(np.float64)), idx)
    got_k = host(kth)
    assert np.isnan(got_k[2]) and np.isnan(want_k[2])
    m = ~np.isnan(want_k)
    assert np.array_equal(got_k[m].astype(np.float64), want_k[m])
    want_t = oracle.ema_update(np.array([np.nan, 1.0, 2.0, -1.0, 0.25]), want_k, 0.5)
    assert np.array_equal(host(theta), want_t.astype(np.float32))      # one float32 rounding


@pytest.mark.parametrize("prefetch", [False, True])
def test_prefill_chunk_loop(prefetch):
    announce("prefill chunk loop prefetch=%s" % prefetch)
    n, chunk, k = 800, 300, 32
    q, w, kk = gen.make_prefill_inputs(n, seed=74)
    req_to_host = np.random.default_rng(75).permutation(n).astype(np.int32)
    host_kv = gen.fill_latent_rows(74, np.empty((n, 576), np.uint16))
    st0 = oracle.PoolState.empty(n, n)
    _, recs = iq.prefill_chunk_loop(q, w, kk, req_to_host, st0.copy(), host_kv, chunk, k, step0=20)
    pool = gen.PoolArrays(st0.free, st0.priority, st0.to_host, st0.host_to_gpu, st0.indices_buf,
                          st0.gpu_kv, step_id=20)
    rn = PrefillChunkRunner(q, w, kk, req_to_host, pool, host_kv, chunk, k, prefetch=prefetch)
    moved = 0
    try:
        for c, rec in enumerate(recs):
            rows = rn.run_chunk(c, 20 + c)
            got = rn.results(rows)
            assert got["status"] == 0
            assert np.array_equal(got["idx"], rec["idx"]), "chunk %d selection" % c
            assert np.array_equal(got["uni"], rec["union"]) and np.array_equal(got["uni_cnt"], rec["union_cnt"])
            assert got["kth"] == rec["kth_last"]
            if prefetch:
                for r in range(rows):
                    sub, thr, S = rec["subsets"][r]
                    assert got["subset_cnt"][r] == S and np.array_equal(got["subset"][r, :S], sub)
                assert np.array_equal(got["pre"], rec["prefetch"])
                moved += got["n_prefetched"]
                toks = rec["union"][rec["union"] >= 0]
                oracle.check_pool_invariants(
                    oracle.PoolState(**{nm: got["pool"][nm] for nm in ("free", "priority", "to_host",
                                                                      "host_to_gpu", "indices_buf",
                                                                      "gpu_kv")}),
                    host_kv, req_to_host[toks], got["slot"][rec["union"] >= 0])
            else:
                assert got["n_miss"] == rec["result"].n_miss
                assert np.array_equal(got["slot"], rec["result"].topk_slot)
                assert_pool_equal(oracle.PoolState(**{nm: got["pool"][nm] for nm in (
                    "free", "priority", "to_host", "host_to_gpu", "indices_buf", "gpu_kv")}),
                    rec["state"], "chunk %d" % c)
        if prefetch:
            assert moved > 0
    finally:
        rn.close()
