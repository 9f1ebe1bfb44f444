"""Pins of the oracle's inter-query prefetch (oracle/interquery.py) against what the ECHO page
(§6.2) and the mathematics fix: the page's inequality for the threshold bin, the subset's
inclusion in the exact top-k (brute force), special cases, the threshold bin shrinking under
the shift, the segment unions, and the chunk loop's invariants and losslessness."""

import numpy as np
import pytest

import oracle
from oracle import interquery as iq
from dsa_indexer_top_amd import inputs as gen


def _rows(rng, n_rows, L, ties):
    s = rng.standard_normal((n_rows, L)).astype(np.float32) * 3
    if ties:
        s = np.round(s * 2) / 2                      # many equal scores
    return s


@pytest.mark.parametrize("ties", [False, True])
def test_subset_inside_exact_topk_and_page_inequality(ties):
    rng = np.random.default_rng(61 + ties)
    for trial in range(120):
        L = int(rng.integers(1, 400))
        k = int(rng.integers(1, 120))
        row = _rows(rng, 1, L, ties)[0]
        shift = float(rng.choice([0.0, rng.standard_normal() * 3, np.sort(row)[::-1][min(k, L) - 1]]))
        sub, thr_cnt, S = iq.approx_subset(row, k, shift)
        exact = oracle.topk_row(row.astype(np.float64), k)
        exact = set(exact[exact >= 0].tolist())
        assert set(sub.tolist()) <= exact
        assert len(sub) == S <= k
        if k >= L:
            assert len(sub) == L and thr_cnt == 0
        elif thr_cnt:
            assert S > k - thr_cnt                   # the page's inequality
        # every subset token scores above every token outside it
        rest = np.setdiff1d(np.arange(L), sub)
        if len(sub) and len(rest):
            assert row[sub].min() > row[rest].max()


def test_subset_special_cases():
    row = np.full(50, 1.25, np.float32)
    sub, thr, S = iq.approx_subset(row, 10, 0.0)
    assert len(sub) == 0 and thr == 50 and S == 0     # one bin holds everything
    sub, thr, S = iq.approx_subset(row, 50, 0.0)
    assert len(sub) == 50 and thr == 0
    row = np.array([-0.0, 0.0, 5.0, -3.0], np.float32)
    sub, thr, S = iq.approx_subset(row, 1, 0.0)
    assert sub.tolist() == [2]


def test_shift_shrinks_the_threshold_bin():
    # scores concentrated away from zero (the page's layers have k-th scores near 2.0 or -3.5):
    # unshifted, the k-th score falls in a wide bin; shifted by its prediction, in a narrow one
    rng = np.random.default_rng(63)
    plain, shifted = [], []
    for off in (2.0, -3.5):
        rows = (rng.standard_normal((40, 8192)) * 0.5 + off).astype(np.float32)
        for row in rows:
            kth = np.sort(row)[::-1][255]
            plain.append(iq.approx_subset(row, 256, 0.0)[1])
            shifted.append(iq.approx_subset(row, 256, kth + 0.01)[1])
    assert np.median(shifted) * 4 < np.median(plain)


def test_union_segments():
    rng = np.random.default_rng(64)
    n_keys = 9000
    rows = [rng.integers(-1, n_keys, 300) for _ in range(7)]
    out, cnt = iq.union_segments(rows, n_keys)
    want = np.unique(np.concatenate([r[r >= 0] for r in rows]))
    got = np.concatenate([out[g, :cnt[g]] for g in range(len(cnt))])
    assert np.array_equal(got, want)
    assert out.shape == (3, 4096)
    for g in range(3):
        assert (out[g, :cnt[g]] // 4096 == g).all() and (out[g, cnt[g]:] == -1).all()


def test_chunk_loop_invariants_and_shift():
    n, chunk, k = 900, 300, 32
    q, w, kk = gen.make_prefill_inputs(n, seed=65)
    req_to_host = np.random.default_rng(66).permutation(n).astype(np.int32)
    host_kv = gen.fill_latent_rows(65, np.empty((n, 576), np.uint16))
    st = oracle.PoolState.empty(n, n)
    st_T, recs = iq.prefill_chunk_loop(q, w, kk, req_to_host, st, host_kv, chunk, k, step0=10)
    assert recs[0]["shift"] == 0.0
    for c, rec in enumerate(recs):
        assert rec["result"].status == 0
        toks = rec["union"][rec["union"] >= 0]
        oracle.check_pool_invariants(rec["state"], host_kv, req_to_host[toks],
                                     rec["result"].topk_slot[rec["union"] >= 0])
        # the prefetch set is inside the exact union
        pre = rec["prefetch"][rec["prefetch"] >= 0]
        assert set(pre.tolist()) <= set(toks.tolist())
        # the shift of the next chunk is the EMA of the last rows' k-th scores
        if c + 1 < len(recs):
            ks = [r["kth_last"] for r in recs[:c + 1]]
            th = oracle.ema_update(np.array([np.nan]), np.array([ks[0]]), 0.5)
            for v in ks[1:]:
                th = oracle.ema_update(th, np.array([v]), 0.5)
            assert recs[c + 1]["shift"] == float(np.float32(th[0]))
