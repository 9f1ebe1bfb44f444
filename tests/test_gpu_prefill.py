"""GPU parity of the causal prefill indexer (echo_index_scores_prefill) and its per-row top-k
against the oracle: bit-exact on integer-grid inputs, within 1e-4 * T (T = the magnitude of all
terms of a score) on general FP8 inputs and on head weights spread over a wide dynamic range;
sampled rows at the full 32768^2 size."""

import numpy as np
import pytest
import torch

import oracle
from dsa_indexer_top_amd import binding as B, inputs as gen
from gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _run(q, w, k, q_pos0=0, ld=None):
    n_q, n_k = q.shape[0], k.shape[0]
    ld = n_k + 3 if ld is None else ld
    sc = torch.full((n_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    B.index_scores_prefill(dev(q), dev(w), dev(k), sc, q_pos0=q_pos0, ld=ld)
    return sc


def _check_rows(q, w, k, got, rows, q_pos0=0):
    """got: [n_q, ld] array, or a dict row -> row array."""
    n_k = k.shape[0]
    for t in rows:
        lim = min(n_k, q_pos0 + t + 1)
        want = oracle.index_scores(q[t:t + 1], w[t:t + 1], k, None, np.array([0]), np.array([lim]))[0]
        row = got[t]
        g = row[:lim].astype(np.float64)
        bad = np.flatnonzero(g != want)
        assert len(bad) == 0, "row %d: %d mismatches (first s=%d gpu %r oracle %r)" % (
            t, len(bad), bad[0], g[bad[0]], want[bad[0]])
        assert np.isnan(row[lim:]).all(), "row %d wrote past its causal limit" % t


def _check_rows_tol(q, w, k, got, rows):
    n_k = k.shape[0]
    for t in rows:
        lim = min(n_k, t + 1)
        args = (q[t:t + 1], w[t:t + 1], k, None, np.array([0]), np.array([lim]))
        want, T = oracle.index_scores(*args)[0], oracle.error_scale(*args)[0]
        err = np.abs(got[t][:lim].astype(np.float64) - want)
        worst = int(np.argmax(err - TOL * T))
        assert (err <= TOL * T).all(), "row %d key %d: err %g > %g" % (t, worst, err[worst], TOL * T[worst])
        assert np.isnan(got[t][lim:]).all(), "row %d wrote past its causal limit" % t


# 12 queries per workgroup and 192-key stages of 64-key groups: sizes on both sides of each
@pytest.mark.parametrize("n", [1, 13, 17, 63, 64, 65, 191, 192, 193, 300, 385, 1000])
def test_prefill_small_exact(n):
    announce("prefill", n)
    q, w, k = gen.make_prefill_inputs(n, seed=60 + n)
    got = host(_run(q, w, k))
    _check_rows(q, w, k, got, range(n))


def test_prefill_chunk_offset_exact():
    announce("prefill chunk offset")
    q_all, w_all, k = gen.make_prefill_inputs(1500, seed=71)
    q, w = q_all[1000:1300], w_all[1000:1300]           # a chunk of 300 queries at 1000..1299
    got = host(_run(q, w, k, q_pos0=1000))
    _check_rows(q, w, k, got, range(300), q_pos0=1000)


def test_prefill_keys_shorter_than_positions_exact():
    # queries at positions 500..899 over only 700 keys: rows from position 699 on see all keys
    announce("prefill keys shorter than positions")
    q_all, w_all, k_all = gen.make_prefill_inputs(900, seed=74)
    q, w, k = q_all[500:900], w_all[500:900], k_all[:700]
    got = host(_run(q, w, k, q_pos0=500))
    _check_rows(q, w, k, got, range(400), q_pos0=500)


def test_prefill_general_fp8_tolerance():
    announce("prefill general fp8")
    q, w, k = gen.make_prefill_inputs(600, grid="normal", seed=81)
    _check_rows_tol(q, w, k, host(_run(q, w, k)), range(600))


def test_prefill_wide_weight_range_tolerance():
    # Head weights from 2^-40 to 2^40 in magnitude, some queries with zero heads, and in every
    # other query one key dimension fed only by a head of weight 2^-30, so that the
    # head-weighted sum of q has one element about 2^-30 times the others.
    announce("prefill wide weight range")
    q, w, k = gen.make_prefill_inputs(300, grid="normal", seed=82)
    rng = np.random.default_rng(83)
    w = (w * np.exp2(rng.integers(-40, 41, w.shape))).astype(np.float32)
    w[::3, :32] = 0.0
    q = q.copy()
    q[::2, :, 5] = 0
    q[::2, 0, 5] = 0x38                                   # 1.0
    w[::2, 0] = np.float32(2.0 ** -30)
    _check_rows_tol(q, w, k, host(_run(q, w, k)), range(300))


def test_prefill_topk_rows_exact():
    announce("prefill + top-k 3000 rows")
    n, kk = 3000, 256
    q, w, k = gen.make_prefill_inputs(n, seed=73)
    sc = _run(q, w, k, ld=n)
    lens = torch.arange(1, n + 1, dtype=torch.int32, device="cuda")
    idx = torch.empty((n, kk), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(B.topk_workspace_bytes(n, n), 256), dtype=torch.uint8, device="cuda")
    B.topk(sc, lens, n, kk, idx, ws, ld=n)
    got = host(idx)
    for t in [0, 1, 254, 255, 256, 257, 1000, 2999]:
        want_s = oracle.index_scores(q[t:t + 1], w[t:t + 1], k, None, np.array([0]), np.array([t + 1]))[0]
        assert np.array_equal(got[t], oracle.topk_row(want_s, kk)), t


def _full_size_rows(n):
    """Rows 0..2047 (the rows shorter than k), every 16th row, and the last 64 rows."""
    return np.unique(np.concatenate([np.arange(min(2048, n)), np.arange(0, n, 16),
                                     np.arange(max(0, n - 64), n)]))


def test_prefill_32k_full_sampled():
    # the full 32768^2 causal prefill in the launch configuration the benchmark times; scores and
    # top-2048 index sets of rows 0..2047, every 16th row and the last 64 rows (4160 rows) against
    # the oracle, bit-exact
    cfg = gen.PREFILL["prefill_32k"]
    n = cfg["n"]
    rows = _full_size_rows(n)
    announce("prefill 32768^2 full size, %d rows against the oracle" % len(rows))
    q, w, k = gen.make_prefill_inputs(n, seed=cfg["seed"])
    sc = _run(q, w, k, ld=n)
    lens = torch.arange(1, n + 1, dtype=torch.int32, device="cuda")
    idx = torch.empty((n, cfg["topk"]), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(B.topk_workspace_bytes(n, n), 256), dtype=torch.uint8, device="cuda")
    B.topk(sc, lens, n, cfg["topk"], idx, ws, ld=n)
    sel = torch.from_numpy(rows).cuda()
    got_rows = sc.index_select(0, sel).cpu().numpy()
    got_idx = idx.index_select(0, sel).cpu().numpy()
    del sc
    for i0 in range(0, len(rows), 256):
        part = rows[i0:i0 + 256]
        want = oracle.prefill_scores_rows(q, w, k, part)
        for j, t in enumerate(part):
            g = got_rows[i0 + j, :t + 1].astype(np.float64)
            bad = np.flatnonzero(g != want[j])
            assert len(bad) == 0, "row %d: %d score mismatches, first s=%d" % (t, len(bad), bad[0])
            assert np.array_equal(got_idx[i0 + j], oracle.topk_row(want[j], cfg["topk"])), \
                "row %d index set" % t
        announce("  rows up to %d checked" % part[-1])
