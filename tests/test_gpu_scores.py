"""GPU parity of echo_index_scores against the oracle (bit-exact on the integer grid,
|gpu - oracle| <= 1e-4 * T on general FP8 with per-token scales)."""

import numpy as np
import pytest
import torch

import oracle
from dsa_indexer_top_amd import binding as B, inputs as gen
from gpu_util import announce, dev, host, decode_inputs_to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _run_scores(inp, ld=None):
    d = decode_inputs_to_dev(inp)
    max_len = int(inp.key_len.max()) if len(inp.key_len) else 0
    ld = max(max_len, 1) if ld is None else ld
    scores = torch.full((len(inp.key_len), ld), float("nan"), dtype=torch.float32, device="cuda")
    B.index_scores(d["q"], d["w"], d["k"], d["k_scale"], d["key_begin"], d["key_len"],
                   max_len, scores, ld=ld)
    return host(scores)


def _check(inp, got, rows=None, exact=True):
    rows = range(len(inp.key_len)) if rows is None else rows
    for r in rows:
        L = int(inp.key_len[r])
        sl = slice(r, r + 1)
        want = oracle.index_scores(inp.q[sl], inp.w[sl], inp.k, inp.k_scale,
                                   inp.key_begin[sl], inp.key_len[sl])[0]
        g = got[r, :L].astype(np.float64)
        if exact:
            bad = np.flatnonzero(g != want)
            assert len(bad) == 0, "row %d: %d mismatches, first at %d: gpu %r oracle %r" % (
                r, len(bad), bad[0], g[bad[0]], want[bad[0]])
        else:
            T = oracle.error_scale(inp.q[sl], inp.w[sl], inp.k, inp.k_scale,
                                   inp.key_begin[sl], inp.key_len[sl])[0]
            err = np.abs(g - want)
            worst = np.argmax(err - TOL * T)
            assert (err <= TOL * T).all(), "row %d tok %d err %g > %g" % (r, worst, err[worst], TOL * T[worst])
        # entries past the row length are not written
        assert np.isnan(got[r, L:]).all()


@pytest.mark.parametrize("lens", [[4096], [1, 63, 64, 65], [127, 128, 129, 0, 3000], [70000]])
def test_scores_integer_grid_exact(lens):
    announce("scores int-grid", lens)
    cfg = gen.DecodeConfig("t", len(lens), 0, 16, "int", False, 0.5, 2, seed=101 + sum(lens) % 97)
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    _check(inp, _run_scores(inp, ld=max(lens) + 5))


@pytest.mark.parametrize("lens", [[5000, 1, 130, 2048], [9000]])
def test_scores_general_fp8_scaled_tolerance(lens):
    announce("scores general fp8", lens)
    cfg = gen.DecodeConfig("g", len(lens), 0, 16, "general", True, 0.5, 2, seed=202 + len(lens))
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    _check(inp, _run_scores(inp), exact=False)


def test_scores_tiny_workload():
    announce("scores tiny workload")
    inp = gen.make_decode_inputs(gen.CONFIGS["tiny"])
    _check(inp, _run_scores(inp))


def test_scores_b8_64k_full_exact():
    announce("scores b8_64k full size")
    inp = gen.make_decode_inputs(gen.CONFIGS["b8_64k"])
    _check(inp, _run_scores(inp))


def test_scores_b32_ragged_full_tolerance():
    announce("scores b32_ragged full size")
    inp = gen.make_decode_inputs(gen.CONFIGS["b32_ragged"])
    got = _run_scores(inp)
    _check(inp, got, exact=False)                      # every one of the 32 requests


def _hist_of(scores_f32):
    """2048-bin histogram of the top 11 bits of the descending-order key (bin 0 = highest)."""
    key = ~oracle.topk.f32_order_key(np.asarray(scores_f32, np.float32))
    return np.bincount((key >> 21).astype(np.int64), minlength=2048)


@pytest.mark.parametrize("grid,lens", [("int", [4096, 1, 0, 130, 70000]),
                                       ("general", [5000, 129, 9000])])
def test_scores_with_topk_histogram(grid, lens):
    # echo_index_scores_hist (the decode step's scoring launch): the same scores, and per request
    # the histogram of the top 11 bits of the descending-order key of exactly those scores,
    # added to what the histogram held (accumulated twice here)
    announce("scores + histogram", grid, lens)
    cfg = gen.DecodeConfig("h", len(lens), 0, 16, grid, grid == "general", 0.5, 2, seed=211)
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    d = decode_inputs_to_dev(inp)
    max_len = max(lens)
    sc = torch.full((len(lens), max_len), float("nan"), dtype=torch.float32, device="cuda")
    hist = torch.zeros((len(lens), 2048), dtype=torch.int32, device="cuda")
    for _ in range(2):
        B.index_scores_hist(d["q"], d["w"], d["k"], d["k_scale"], d["key_begin"], d["key_len"],
                            max_len, sc, hist)
    got, gh = host(sc), host(hist)
    _check(inp, got, exact=grid == "int")
    for r, L in enumerate(lens):
        assert np.array_equal(gh[r], 2 * _hist_of(got[r, :L])), "histogram of request %d" % r


@pytest.mark.parametrize("grid,lens,page", [("int", [4096, 1, 0, 130, 70000, 3000], 64),
                                            ("int", [5000, 129, 257], 16),
                                            ("general", [9000, 1, 300], 256),
                                            ("general", [3000, 4096, 4097], 4096)])
def test_scores_paged_key_cache(grid, lens, page):
    # a paged indexer-K cache (pages of `page` tokens in a random order): the same scores as the
    # contiguous layout, bit for bit (same kernel arithmetic), and the oracle's (bit-exact on the
    # integer grid, within 1e-4 T otherwise)
    announce("scores paged", grid, lens, page)
    cfg = gen.DecodeConfig("p", len(lens), 0, 16, grid, grid == "general", 0.5, 2, seed=221 + page)
    inp = gen.make_decode_inputs(cfg, lengths=lens)
    pk = gen.page_key_cache(inp.k, inp.k_scale, inp.key_begin, inp.key_len, page, seed=7)
    d = decode_inputs_to_dev(inp)
    max_len = max(lens)
    sc = torch.full((len(lens), max_len), float("nan"), dtype=torch.float32, device="cuda")
    B.index_scores_paged(d["q"], d["w"], dev(pk.k_pages),
                         None if pk.k_scale_pages is None else dev(pk.k_scale_pages),
                         dev(pk.page_table), page, d["key_len"], max_len, sc)
    got = host(sc)
    contiguous = _run_scores(inp, ld=max_len)
    for r, L in enumerate(lens):
        assert np.array_equal(got[r, :L], contiguous[r, :L]), "request %d" % r
    _check(inp, got, exact=grid == "int")
