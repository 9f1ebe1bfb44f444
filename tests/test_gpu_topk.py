"""GPU parity of echo_topk against the oracle on the same float32 scores (exact index sets,
ascending order, -1 padding), including ties, signed zeros, short and empty rows."""

import numpy as np
import pytest
import torch

import oracle
from dsa_indexer_top_amd import binding as B, inputs as gen
from gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu


def _run(scores, lens, k):
    n_rows, ld = scores.shape
    max_len = int(max(lens)) if len(lens) else 0
    s = dev(scores)
    ln = dev(np.asarray(lens, np.int32))
    idx = torch.full((n_rows, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.topk_workspace_bytes(n_rows, max_len), dtype=torch.uint8, device="cuda")
    B.topk(s, ln, max_len, k, idx, ws, ld=ld)
    return host(idx)


def _check(scores, lens, k):
    got = _run(scores, lens, k)
    for r, L in enumerate(lens):
        want = oracle.topk_row(scores[r, :L], k)
        if not np.array_equal(got[r], want):
            d = np.flatnonzero(got[r] != want)
            raise AssertionError("row %d (L=%d k=%d): %d diffs, first at %d gpu %d oracle %d" % (
                r, L, k, len(d), d[0], got[r, d[0]], want[d[0]]))


@pytest.mark.parametrize("lens,k,ties", [
    ([1], 1, 0.0), ([0, 5, 4096], 256, 0.0), ([4095, 4096, 4097, 10000], 2048, 0.5),
    ([3000, 2048, 2047, 1], 2048, 0.9), ([65536] * 2, 2048, 0.3), ([8193, 12000], 7, 1.0),
    ([16384, 16385, 32768, 9000, 1, 20000], 2048, 0.3),
    ([2047, 2048, 2049, 8191, 8192, 8193, 16383], 700, 0.2),
    ([100000], 4096, 0.2)])
def test_topk_random_with_ties(lens, k, ties):
    announce("topk", lens, k, ties)
    sc = gen.random_scores(len(lens) * 7 + k, len(lens), max(max(lens), 1) + 3, tie_frac=ties)
    _check(sc, lens, k)


def test_topk_all_equal_and_signed_zero():
    announce("topk all-equal / signed zero")
    n = 9000
    sc = np.zeros((3, n), np.float32)
    sc[1, ::2] = -0.0
    sc[2] = 1.5
    sc[2, 5000:5003] = 2.0
    _check(sc, [n, n, n], 2048)


def test_topk_extreme_values():
    announce("topk extremes")
    sc = gen.random_scores(5, 2, 6000)
    sc[0, :100] = np.finfo(np.float32).max
    sc[0, 100:200] = -np.finfo(np.float32).max
    sc[1, ::3] = np.float32(1e-40)      # subnormals
    sc[1, 1::3] = -np.float32(1e-40)
    _check(sc, [6000, 6000], 150)
    # infinities, and a row whose span overflows to infinity
    sc = gen.random_scores(6, 3, 7000)
    sc[0, 10:40] = np.inf
    sc[0, 50:5000:7] = -np.inf
    sc[1, :3000:2] = -np.inf
    sc[2, 0] = np.float32(3e38)
    sc[2, 1] = np.float32(-3e38)
    _check(sc, [7000, 7000, 7000], 200)
    _check(sc, [7000, 7000, 7000], 4000)


def test_topk_decode_shapes_full():
    announce("topk 64 x 131072 k=2048")
    sc = gen.random_scores(11, 64, 131072, tie_frac=0.05)
    got = _run(sc, [131072] * 64, 2048)
    for r in range(64):                                  # every row against the oracle
        assert np.array_equal(got[r], oracle.topk_row(sc[r], 2048)), r
    assert (np.diff(got, axis=1) > 0).all()


def test_topk_threshold_bin_paths():
    # rows whose threshold bin (a linear bin of the value between the row's extremes) holds at
    # most 64 elements, up to 4096 (resolved in LDS) and more (resolved from the row again), in
    # both classes of rows (20000 scores and 16000 scores)
    announce("topk threshold-bin paths")
    rng = np.random.default_rng(77)
    n, k = 20000, 2048
    rows = []
    r0 = rng.standard_normal(n).astype(np.float32)                 # a few elements per bin
    rows.append(r0)
    # 600 distinct values in one bin, at the threshold: about 1700 scores lie above them
    r1 = rng.standard_normal(n).astype(np.float32)
    r1[rng.permutation(n)[:600]] = np.float32(1.35) + rng.random(600).astype(np.float32) * np.float32(1e-4)
    rows.append(r1)
    # 6000 distinct values in one bin, at the threshold: about 900 scores lie above them
    r2 = rng.standard_normal(n).astype(np.float32) * np.float32(50)
    r2[rng.permutation(n)[:6000]] = np.float32(75.0) + rng.random(6000).astype(np.float32) * np.float32(1e-3)
    rows.append(r2)
    r3 = np.full(n, 3.0, np.float32)                                 # 3000 ties straddling k
    r3[:n - 3000] = rng.standard_normal(n - 3000).astype(np.float32)
    r3[rng.permutation(n)[:500]] = np.float32(9.0)
    rows.append(r3)
    # 2000 distinct values in one bin, at the threshold: about 460 scores lie above them
    r4 = rng.standard_normal(n).astype(np.float32)
    r4[rng.permutation(n)[:2000]] = np.float32(2.0) + rng.random(2000).astype(np.float32) * np.float32(1e-4)
    rows.append(r4)
    sc = np.stack(rows)
    _check(sc, [n] * len(rows), k)
    # such a bin in a row of 16000 scores: 2000 distinct values at the threshold, about 150
    # scores above them
    m = 16000
    r5 = rng.standard_normal(m).astype(np.float32)
    r5[rng.permutation(m)[:2000]] = np.float32(2.3) + rng.random(2000).astype(np.float32) * np.float32(1e-4)
    _check(r5[None, :], [m], k)
