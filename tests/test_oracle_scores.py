"""Pins of the oracle's indexer scores: closed forms, homogeneity, invariances, exactness."""

import numpy as np
import pytest

from oracle import index_scores, error_scale, prefill_scores_rows, E4M3FN_TABLE

H, D = 64, 128
ONE, TWO, MINUS_ONE = 0x38, 0x40, 0xB8      # E4M3FN codes of 1, 2, -1


def _codes_of(values):
    """E4M3FN codes of exactly representable values, looked up in the table."""
    lut = {float(v): c for c, v in enumerate(E4M3FN_TABLE) if not np.isnan(v)}
    lut[0.0] = 0
    return np.vectorize(lambda v: lut[float(v)])(np.asarray(values, np.float64)).astype(np.uint8)


def _rand_int_case(rng, n_q, lens):
    q = _codes_of(rng.integers(-8, 9, (n_q, H, D)))
    k = _codes_of(rng.integers(-8, 9, (sum(lens), D)))
    w = (rng.integers(-4, 5, (n_q, H)) / 64).astype(np.float32)
    begin = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return q, w, k, begin, np.array(lens, np.int32)


def test_one_hot_weight_is_single_head_relu():
    # w = e_h: the score is ReLU of head h's dot product alone
    q = np.zeros((1, H, D), np.uint8)
    q[0, 5, :] = ONE                        # head 5: all ones
    q[0, 6, :] = MINUS_ONE                  # head 6: all minus ones
    k = np.full((3, D), TWO, np.uint8)      # every key all twos -> dot(head5) = 256
    k[1, :64] = MINUS_ONE                   # token 1: 64 * -1 + 64 * 2 = 64
    w = np.zeros((1, H), np.float32)
    w[0, 5] = 1.0
    s = index_scores(q, w, k, None, np.array([0]), np.array([3]))[0]
    assert s.tolist() == [256.0, 64.0, 256.0]
    w[0, 5], w[0, 6] = 0.0, 1.0             # head 6: dot is negative -> ReLU -> 0
    s = index_scores(q, w, k, None, np.array([0]), np.array([3]))[0]
    assert s.tolist() == [0.0, 0.0, 0.0]


def test_q_equal_minus_k_scores_zero():
    rng = np.random.default_rng(0)
    kv = rng.integers(-8, 9, D)
    k = _codes_of(kv)[None, :]
    q = np.broadcast_to(_codes_of(-kv), (1, H, D)).copy()
    w = rng.standard_normal((1, H)).astype(np.float32)
    assert index_scores(q, w, k, None, np.array([0]), np.array([1]))[0][0] == 0.0


def test_q_equal_k_scores_norm():
    rng = np.random.default_rng(1)
    kv = rng.integers(-8, 9, D)
    k = _codes_of(kv)[None, :]
    q = np.broadcast_to(_codes_of(kv), (1, H, D)).copy()
    w = np.full((1, H), 1 / 64, np.float32)
    # every head sees |k|^2 >= 0; 64 heads of weight 1/64 sum to |k|^2
    assert index_scores(q, w, k, None, np.array([0]), np.array([1]))[0][0] == float((kv * kv).sum())


def test_all_positive_reduces_to_matvec():
    # ReLU is the identity when every product is >= 0: score[s] = k[s] . (Q^T w)
    rng = np.random.default_rng(2)
    qv = rng.integers(0, 9, (1, H, D))
    kv = rng.integers(0, 9, (50, D))
    w = (rng.integers(-4, 5, (1, H)) / 64).astype(np.float32)
    s = index_scores(_codes_of(qv), w, _codes_of(kv), None, np.array([0]), np.array([50]))[0]
    v = qv[0].astype(np.float64).T @ w[0].astype(np.float64)     # [D]
    assert np.array_equal(s, kv.astype(np.float64) @ v)


def test_homogeneity_in_w_and_scale():
    rng = np.random.default_rng(3)
    q, w, k, b, L = _rand_int_case(rng, 2, [40, 33])
    s1 = index_scores(q, w, k, None, b, L)
    s2 = index_scores(q, 2 * w, k, None, b, L)
    for a, c in zip(s1, s2):
        assert np.array_equal(2 * a, c)
    scale = np.full(k.shape[0], 2.0, np.float32)
    s3 = index_scores(q, w, k, scale, b, L)
    for a, c in zip(s1, s3):
        assert np.array_equal(2 * a, c)
    # a per-token scale acts per token
    scale = rng.uniform(0.5, 2, k.shape[0]).astype(np.float32)
    s4 = index_scores(q, w, k, scale, b, L)
    for r, (a, c) in enumerate(zip(s1, s4)):
        sc = scale[b[r]:b[r] + L[r]].astype(np.float64)
        np.testing.assert_allclose(c, a * sc, rtol=1e-14, atol=0)


def test_additive_in_w():
    rng = np.random.default_rng(4)
    q, w, k, b, L = _rand_int_case(rng, 1, [64])
    w2 = (rng.integers(-4, 5, (1, H)) / 64).astype(np.float32)
    a = index_scores(q, w, k, None, b, L)[0]
    c = index_scores(q, w2, k, None, b, L)[0]
    ac = index_scores(q, (w + w2).astype(np.float32), k, None, b, L)[0]
    assert np.array_equal(a + c, ac)


def test_head_permutation_invariance():
    rng = np.random.default_rng(5)
    q, w, k, b, L = _rand_int_case(rng, 1, [70])
    perm = rng.permutation(H)
    a = index_scores(q, w, k, None, b, L)[0]
    c = index_scores(q[:, perm], w[:, perm], k, None, b, L)[0]
    assert np.array_equal(a, c)


def test_requests_see_only_their_keys():
    rng = np.random.default_rng(6)
    q, w, k, b, L = _rand_int_case(rng, 3, [5, 0, 9])
    s = index_scores(q, w, k, None, b, L)
    assert [len(x) for x in s] == [5, 0, 9]
    solo = index_scores(q[2:3], w[2:3], k[5:], None, np.array([0]), np.array([9]))[0]
    assert np.array_equal(s[2], solo)


def test_integer_grid_scores_on_1_64_grid():
    rng = np.random.default_rng(7)
    q, w, k, b, L = _rand_int_case(rng, 2, [300, 200])
    for s in index_scores(q, w, k, None, b, L):
        assert np.array_equal(s * 64, np.round(s * 64))
        assert np.abs(s).max() <= 32768
        # exact in float32, the basis for bit-exact GPU parity on this grid
        assert np.array_equal(s.astype(np.float32).astype(np.float64), s)


def test_error_scale_bounds_score():
    rng = np.random.default_rng(8)
    q, w, k, b, L = _rand_int_case(rng, 2, [50, 60])
    sc = rng.uniform(0.5, 2, k.shape[0]).astype(np.float32)
    for s, t in zip(index_scores(q, w, k, sc, b, L), error_scale(q, w, k, sc, b, L)):
        assert (np.abs(s) <= t + 1e-9).all()
        assert (t >= 0).all()


def test_prefill_rows_are_causal_prefixes():
    rng = np.random.default_rng(9)
    n = 40
    q = _codes_of(rng.integers(-8, 9, (n, H, D)))
    k = _codes_of(rng.integers(-8, 9, (n, D)))
    w = (rng.integers(-4, 5, (n, H)) / 64).astype(np.float32)
    rows = [0, 7, 39]
    got = prefill_scores_rows(q, w, k, rows)
    assert [len(g) for g in got] == [1, 8, 40]
    full = index_scores(q[39:40], w[39:40], k, None, np.array([0]), np.array([n]))[0]
    assert np.array_equal(got[2], full)
    # the causal row is the prefix of the same query scored against every key
    row7_all = index_scores(q[7:8], w[7:8], k, None, np.array([0]), np.array([n]))[0]
    assert np.array_equal(got[1], row7_all[:8])
