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


# ---------------------------------------------------------------- the error scale T, by value
# T[r,s] = scale_s * sum_h |w[r,h]| * sum_d |q[r,h,d] * k[s,d]| bounds the terms of score[r,s];
# every general-FP8 tolerance is 1e-4 * T, so T is pinned by values worked out by hand and by
# the case where it must equal the score, so that an inflated T fails.
HALF, QUARTER, MINUS_TWO = 0x30, 0x28, 0xC0     # E4M3FN codes of 0.5, 0.25, -2


def _t_hand_cases():
    """(q, w, k, scale, expected score, expected T), each worked out by hand."""
    cases = []
    # q = +1 everywhere, k alternating +1 / -1, w = (2, 0, ..., 0), scale 1.5: every head's dot
    # product is 0, so the score is 0; T = 1.5 * 2 * 128 * |1 * 1| = 384
    q = np.full((1, H, D), ONE, np.uint8)
    k = np.where(np.arange(D) % 2 == 0, ONE, MINUS_ONE).astype(np.uint8)[None, :]
    w = np.zeros((1, H), np.float32)
    w[0, 0] = 2.0
    cases.append((q, w, k, np.array([1.5], np.float32), 0.0, 384.0))
    # head 0: q = 2, head 1: q = -1, other heads 0; w = (0.5, -0.25, 0, ...); k = 1 on the
    # first 64 dims, -2 on the rest; scale 2.
    #   head 0: dot = 64*2 - 64*4 = -128 -> ReLU 0;   sum |q k| = 64*2 + 64*4 = 384
    #   head 1: dot = -64 + 128 = 64 -> 2*64 = 128 -> times -0.25 = -32;  sum |q k| = 64 + 128 = 192
    #   score = -32;  T = 2 * (0.5 * 384 + 0.25 * 192) = 2 * 240 = 480
    q = np.zeros((1, H, D), np.uint8)
    q[0, 0, :] = TWO
    q[0, 1, :] = MINUS_ONE
    w = np.zeros((1, H), np.float32)
    w[0, 0], w[0, 1] = 0.5, -0.25
    k = np.concatenate([np.full(64, ONE), np.full(64, MINUS_TWO)]).astype(np.uint8)[None, :]
    cases.append((q, w, k, np.array([2.0], np.float32), -32.0, 480.0))
    # every head q = 0.5 on dims 0..3 only, k = 0.25 on dims 2..5, w = 1/64 each, no scale:
    # overlap on dims 2, 3 -> dot = 2 * 0.125 = 0.25 per head; score = 64 * 0.25 / 64 = 0.25;
    # all terms are positive, so T = score = 0.25
    q = np.zeros((1, H, D), np.uint8)
    q[0, :, 0:4] = HALF
    k = np.zeros((1, D), np.uint8)
    k[0, 2:6] = QUARTER
    w = np.full((1, H), 1 / 64, np.float32)
    cases.append((q, w, k, None, 0.25, 0.25))
    return cases


def _check_error_scale(fn):
    for q, w, k, scale, want_s, want_t in _t_hand_cases():
        s = index_scores(q, w, k, scale, np.array([0]), np.array([1]))[0][0]
        assert s == want_s, (s, want_s)
        t = fn(q, w, k, scale, np.array([0]), np.array([1]))[0][0]
        assert t == want_t, (t, want_t)
    # q, k and w all >= 0: ReLU is the identity and every term is positive, so T is the score
    rng = np.random.default_rng(10)
    q = _codes_of(rng.integers(0, 9, (2, H, D)))
    k = _codes_of(rng.integers(0, 9, (90, D)))
    w = (rng.integers(0, 5, (2, H)) / 64).astype(np.float32)
    sc = rng.uniform(0.5, 2, 90).astype(np.float32)
    b, L = np.array([0, 40]), np.array([40, 50])
    for s, t in zip(index_scores(q, w, k, sc, b, L), fn(q, w, k, sc, b, L)):
        np.testing.assert_allclose(t, s, rtol=1e-15, atol=0)


def test_error_scale_values_by_hand():
    _check_error_scale(error_scale)


def test_error_scale_pins_catch_planted_mistakes():
    # an inflated or deflated T must fail the pins above
    from oracle.fp8 import decode_e4m3fn

    def product_of_sums(q, w, k, k_scale, key_begin, key_len):     # sum|q| * sum|k| per head
        qa, out = np.abs(decode_e4m3fn(q)), []
        for r in range(q.shape[0]):
            kr = np.abs(decode_e4m3fn(k[key_begin[r]:key_begin[r] + key_len[r]]))
            t = np.abs(w[r]).astype(np.float64) @ qa[r].sum(axis=1) * kr.sum(axis=1)
            if k_scale is not None:
                t = t * k_scale[key_begin[r]:key_begin[r] + key_len[r]]
            out.append(t)
        return out

    def scale_squared(*a):
        t = error_scale(*a)
        sc = a[3]
        if sc is None:
            return t
        return [ti * np.asarray(sc[a[4][r]:a[4][r] + a[5][r]], np.float64) for r, ti in enumerate(t)]

    def no_scale(q, w, k, k_scale, key_begin, key_len):
        return error_scale(q, w, k, None, key_begin, key_len)

    def signed_w(q, w, k, k_scale, key_begin, key_len):            # |w| dropped
        qa, out = np.abs(decode_e4m3fn(q)), []
        for r in range(q.shape[0]):
            kr = np.abs(decode_e4m3fn(k[key_begin[r]:key_begin[r] + key_len[r]]))
            t = (kr @ qa[r].T) @ w[r].astype(np.float64)
            if k_scale is not None:
                t = t * k_scale[key_begin[r]:key_begin[r] + key_len[r]]
            out.append(t)
        return out

    for bad in (product_of_sums, scale_squared, no_scale, signed_w):
        with pytest.raises(AssertionError):
            _check_error_scale(bad)
            raise RuntimeError("not caught: " + bad.__name__)


def test_scores_against_per_head_loops():
    # brute force: plain Python loops over heads and dimensions on the values of the E4M3FN
    # table, float64 throughout, against the oracle's matrix formulation
    rng = np.random.default_rng(11)
    q = rng.integers(0, 256, (2, H, D)).astype(np.uint8)
    k = rng.integers(0, 256, (7, D)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0                       # no NaN codes
    k[(k & 0x7F) == 0x7F] = 0
    w = rng.standard_normal((2, H)).astype(np.float32)
    sc = rng.uniform(0.5, 2, 7).astype(np.float32)
    b, L = np.array([0, 3]), np.array([3, 4])
    got = index_scores(q, w, k, sc, b, L)
    tab = [float(v) for v in E4M3FN_TABLE]
    for r in range(2):
        for s in range(int(L[r])):
            tok = int(b[r]) + s
            total = 0.0
            for h in range(H):
                dot = 0.0
                for d in range(D):
                    dot += tab[q[r, h, d]] * tab[k[tok, d]]
                total += float(w[r, h]) * max(float(sc[tok]) * dot, 0.0)
            assert abs(got[r][s] - total) <= 1e-12 * max(1.0, abs(total)), (r, s)
