"""The seeded generator's documented recipe, and the oracle's whole decode step on the
tiny workload checked against the step's invariants (count, order, residency, bitwise rows)."""

import numpy as np

import oracle
from dsa_indexer_top_amd import inputs as gen


def test_generator_recipe_and_determinism():
    cfg = gen.CONFIGS["tiny"]
    a = gen.make_decode_inputs(cfg)
    b = gen.make_decode_inputs(cfg)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.q, b.q) and np.array_equal(a.w, b.w)
    assert a.q.shape == (1, 64, 128) and a.q.dtype == np.uint8
    assert a.k.shape == (4096, 128) and a.w.dtype == np.float32
    qv = oracle.decode_e4m3fn(a.q)
    assert set(np.unique(qv).tolist()) <= set(range(-8, 9))
    assert set(np.unique(a.w * 64).tolist()) <= set(range(-4, 5))
    assert sorted(a.req_to_host.tolist()) == list(range(4096))
    assert a.n_gpu == 2048
    # general FP8 + scale recipe
    c = gen.DecodeConfig("g", 2, (100, 300), 16, "general", True, 0.5, 4, seed=9)
    g = gen.make_decode_inputs(c)
    assert ((g.k_scale >= 0.5) & (g.k_scale <= 2.0)).all()
    assert 100 <= g.key_len.min() and g.key_len.max() <= 300
    kv = oracle.decode_e4m3fn(g.k)
    assert abs(kv.std() - 1.0) < 0.1


def test_latent_rows_finite_and_not_poison():
    rows = gen.fill_latent_rows(3, np.empty((1000, 576), np.uint16))
    assert not (rows == gen.POISON).any()
    assert ((rows & 0x7F80) != 0x7F80).all()      # bf16 exponent never all-ones


def test_tiny_step_invariants():
    cfg = gen.CONFIGS["tiny"]
    inp = gen.make_decode_inputs(cfg)
    host_kv = gen.fill_latent_rows(cfg.seed, np.empty((inp.n_host, 576), np.uint16))
    scores = oracle.index_scores(inp.q, inp.w, inp.k, inp.k_scale, inp.key_begin, inp.key_len)
    idx = oracle.topk_rows(scores, cfg.topk)
    p = gen.make_pool_state(inp, idx, host_kv)
    st = oracle.PoolState(p.free, p.priority, p.to_host, p.host_to_gpu, p.indices_buf, p.gpu_kv)
    oracle.check_pool_invariants(st)
    assert (st.free == 0).all()                    # the tiny pool starts full
    new, res = oracle.pool_step(st, host_kv, idx, inp.key_begin, inp.req_to_host, p.step_id)
    assert res.status == 0
    sel = idx[0]
    assert (sel >= 0).sum() == 256 and (np.diff(sel) > 0).all()
    s = scores[0]
    mask = np.zeros(len(s), bool)
    mask[sel] = True
    assert s[mask].min() >= s[~mask].max()
    hosts = inp.req_to_host[sel]
    oracle.check_pool_invariants(new, host_kv, hosts, res.topk_slot[0])
    # about half of the selected rows were resident (random half of all tokens)
    assert 64 < res.n_miss < 192
    assert res.n_evicted == res.n_miss


def test_pool_state_hit_rate():
    c = gen.DecodeConfig("h", 3, 2000, 64, "int", False, 0.9, 8, reserve=10, seed=7)
    inp = gen.make_decode_inputs(c)
    host_kv = gen.fill_latent_rows(c.seed, np.empty((inp.n_host, 576), np.uint16))
    scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
    idx = oracle.topk_rows(scores, c.topk)
    p = gen.make_pool_state(inp, idx, host_kv)
    assert int(p.free.sum()) == 10
    for r in range(3):
        h = inp.req_to_host[inp.key_begin[r] + idx[r]]
        assert (p.host_to_gpu[h] != gen.INF).sum() == round(0.9 * 64)
