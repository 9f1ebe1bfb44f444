"""Host-side logic of the C ABI, exercised without a GPU: every call here is rejected by its
argument checks, or is a pure size query, before the library touches the HIP runtime.

Checked: the documented error codes and the thread-local error text, the workspace-size
queries (monotone in the sizes they depend on, zero for invalid sizes, large enough for the
decode step's staging rows), and the pool metadata footprint against the oracle's formula
(the ECHO page's 4 N_H + 13 N_G, §5.1)."""

import ctypes as C
import os
import threading

import pytest

from dsa_indexer_top_amd import binding as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")

FAKE = C.c_void_p(0x1000)      # never dereferenced: every call below fails before any access


def _err():
    return B.lib().echo_last_error().decode()


def _decode_args(**kw):
    a = B.DecodeArgs(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 8, 65536, 2048, 7, 0, 4, 4096,
                     95.0, 2048, 1024)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _pool(n_gpu=1024, n_host=4096):
    return B.Pool(n_gpu, n_host, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def _out():
    return B.DecodeOut(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def test_index_scores_argument_errors():
    L = B.lib()
    assert L.echo_index_scores(FAKE, FAKE, FAKE, None, FAKE, FAKE, -1, 16, FAKE, 16, None) == B.ECHO_EINVAL
    assert "negative" in _err()
    assert L.echo_index_scores(FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 16, FAKE, 8, None) == B.ECHO_EINVAL
    assert "ld" in _err()
    assert L.echo_index_scores(FAKE, FAKE, FAKE, None, FAKE, FAKE, 70000, 16, FAKE, 16, None) == B.ECHO_EUNSUPPORTED
    assert L.echo_index_scores(None, FAKE, FAKE, None, FAKE, FAKE, 1, 16, FAKE, 16, None) == B.ECHO_EINVAL
    assert "NULL" in _err()


def test_paged_key_cache_argument_errors():
    L = B.lib()
    ok = dict(page_size=64, max_pages=4)
    call = lambda ps, mp, tbl=FAKE, ml=256: L.echo_index_scores_paged(
        FAKE, FAKE, FAKE, None, tbl, ps, mp, FAKE, 2, ml, FAKE, 256, None)
    assert call(48, 4) == B.ECHO_EUNSUPPORTED and "power of two" in _err()
    assert call(8, 64) == B.ECHO_EUNSUPPORTED
    assert call(64, 3) == B.ECHO_EINVAL and "pages" in _err()      # 3 x 64 < 256
    assert call(64, 4, tbl=None) == B.ECHO_EINVAL and "page table" in _err()
    # the decode step: the same checks, and no fused prefetch over pages
    pool, out = _pool(), _out()
    for ps, mp, mode, code in ((48, 4, 0, B.ECHO_EUNSUPPORTED), (64, 1, 0, B.ECHO_EINVAL),
                               (64, 1024, 2, B.ECHO_EUNSUPPORTED)):
        a = _decode_args(max_key_len=256, prefetch=mode)
        a.k_page_table, a.k_page_size, a.k_max_pages = FAKE, ps, mp
        assert L.echo_decode_select(C.byref(a), C.byref(pool), C.byref(out), FAKE, 1 << 40,
                                    None, None) == code, (ps, mp, mode)


def test_prefill_and_topk_argument_errors():
    L = B.lib()
    assert L.echo_index_scores_prefill(FAKE, FAKE, FAKE, -1, 8, 0, FAKE, 8, None) == B.ECHO_EINVAL
    assert L.echo_index_scores_prefill(FAKE, FAKE, FAKE, 8, 8, 0, FAKE, 4, None) == B.ECHO_EINVAL
    assert L.echo_index_scores_prefill(None, FAKE, FAKE, 8, 8, 0, FAKE, 8, None) == B.ECHO_EINVAL
    for k in (0, 4097):
        assert L.echo_topk(FAKE, 64, FAKE, 1, 64, k, FAKE, None, 0, None) == B.ECHO_EUNSUPPORTED
        assert "outside" in _err()
    assert L.echo_topk(FAKE, 32, FAKE, 1, 64, 8, FAKE, None, 0, None) == B.ECHO_EINVAL
    assert L.echo_topk(None, 64, FAKE, 1, 64, 8, FAKE, None, 0, None) == B.ECHO_EINVAL


def test_empty_calls_are_no_ops():
    # no queries, no keys or no rows: ECHO_OK with nothing enqueued and nothing read or written
    # (the pointers here are never valid, and no HIP runtime call is made)
    L = B.lib()
    assert L.echo_index_scores_prefill(FAKE, FAKE, FAKE, 0, 8, 0, FAKE, 8, None) == B.ECHO_OK
    assert L.echo_index_scores_prefill(FAKE, FAKE, FAKE, 8, 0, 0, FAKE, 0, None) == B.ECHO_OK
    assert L.echo_topk(FAKE, 64, FAKE, 0, 64, 8, FAKE, None, 0, None) == B.ECHO_OK
    assert L.echo_index_scores(FAKE, FAKE, FAKE, None, FAKE, FAKE, 0, 16, FAKE, 16, None) == B.ECHO_OK
    assert L.echo_index_scores(FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 0, FAKE, 0, None) == B.ECHO_OK


def test_static_pool_entry_point_errors():
    # the no-allocation variant rejects, before touching the runtime, what the plain entry point
    # rejects, and any size whose workspace would not fit its fixed scratch array
    L = B.lib()
    none = C.POINTER(B.Pool)()
    args = (FAKE, FAKE, FAKE, 4096, 1, 8, 3, FAKE, FAKE, FAKE, FAKE, None)
    assert L.echo_pool_lookup_alloc_static(none, *args) == B.ECHO_EINVAL
    bad_k = (FAKE, FAKE, FAKE, 4096, 1, 5000, 3, FAKE, FAKE, FAKE, FAKE, None)
    assert L.echo_pool_lookup_alloc_static(C.byref(_pool()), *bad_k) == B.ECHO_EINVAL
    assert L.echo_pool_lookup_alloc_static(C.byref(_pool()), FAKE, FAKE, FAKE, 4096, 1, 8, 3, FAKE,
                                           FAKE, None, FAKE, None) == B.ECHO_EINVAL
    # the largest pool the array serves: the bench's biggest workload (64 x top-2048 over 2^20
    # slots) fits; 4M slots do not
    assert B.lib().echo_pool_workspace_bytes(64, 2048, 1 << 20) <= B.STATIC_SCRATCH_BYTES
    big = _pool(n_gpu=1 << 22)
    assert B.lib().echo_pool_workspace_bytes(64, 2048, 1 << 22) > B.STATIC_SCRATCH_BYTES
    too_big = (FAKE, FAKE, FAKE, 4096, 64, 2048, 3, FAKE, FAKE, FAKE, FAKE, None)
    assert L.echo_pool_lookup_alloc_static(C.byref(big), *too_big) == B.ECHO_EUNSUPPORTED
    assert "scratch" in _err()


def test_pool_entry_point_errors():
    L = B.lib()
    none = C.POINTER(B.Pool)()
    args = (FAKE, FAKE, FAKE, 4096, 1, 8, 3, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert L.echo_pool_lookup_alloc(none, *args) == B.ECHO_EINVAL
    big = _pool(n_gpu=(1 << 22) + 1)
    assert L.echo_pool_lookup_alloc(C.byref(big), *args) == B.ECHO_EUNSUPPORTED
    p = _pool()
    bad_k = (FAKE, FAKE, FAKE, 4096, 1, 5000, 3, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert L.echo_pool_lookup_alloc(C.byref(p), *bad_k) == B.ECHO_EINVAL
    assert L.echo_recall(none, FAKE, FAKE, FAKE, 8, B.RECALL_GATHER, None) == B.ECHO_EINVAL
    assert L.echo_recall(C.byref(p), FAKE, FAKE, FAKE, -1, B.RECALL_GATHER, None) == B.ECHO_EINVAL
    assert L.echo_recall(C.byref(p), FAKE, FAKE, FAKE, 8, 7, None) == B.ECHO_EINVAL
    assert "mode" in _err()
    for member in ("gpu_kv", "host_kv", "status", "host_to_gpu"):
        q = _pool()
        setattr(q, member, None)
        assert L.echo_recall(C.byref(q), FAKE, FAKE, FAKE, 8, B.RECALL_GATHER, None) == B.ECHO_EINVAL, member
    assert L.echo_recall(C.byref(_pool(n_host=0)), FAKE, FAKE, FAKE, 8, B.RECALL_GATHER, None) == B.ECHO_EINVAL
    assert L.echo_status_clear(None, None) == B.ECHO_EINVAL
    assert L.echo_pool_init(none, None) == B.ECHO_EINVAL
    gather = (FAKE, FAKE, FAKE, FAKE, 8, 16, FAKE, FAKE, FAKE, None)
    for member in ("gpu_free", "gpu_priority", "gpu_to_host", "host_to_gpu", "gpu_kv", "host_kv", "status"):
        q = _pool()
        setattr(q, member, None)
        assert L.echo_prefetch_gather(C.byref(q), *gather) == B.ECHO_EINVAL, member
    assert L.echo_prefetch_gather(C.byref(_pool(n_gpu=0)), *gather) == B.ECHO_EINVAL
    assert L.echo_prefetch_begin(C.byref(_pool()), None, FAKE, None) == B.ECHO_EINVAL


def test_decode_select_argument_errors():
    L = B.lib()
    p, o = _pool(), _out()
    cases = [
        (dict(n_rows=0), B.ECHO_EUNSUPPORTED),
        (dict(n_rows=70000), B.ECHO_EUNSUPPORTED),
        (dict(topk=0), B.ECHO_EUNSUPPORTED),
        (dict(topk=4097), B.ECHO_EUNSUPPORTED),
        (dict(max_key_len=-1), B.ECHO_EINVAL),
        (dict(q=None), B.ECHO_EINVAL),
        (dict(prefetch=1, n_chunks=0), B.ECHO_EUNSUPPORTED),
        (dict(prefetch=1, n_chunks=17), B.ECHO_EUNSUPPORTED),
        (dict(prefetch=1, n_sample=1000), B.ECHO_EUNSUPPORTED),
        (dict(prefetch=1, percentile=0.0), B.ECHO_EINVAL),
        (dict(prefetch=1, cap=0), B.ECHO_EINVAL),
        (dict(prefetch=3), B.ECHO_EUNSUPPORTED),
        (dict(prefetch=-1), B.ECHO_EUNSUPPORTED),
        (dict(prefetch=2, pf_range=100), B.ECHO_EUNSUPPORTED),
        (dict(prefetch=2, pf_range=8192 + 128), B.ECHO_EUNSUPPORTED),
        (dict(prefetch=2, cap_div=0), B.ECHO_EINVAL),
        (dict(prefetch=2, n_sample=100), B.ECHO_EUNSUPPORTED),
    ]
    for kw, code in cases:
        a = _decode_args(**kw)
        assert L.echo_decode_select(C.byref(a), C.byref(p), C.byref(o), FAKE, 1 << 30, None, None) == code, kw
    a = _decode_args()
    short = L.echo_decode_workspace_bytes(C.byref(a), p.n_gpu) - 1
    assert L.echo_decode_select(C.byref(a), C.byref(p), C.byref(o), FAKE, short, None, None) == B.ECHO_EWORKSPACE
    assert "workspace" in _err()
    g = C.c_void_p()
    assert L.echo_graph_capture_decode(C.byref(a), C.byref(p), C.byref(o), FAKE, 1 << 30, None, None,
                                       None) == B.ECHO_EINVAL
    assert L.echo_graph_capture_decode(C.byref(a), C.byref(p), C.byref(o), FAKE, 1 << 30, None, None,
                                       C.byref(g)) == B.ECHO_EINVAL          # NULL main stream
    assert not g.value
    assert L.echo_graph_launch(None, None) == B.ECHO_EINVAL
    assert L.echo_graph_destroy(None) == B.ECHO_OK


def _append_args(**kw):
    a = B.AppendArgs(4, 1024, 4096, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 9)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_decode_append_and_ema_argument_errors():
    L = B.lib()
    p = _pool()
    slot = FAKE
    cases = [
        (dict(n_rows=0), B.ECHO_EUNSUPPORTED),
        (dict(n_rows=70000), B.ECHO_EUNSUPPORTED),
        (dict(capacity=0), B.ECHO_EINVAL),
        (dict(n_k=0), B.ECHO_EINVAL),
        (dict(new_kv=None), B.ECHO_EINVAL),
        (dict(host_kv_w=None), B.ECHO_EINVAL),
        (dict(key_len=None), B.ECHO_EINVAL),
        (dict(k_scale=FAKE), B.ECHO_EINVAL),              # a key scale with no new scales
        (dict(new_scale=FAKE), B.ECHO_EINVAL),
    ]
    for kw, code in cases:
        a = _append_args(**kw)
        assert L.echo_decode_append(C.byref(a), C.byref(p), slot, FAKE, 1 << 30, None) == code, kw
    a = _append_args()
    assert L.echo_decode_append(C.byref(a), C.byref(p), None, FAKE, 1 << 30, None) == B.ECHO_EINVAL
    assert L.echo_decode_append(C.byref(a), C.POINTER(B.Pool)(), slot, FAKE, 1 << 30, None) == B.ECHO_EINVAL
    q = _pool()
    q.gpu_kv = None
    assert L.echo_decode_append(C.byref(a), C.byref(q), slot, FAKE, 1 << 30, None) == B.ECHO_EINVAL
    short = L.echo_append_workspace_bytes(4, p.n_gpu) - 1
    assert L.echo_decode_append(C.byref(a), C.byref(p), slot, FAKE, short, None) == B.ECHO_EWORKSPACE
    assert L.echo_append_workspace_bytes(-1, 8) == 0
    assert L.echo_append_workspace_bytes(8, 1 << 20) > L.echo_append_workspace_bytes(8, 1024)
    assert L.echo_step_advance(None, None) == B.ECHO_EINVAL
    assert L.echo_graph_begin(None) == B.ECHO_EINVAL
    assert L.echo_graph_end(None, None) == B.ECHO_EINVAL
    # the EMA weight must lie in [0, 1] when an estimate buffer is given
    for alpha in (-0.5, 1.5, float("nan")):
        d = _decode_args(theta_ema=FAKE, ema_alpha=alpha)
        assert L.echo_decode_select(C.byref(d), C.byref(p), C.byref(_out()), FAKE, 1 << 30, None,
                                    None) == B.ECHO_EINVAL, alpha
        assert "ema_alpha" in _err()


def test_interquery_argument_errors():
    L = B.lib()
    # echo_topk_subset(scores, ld, len, n_rows, max_len, k, shift, subset, cnt, thr, stream)
    assert L.echo_topk_subset(FAKE, 64, FAKE, -1, 64, 8, None, FAKE, FAKE, None, None) == B.ECHO_EINVAL
    for k in (0, 4097):
        assert L.echo_topk_subset(FAKE, 64, FAKE, 1, 64, k, None, FAKE, FAKE, None, None) == B.ECHO_EUNSUPPORTED
    assert L.echo_topk_subset(FAKE, 32, FAKE, 1, 64, 8, None, FAKE, FAKE, None, None) == B.ECHO_EINVAL
    assert L.echo_topk_subset(FAKE, 64, FAKE, 1, 64, 8, None, None, FAKE, None, None) == B.ECHO_EINVAL
    assert L.echo_topk_subset(None, 64, None, 0, 64, 8, None, None, None, None, None) == B.ECHO_OK
    # echo_union_rows(idx, n_rows, k, n_keys, out, cnt, ws, ws_bytes, stream)
    assert L.echo_union_rows(FAKE, 2, 8, -1, FAKE, FAKE, FAKE, 1 << 20, None) == B.ECHO_EINVAL
    assert L.echo_union_rows(None, 2, 8, 100, FAKE, FAKE, FAKE, 1 << 20, None) == B.ECHO_EINVAL
    need = L.echo_union_workspace_bytes(9000)
    assert need == 3 * 4096 // 8 and L.echo_union_workspace_bytes(0) == 512
    assert L.echo_union_workspace_bytes(-1) == 0
    assert L.echo_union_rows(FAKE, 2, 8, 9000, FAKE, FAKE, FAKE, need - 1, None) == B.ECHO_EWORKSPACE
    # echo_threshold_ema(scores, ld, idx, n_rows, k, alpha, theta, kth, stream)
    assert L.echo_threshold_ema(FAKE, 64, FAKE, 1, 8, 1.5, FAKE, None, None) == B.ECHO_EINVAL
    assert L.echo_threshold_ema(FAKE, 64, FAKE, 1, 0, 0.5, FAKE, None, None) == B.ECHO_EUNSUPPORTED
    assert L.echo_threshold_ema(FAKE, 64, FAKE, 1, 8, 0.5, None, None, None) == B.ECHO_EINVAL


def test_fused_prefetch_argument_errors():
    L = B.lib()
    p, ws = _pool(), 1 << 30

    def call(n_q=2, max_len=4096, ld=4096, cap=64, cap_div=8, rng=0, pool=p, w=FAKE, nbytes=ws,
             theta=FAKE):
        return L.echo_index_scores_fused(FAKE, FAKE, FAKE, None, FAKE, FAKE, n_q, max_len, FAKE, ld,
                                         theta, FAKE, C.byref(pool) if pool is not None else None,
                                         cap, cap_div, rng, FAKE, None, w, nbytes, None)
    assert call(n_q=-1) == B.ECHO_EINVAL and "negative" in _err()
    assert call(n_q=70000) == B.ECHO_EUNSUPPORTED
    assert call(max_len=(1 << 22) + 1, ld=(1 << 22) + 1) == B.ECHO_EUNSUPPORTED
    assert call(ld=100) == B.ECHO_EINVAL and "ld" in _err()
    assert call(cap=-1) == B.ECHO_EINVAL
    assert call(cap_div=0) == B.ECHO_EINVAL
    assert call(pool=None) == B.ECHO_EINVAL
    assert call(pool=_pool(n_gpu=0)) == B.ECHO_EINVAL
    assert call(pool=_pool(n_gpu=(1 << 22) + 1)) == B.ECHO_EUNSUPPORTED
    assert call(w=None) == B.ECHO_EINVAL
    assert call(theta=None) == B.ECHO_EINVAL and "NULL" in _err()
    need = L.echo_fused_workspace_bytes(2, p.n_gpu)
    assert need >= p.n_gpu * 4                       # the free-slot list fits
    assert call(nbytes=need - 1) == B.ECHO_EWORKSPACE and "workspace" in _err()
    for rng in (64, 129, 8192 + 128, -128):
        assert call(rng=rng) == B.ECHO_EUNSUPPORTED, rng
        assert "range" in _err()
    assert L.echo_fused_workspace_bytes(-1, 8) == 0
    assert L.echo_fused_workspace_bytes(8, 1 << 20) > L.echo_fused_workspace_bytes(8, 1 << 16)


def test_workspace_sizes():
    L = B.lib()
    assert L.echo_pool_workspace_bytes(-1, 8, 8) == 0
    assert L.echo_topk_workspace_bytes(-1, 8) == 0
    base = L.echo_pool_workspace_bytes(8, 2048, 65536)
    assert L.echo_pool_workspace_bytes(16, 2048, 65536) > base
    assert L.echo_pool_workspace_bytes(8, 2048, 1 << 20) > base
    prev = 0
    for n_rows, k in [(1, 256), (8, 2048), (32, 2048), (64, 2048)]:
        a = _decode_args(n_rows=n_rows, topk=k, max_key_len=131072)
        ws = L.echo_decode_workspace_bytes(C.byref(a), 1 << 20)
        assert ws >= n_rows * k * 576 * 2          # the staged recall rows fit
        assert ws > prev
        prev = ws
    a = _decode_args()
    pf = _decode_args(prefetch=1)
    assert L.echo_decode_workspace_bytes(C.byref(pf), 65536) > L.echo_decode_workspace_bytes(C.byref(a), 65536)
    fz = _decode_args(prefetch=2, n_chunks=0)
    assert L.echo_decode_workspace_bytes(C.byref(fz), 65536) >= (
        L.echo_decode_workspace_bytes(C.byref(a), 65536) + L.echo_fused_workspace_bytes(8, 65536))
    assert L.echo_decode_workspace_bytes(C.byref(_decode_args(n_rows=-1)), 65536) == 0
    assert L.echo_decode_workspace_bytes(C.byref(a), -1) == 0


def test_metadata_footprint_matches_oracle():
    import oracle
    L = B.lib()
    for n_host, n_gpu in [(1, 1), (4096, 2048), (524288, 65536), (8388608, 1048576)]:
        assert L.echo_pool_metadata_bytes(n_host, n_gpu) == oracle.metadata_bytes(n_host, n_gpu)


def test_error_text_is_per_thread():
    L = B.lib()
    assert L.echo_topk(FAKE, 64, FAKE, 1, 64, 0, FAKE, None, 0, None) == B.ECHO_EUNSUPPORTED
    here = _err()
    seen = []

    def other():
        seen.append(B.lib().echo_last_error().decode())
        B.lib().echo_index_scores(None, FAKE, FAKE, None, FAKE, FAKE, 1, 16, FAKE, 16, None)
        seen.append(B.lib().echo_last_error().decode())

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen[0] == ""
    assert "NULL" in seen[1]
    assert _err() == here
