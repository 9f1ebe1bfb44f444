"""ctypes binding of libecho.so: the same names as the C ABI, argument marshalling only.

Every step of the decode path runs in the HIP library; this module passes device pointers,
sizes and stream handles through and turns nonzero return codes into exceptions.  torch is
used only to hold device memory and to name streams.  If the library is missing the import of
`lib()` raises: there is no fallback path.
"""

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libecho.so")

ECHO_OK, ECHO_EINVAL, ECHO_EUNSUPPORTED, ECHO_EHIP, ECHO_EWORKSPACE = 0, -1, -2, -3, -4
ST_EXHAUSTED, ST_BAD_HOST, ST_DUP_HOST, ST_CACHE_FULL = 1, 2, 4, 8
RECALL_GATHER, RECALL_MEMCPY = 0, 1
PREFETCH_OFF, PREFETCH_RANGED, PREFETCH_FUSED = 0, 1, 2
FUSED_MAX_RANGE, FUSED_MAX_PER_RANGE = 8192, 128
INF = 0x7FFFFFFF
ROW_ELEMS = 576

P = C.c_void_p
I32, I64, SZ, F32 = C.c_int32, C.c_int64, C.c_size_t, C.c_float


class EchoError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__("%s returned %d: %s" % (fn, code, msg))
        self.code = code


class Pool(C.Structure):
    _fields_ = [("n_gpu", I32), ("n_host", I32), ("gpu_free", P), ("gpu_priority", P),
                ("gpu_to_host", P), ("host_to_gpu", P), ("indices_buf", P), ("gpu_kv", P),
                ("host_kv", P), ("status", P)]


class DecodeArgs(C.Structure):
    _fields_ = [("q", P), ("w", P), ("k", P), ("k_scale", P), ("key_begin", P),
                ("key_len", P), ("req_to_host", P), ("n_rows", I32), ("max_key_len", I32),
                ("topk", I32), ("step_id", I32), ("prefetch", I32), ("n_chunks", I32),
                ("n_sample", I32), ("percentile", F32), ("cap", I32), ("cap_div", I32),
                ("theta_ema", P), ("ema_alpha", F32), ("step_dev", P), ("reserve_free", I32),
                ("pf_range", I32), ("k_page_table", P), ("k_page_size", I32), ("k_max_pages", I32)]


class DecodeOut(C.Structure):
    _fields_ = [("scores", P), ("topk_idx", P), ("topk_slot", P), ("miss_host", P),
                ("miss_slot", P), ("counters", P), ("kth", P)]


class AppendArgs(C.Structure):
    _fields_ = [("n_rows", I32), ("capacity", I32), ("n_k", I64), ("new_k", P), ("new_scale", P),
                ("new_kv", P), ("new_host", P), ("k", P), ("k_scale", P), ("key_begin", P),
                ("key_len", P), ("req_to_host", P), ("host_kv_w", P), ("step_id", I32),
                ("step_dev", P)]


_SIGS = {
    "echo_last_error": (C.c_char_p, []),
    "echo_version": (C.c_char_p, []),
    "echo_pool_metadata_bytes": (SZ, [I32, I32]),
    "echo_pool_init": (C.c_int, [C.POINTER(Pool), P]),
    "echo_status_clear": (C.c_int, [P, P]),
    "echo_index_scores": (C.c_int, [P, P, P, P, P, P, I32, I32, P, I64, P]),
    "echo_index_scores_hist": (C.c_int, [P, P, P, P, P, P, I32, I32, P, I64, P, P]),
    "echo_index_scores_paged": (C.c_int, [P, P, P, P, P, I32, I32, P, I32, I32, P, I64, P]),
    "echo_index_scores_prefetch": (C.c_int, [P, P, P, P, P, P, I32, I32, I32, I32, P, I64,
                                             P, P, P, I32, P, P, P, I32, I32, P]),
    "echo_prefetch_threshold": (C.c_int, [P, P, P, P, P, P, I32, I32, I32, F32, P, P]),
    "echo_fused_workspace_bytes": (SZ, [I32, I32]),
    "echo_index_scores_fused": (C.c_int, [P, P, P, P, P, P, I32, I32, P, I64, P, P,
                                          C.POINTER(Pool), I32, I32, I32, P, P, P, SZ, P]),
    "echo_index_scores_prefill": (C.c_int, [P, P, P, I32, I32, I32, P, I64, P]),
    "echo_topk_workspace_bytes": (SZ, [I32, I32]),
    "echo_topk": (C.c_int, [P, I64, P, I32, I32, I32, P, P, SZ, P]),
    "echo_topk_subset": (C.c_int, [P, I64, P, I32, I32, I32, P, P, P, P, P]),
    "echo_union_workspace_bytes": (SZ, [I32]),
    "echo_union_rows": (C.c_int, [P, I32, I32, I32, P, P, P, SZ, P]),
    "echo_threshold_ema": (C.c_int, [P, I64, P, I32, I32, F32, P, P, P]),
    "echo_pool_workspace_bytes": (SZ, [I32, I32, I32]),
    "echo_pool_lookup_alloc": (C.c_int, [C.POINTER(Pool), P, P, P, I64, I32, I32, I32, P, P, P,
                                         P, P, SZ, P]),
    "echo_pool_lookup_alloc_static": (C.c_int, [C.POINTER(Pool), P, P, P, I64, I32, I32, I32, P,
                                                P, P, P, P]),
    "echo_recall": (C.c_int, [C.POINTER(Pool), P, P, P, I32, I32, P]),
    "echo_prefetch_begin": (C.c_int, [C.POINTER(Pool), P, P, P]),
    "echo_prefetch_gather": (C.c_int, [C.POINTER(Pool), P, P, P, P, I32, I32, P, P, P, P]),
    "echo_decode_workspace_bytes": (SZ, [C.POINTER(DecodeArgs), I32]),
    "echo_decode_select": (C.c_int, [C.POINTER(DecodeArgs), C.POINTER(Pool),
                                     C.POINTER(DecodeOut), P, SZ, P, P]),
    "echo_append_workspace_bytes": (SZ, [I32, I32]),
    "echo_decode_append": (C.c_int, [C.POINTER(AppendArgs), C.POINTER(Pool), P, P, SZ, P]),
    "echo_graph_capture_decode": (C.c_int, [C.POINTER(DecodeArgs), C.POINTER(Pool),
                                            C.POINTER(DecodeOut), P, SZ, P, P, C.POINTER(P)]),
    "echo_step_advance": (C.c_int, [P, P]),
    "echo_graph_begin": (C.c_int, [P]),
    "echo_graph_end": (C.c_int, [P, C.POINTER(P)]),
    "echo_graph_launch": (C.c_int, [P, P]),
    "echo_graph_destroy": (C.c_int, [P]),
    "echo_host_alloc": (C.c_int, [SZ, C.c_int, C.POINTER(P), C.POINTER(P)]),
    "echo_host_free": (C.c_int, [P]),
}

EXPORTED = sorted(_SIGS)
STATIC_SCRATCH_BYTES = 16 << 20      # echo.h ECHO_STATIC_SCRATCH_BYTES

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libecho.so not built at %s (run __graft_entry__.build())" % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn, code):
    if code != ECHO_OK:
        raise EchoError(fn, code, lib().echo_last_error().decode())


def _call(name, *args):
    _check(name, getattr(lib(), name)(*args))


# ---------------------------------------------------------------- torch plumbing helpers
def ptr(t):
    """Device (or host) address of a tensor, None for None."""
    return None if t is None else t.data_ptr()


def stream_handle(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ---------------------------------------------------------------- entry points
def version():
    return lib().echo_version().decode()


def pool_metadata_bytes(n_host, n_gpu):
    return lib().echo_pool_metadata_bytes(n_host, n_gpu)


def index_scores(q, w, k, k_scale, key_begin, key_len, max_key_len, scores, ld=None, stream=None):
    ld = scores.shape[-1] if ld is None else ld
    _call("echo_index_scores", ptr(q), ptr(w), ptr(k), ptr(k_scale), ptr(key_begin),
          ptr(key_len), q.shape[0], max_key_len, ptr(scores), ld, stream_handle(stream))


def index_scores_paged(q, w, k_pages, k_scale_pages, page_table, page_size, key_len, max_key_len,
                       scores, ld=None, stream=None):
    ld = scores.shape[-1] if ld is None else ld
    _call("echo_index_scores_paged", ptr(q), ptr(w), ptr(k_pages), ptr(k_scale_pages),
          ptr(page_table), page_size, page_table.shape[1], ptr(key_len), q.shape[0], max_key_len,
          ptr(scores), ld, stream_handle(stream))


def index_scores_hist(q, w, k, k_scale, key_begin, key_len, max_key_len, scores, hist, ld=None,
                      stream=None):
    ld = scores.shape[-1] if ld is None else ld
    _call("echo_index_scores_hist", ptr(q), ptr(w), ptr(k), ptr(k_scale), ptr(key_begin),
          ptr(key_len), q.shape[0], max_key_len, ptr(scores), ld, ptr(hist), stream_handle(stream))


def index_scores_prefetch(q, w, k, k_scale, key_begin, key_len, max_key_len, tok_lo, tok_hi,
                          scores, theta, req_to_host, host_to_gpu, cand, cand_cnt, total_cnt,
                          cap, cap_div, ld=None, stream=None):
    ld = scores.shape[-1] if ld is None else ld
    _call("echo_index_scores_prefetch", ptr(q), ptr(w), ptr(k), ptr(k_scale), ptr(key_begin),
          ptr(key_len), q.shape[0], max_key_len, tok_lo, tok_hi, ptr(scores), ld, ptr(theta),
          ptr(req_to_host), ptr(host_to_gpu), host_to_gpu.shape[0], ptr(cand), ptr(cand_cnt),
          ptr(total_cnt), cap, cap_div, stream_handle(stream))


def fused_workspace_bytes(n_q, n_gpu):
    return lib().echo_fused_workspace_bytes(n_q, n_gpu)


def index_scores_fused(q, w, k, k_scale, key_begin, key_len, max_key_len, scores, theta,
                       req_to_host, pool, cap, cap_div, range_len, n_prefetched, demand, ws,
                       ld=None, stream=None):
    ld = scores.shape[-1] if ld is None else ld
    _call("echo_index_scores_fused", ptr(q), ptr(w), ptr(k), ptr(k_scale), ptr(key_begin),
          ptr(key_len), q.shape[0], max_key_len, ptr(scores), ld, ptr(theta), ptr(req_to_host),
          C.byref(pool), cap, cap_div, range_len, ptr(n_prefetched), ptr(demand), ptr(ws),
          ws.numel() * ws.element_size(), stream_handle(stream))


def prefetch_mode(prefetch):
    """PREFETCH_* code of False / True / "ranged" / "fused" (or the code itself)."""
    if prefetch in (False, None, 0, "off"):
        return PREFETCH_OFF
    if prefetch in (True, 1, "ranged"):
        return PREFETCH_RANGED
    if prefetch in (2, "fused"):
        return PREFETCH_FUSED
    raise ValueError("prefetch mode %r" % (prefetch,))


def prefetch_begin(pool, free_list, free_count, stream=None):
    _call("echo_prefetch_begin", C.byref(pool), ptr(free_list), ptr(free_count),
          stream_handle(stream))


def prefetch_gather(pool, key_begin, req_to_host, cand, cand_cnt, cap, free_list, free_count,
                    n_prefetched, stream=None):
    _call("echo_prefetch_gather", C.byref(pool), ptr(key_begin), ptr(req_to_host), ptr(cand),
          ptr(cand_cnt), cand_cnt.shape[0], cap, ptr(free_list), ptr(free_count),
          ptr(n_prefetched), stream_handle(stream))


def prefetch_threshold(q, w, k, k_scale, key_begin, key_len, max_key_len, n_sample, percentile,
                       theta, stream=None):
    _call("echo_prefetch_threshold", ptr(q), ptr(w), ptr(k), ptr(k_scale), ptr(key_begin),
          ptr(key_len), q.shape[0], max_key_len, n_sample, percentile, ptr(theta),
          stream_handle(stream))


def index_scores_prefill(q, w, k, scores, q_pos0=0, ld=None, stream=None):
    ld = scores.shape[-1] if ld is None else ld
    _call("echo_index_scores_prefill", ptr(q), ptr(w), ptr(k), q.shape[0], k.shape[0], q_pos0,
          ptr(scores), ld, stream_handle(stream))


def topk_workspace_bytes(n_rows, max_len):
    return lib().echo_topk_workspace_bytes(n_rows, max_len)


def topk(scores, length, max_len, k, idx, ws, ld=None, stream=None):
    ld = scores.shape[-1] if ld is None else ld
    _call("echo_topk", ptr(scores), ld, ptr(length), length.shape[0], max_len, k, ptr(idx),
          ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream))


def topk_subset(scores, length, max_len, k, shift, subset, subset_cnt, thr_cnt=None, ld=None,
                stream=None):
    ld = scores.shape[-1] if ld is None else ld
    _call("echo_topk_subset", ptr(scores), ld, ptr(length), length.shape[0], max_len, k,
          ptr(shift), ptr(subset), ptr(subset_cnt), ptr(thr_cnt), stream_handle(stream))


def union_workspace_bytes(n_keys):
    return lib().echo_union_workspace_bytes(n_keys)


def union_rows(idx, n_keys, out, out_cnt, ws, stream=None):
    _call("echo_union_rows", ptr(idx), idx.shape[0], idx.shape[1], n_keys, ptr(out), ptr(out_cnt),
          ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream))


def threshold_ema(scores, idx, alpha, theta=None, kth=None, ld=None, stream=None):
    ld = scores.shape[-1] if ld is None else ld
    _call("echo_threshold_ema", ptr(scores), ld, ptr(idx), idx.shape[0], idx.shape[1], alpha,
          ptr(theta), ptr(kth), stream_handle(stream))


def make_pool(n_gpu, n_host, free, priority, to_host, host_to_gpu, indices_buf, gpu_kv,
              host_kv_dev, status):
    return Pool(n_gpu, n_host, ptr(free), ptr(priority), ptr(to_host), ptr(host_to_gpu),
                ptr(indices_buf), ptr(gpu_kv), host_kv_dev, ptr(status))


def pool_init(pool, stream=None):
    _call("echo_pool_init", C.byref(pool), stream_handle(stream))


def status_clear(status, stream=None):
    _call("echo_status_clear", ptr(status), stream_handle(stream))


def pool_workspace_bytes(n_rows, k, n_gpu):
    return lib().echo_pool_workspace_bytes(n_rows, k, n_gpu)


def pool_lookup_alloc(pool, idx, key_begin, req_to_host, step_id, topk_slot, miss_host,
                      miss_slot, n_miss, ws, stream=None):
    _call("echo_pool_lookup_alloc", C.byref(pool), ptr(idx), ptr(key_begin), ptr(req_to_host),
          req_to_host.shape[0], idx.shape[0], idx.shape[1], step_id, ptr(topk_slot), ptr(miss_host), ptr(miss_slot),
          ptr(n_miss), ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream))


def pool_lookup_alloc_static(pool, idx, key_begin, req_to_host, step_id, topk_slot, miss_host,
                             miss_slot, n_miss, stream=None):
    _call("echo_pool_lookup_alloc_static", C.byref(pool), ptr(idx), ptr(key_begin),
          ptr(req_to_host), req_to_host.shape[0], idx.shape[0], idx.shape[1], step_id,
          ptr(topk_slot), ptr(miss_host), ptr(miss_slot), ptr(n_miss), stream_handle(stream))


def recall(pool, miss_host, miss_slot, n_miss, max_miss, mode=RECALL_GATHER, stream=None):
    _call("echo_recall", C.byref(pool), ptr(miss_host), ptr(miss_slot), ptr(n_miss), max_miss,
          mode, stream_handle(stream))


def decode_workspace_bytes(args, n_gpu):
    return lib().echo_decode_workspace_bytes(C.byref(args), n_gpu)


def decode_select(args, pool, out, ws, main=None, side=None):
    _call("echo_decode_select", C.byref(args), C.byref(pool), C.byref(out), ptr(ws),
          ws.numel() * ws.element_size(), stream_handle(main),
          stream_handle(side) if side is not None else stream_handle(main))


def append_workspace_bytes(n_rows, n_gpu):
    return lib().echo_append_workspace_bytes(n_rows, n_gpu)


def decode_append(args, pool, new_slot, ws, stream=None):
    _call("echo_decode_append", C.byref(args), C.byref(pool), ptr(new_slot), ptr(ws),
          ws.numel() * ws.element_size(), stream_handle(stream))


def step_advance(step_dev, stream=None):
    _call("echo_step_advance", ptr(step_dev), stream_handle(stream))


class CapturedGraph:
    """Whatever echo_* calls `enqueue(stream)` makes, captured into one graph
    (echo_graph_begin / echo_graph_end); replay with launch()."""

    def __init__(self, enqueue, stream):
        self._h = P()
        _call("echo_graph_begin", stream_handle(stream))
        try:
            enqueue(stream)
        except Exception:
            lib().echo_graph_end(stream_handle(stream), C.byref(P()))
            raise
        _call("echo_graph_end", stream_handle(stream), C.byref(self._h))

    def launch(self, stream=None):
        _call("echo_graph_launch", self._h, stream_handle(stream))

    def close(self):
        if self._h:
            _call("echo_graph_destroy", self._h)
            self._h = P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Graph:
    """A captured decode step (echo_graph_capture_decode); replay with launch()."""

    def __init__(self, args, pool, out, ws, main=None, side=None):
        self._h = P()
        self._keep = (args, pool, out, ws)
        _call("echo_graph_capture_decode", C.byref(args), C.byref(pool), C.byref(out),
              ptr(ws), ws.numel() * ws.element_size(), stream_handle(main),
              stream_handle(side) if side is not None else stream_handle(main),
              C.byref(self._h))

    def launch(self, stream=None):
        _call("echo_graph_launch", self._h, stream_handle(stream))

    def close(self):
        if self._h:
            _call("echo_graph_destroy", self._h)
            self._h = P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class HostBuffer:
    """Pinned, device-mapped host memory (echo_host_alloc) viewed as a numpy array."""

    def __init__(self, nbytes, coherent=False):
        import numpy as np
        self.host = P()
        self.dev = P()
        _call("echo_host_alloc", nbytes, 1 if coherent else 0, C.byref(self.host),
              C.byref(self.dev))
        self.nbytes = nbytes
        buf = (C.c_uint8 * nbytes).from_address(self.host.value)
        self.array = np.frombuffer(buf, dtype=np.uint8)

    @property
    def dev_ptr(self):
        return self.dev.value

    def close(self):
        if self.host:
            self.array = None
            _call("echo_host_free", self.host)
            self.host = P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
