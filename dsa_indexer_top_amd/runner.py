"""Device-buffer plumbing for one decode step: holds the inputs, the pool (with a pristine
copy to restore between timed replays), the outputs and the workspace, and calls the C ABI
(eagerly or through a captured hipGraph).  No arithmetic of the method lives here.
"""

import numpy as np

from . import binding as B

DEFAULT_PREFETCH = dict(n_chunks=4, n_sample=4096, percentile=95.0, cap=2048, cap_div=1024,
                        range=0)


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class DecodeRunner:
    """inp: inputs.DecodeInputs; pool: inputs.PoolArrays; host_kv: uint16 [N_H, 576] numpy
    array, or a binding.HostBuffer already holding it (pass host_buf=...).  prefetch: False,
    True / "ranged" or "fused"; theta (optional, float32 [B]): a given per-request threshold
    in place of the sample percentile (the step's EMA estimate; restored by restore()).
    pages (optional, inputs.PagedKeys of inp's keys): the step reads a paged key cache."""

    def __init__(self, inp, pool, host_kv=None, host_buf=None, prefetch=False, pf=None,
                 topk=None, step_id=None, reserve=0, theta=None, alpha=0.5, pages=None):
        import torch
        self.torch = torch
        cfg = inp.cfg
        self.inp = inp
        self.n_rows = len(inp.key_len)
        self.max_len = int(inp.key_len.max())
        self.topk = cfg.topk if topk is None else topk
        self.step_id = pool.step_id if step_id is None else step_id
        self.q, self.w = _dev(inp.q), _dev(inp.w)
        self.page_table = None
        if pages is None:
            self.k = _dev(inp.k)
            self.k_scale = None if inp.k_scale is None else _dev(inp.k_scale)
        else:
            self.k = _dev(pages.k_pages)
            self.k_scale = None if pages.k_scale_pages is None else _dev(pages.k_scale_pages)
            self.page_table = _dev(pages.page_table)
        self.key_begin, self.key_len = _dev(inp.key_begin), _dev(inp.key_len)
        self.req_to_host = _dev(inp.req_to_host)
        # pool + pristine copy
        names = ("free", "priority", "to_host", "host_to_gpu", "indices_buf", "gpu_kv")
        self.pristine = {n: _dev(getattr(pool, n)) for n in names}
        self.live = {n: t.clone() for n, t in self.pristine.items()}
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        if host_buf is None:
            host_buf = B.HostBuffer(host_kv.nbytes)
            host_buf.array.view(np.uint16).reshape(host_kv.shape)[...] = host_kv
            self._own_buf = True
        else:
            self._own_buf = False
        self.host_buf = host_buf
        self.n_gpu, self.n_host = len(pool.free), len(pool.host_to_gpu)
        L = self.live
        self.pool = B.make_pool(self.n_gpu, self.n_host, L["free"], L["priority"], L["to_host"],
                                L["host_to_gpu"], L["indices_buf"], L["gpu_kv"],
                                host_buf.dev_ptr, self.status)
        # outputs
        i32 = torch.int32
        self.scores = torch.empty((self.n_rows, max(self.max_len, 1)), dtype=torch.float32, device="cuda")
        self.topk_idx = torch.empty((self.n_rows, self.topk), dtype=i32, device="cuda")
        self.topk_slot = torch.empty((self.n_rows, self.topk), dtype=i32, device="cuda")
        self.miss_host = torch.empty(self.n_rows * self.topk, dtype=i32, device="cuda")
        self.miss_slot = torch.empty(self.n_rows * self.topk, dtype=i32, device="cuda")
        self.counters = torch.zeros(8, dtype=i32, device="cuda")
        self.out = B.DecodeOut(self.scores.data_ptr(), self.topk_idx.data_ptr(),
                               self.topk_slot.data_ptr(), self.miss_host.data_ptr(),
                               self.miss_slot.data_ptr(), self.counters.data_ptr())
        p = dict(DEFAULT_PREFETCH)
        p.update(pf or {})
        self.args = B.DecodeArgs(
            self.q.data_ptr(), self.w.data_ptr(), self.k.data_ptr(),
            None if self.k_scale is None else self.k_scale.data_ptr(),
            self.key_begin.data_ptr(), self.key_len.data_ptr(), self.req_to_host.data_ptr(),
            self.n_rows, self.max_len, self.topk, self.step_id, B.prefetch_mode(prefetch),
            p["n_chunks"], p["n_sample"], p["percentile"], p["cap"], p["cap_div"])
        self.args.reserve_free = reserve
        self.args.pf_range = p["range"]
        if pages is not None:
            self.args.k_page_table = self.page_table.data_ptr()
            self.args.k_page_size = pages.page_size
            self.args.k_max_pages = self.page_table.shape[1]
        self.theta0 = self.theta = None
        if theta is not None:
            self.theta0 = _dev(np.asarray(theta, np.float32))
            self.theta = self.theta0.clone()
            self.args.theta_ema = self.theta.data_ptr()
            self.args.ema_alpha = alpha
        nbytes = B.decode_workspace_bytes(self.args, self.n_gpu)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        self.main = torch.cuda.Stream()
        self.side = torch.cuda.Stream()      # prefetch gathers overlap scoring
        self.graph = None

    def restore(self):
        """Put the pool back to its state before the step (outside any timed region)."""
        with self.torch.cuda.stream(self.main):
            for n, t in self.pristine.items():
                self.live[n].copy_(t)
            self.status.zero_()
            if self.theta is not None:
                self.theta.copy_(self.theta0)

    def run_eager(self):
        B.decode_select(self.args, self.pool, self.out, self.ws, self.main, self.side)

    def capture(self):
        self.torch.cuda.synchronize()
        self.graph = B.Graph(self.args, self.pool, self.out, self.ws, self.main, self.side)
        return self.graph

    def replay(self):
        self.graph.launch(self.main)

    def sync(self):
        self.torch.cuda.synchronize()

    def results(self):
        self.sync()
        h = lambda t: t.cpu().numpy()
        return dict(scores=h(self.scores), topk_idx=h(self.topk_idx), topk_slot=h(self.topk_slot),
                    miss_host=h(self.miss_host), miss_slot=h(self.miss_slot),
                    counters=h(self.counters), status=int(h(self.status)[0]),
                    pool={n: h(t) for n, t in self.live.items()})

    def close(self):
        if self.graph is not None:
            self.graph.close()
            self.graph = None
        if self._own_buf:
            self.host_buf.close()


class LoopRunner:
    """Device buffers of several decode steps in a row (inputs.MultiStepInputs): the K cache with
    room for the new tokens, the pool, the pinned host backup (the appends write through to it),
    one step's inputs and the EMA estimate of the k-th score.  run_step(st) uploads step st's
    query and new tokens, then enqueues echo_decode_append and echo_decode_select.  With
    device_step=True the step stamp lives on the device; capture() then records
    echo_step_advance + echo_decode_append + echo_decode_select as one graph, and
    replay_step(st) uploads step st's inputs and replays it.  No arithmetic of the method lives
    here."""

    def __init__(self, m, host_kv, topk, prefetch=False, pf=None, alpha=0.5, ema=True,
                 device_step=False, reserve=0):
        import torch
        self.torch = torch
        self.m = m
        B_, cap = len(m.key_len), m.capacity
        self.n_rows, self.cap, self.topk = B_, cap, topk
        self.k = _dev(m.k)
        self.k_scale = None if m.k_scale is None else _dev(m.k_scale)
        self.key_begin, self.key_len = _dev(m.key_begin), _dev(m.key_len)
        self.req_to_host = _dev(m.req_to_host)
        names = ("free", "priority", "to_host", "host_to_gpu", "indices_buf", "gpu_kv")
        self.live = {n: _dev(getattr(m.pool, n)) for n in names}
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.host_buf = B.HostBuffer(host_kv.nbytes)
        self.host_kv = self.host_buf.array.view(np.uint16).reshape(host_kv.shape)
        self.host_kv[...] = host_kv
        self.n_gpu, self.n_host = len(m.pool.free), len(m.pool.host_to_gpu)
        L = self.live
        self.pool = B.make_pool(self.n_gpu, self.n_host, L["free"], L["priority"], L["to_host"],
                                L["host_to_gpu"], L["indices_buf"], L["gpu_kv"],
                                self.host_buf.dev_ptr, self.status)
        i32, f32 = torch.int32, torch.float32
        dev = "cuda"
        # one step's inputs
        self.q = torch.empty((B_, 64, 128), dtype=torch.uint8, device=dev)
        self.w = torch.empty((B_, 64), dtype=f32, device=dev)
        self.new_k = torch.empty((B_, 128), dtype=torch.uint8, device=dev)
        self.new_scale = None if m.k_scale is None else torch.empty(B_, dtype=f32, device=dev)
        self.new_kv = torch.empty((B_, 576), dtype=torch.int16, device=dev)
        self.new_host = torch.empty(B_, dtype=i32, device=dev)
        # outputs
        self.scores = torch.empty((B_, cap), dtype=f32, device=dev)
        self.topk_idx = torch.empty((B_, topk), dtype=i32, device=dev)
        self.topk_slot = torch.empty((B_, topk), dtype=i32, device=dev)
        self.miss_host = torch.empty(B_ * topk, dtype=i32, device=dev)
        self.miss_slot = torch.empty(B_ * topk, dtype=i32, device=dev)
        self.counters = torch.zeros(8, dtype=i32, device=dev)
        self.kth = torch.empty(B_, dtype=f32, device=dev)
        self.new_slot = torch.empty(B_, dtype=i32, device=dev)
        self.theta = torch.full((B_,), float("nan"), dtype=f32, device=dev)
        self.out = B.DecodeOut(self.scores.data_ptr(), self.topk_idx.data_ptr(),
                               self.topk_slot.data_ptr(), self.miss_host.data_ptr(),
                               self.miss_slot.data_ptr(), self.counters.data_ptr(),
                               self.kth.data_ptr())
        p = dict(DEFAULT_PREFETCH)
        p.update(pf or {})
        self.args = B.DecodeArgs(
            self.q.data_ptr(), self.w.data_ptr(), self.k.data_ptr(),
            None if self.k_scale is None else self.k_scale.data_ptr(),
            self.key_begin.data_ptr(), self.key_len.data_ptr(), self.req_to_host.data_ptr(),
            B_, cap, topk, 0, B.prefetch_mode(prefetch), p["n_chunks"], p["n_sample"],
            p["percentile"], p["cap"], p["cap_div"],
            self.theta.data_ptr() if ema else None, alpha)
        self.args.reserve_free = reserve
        self.args.pf_range = p["range"]
        self.app = B.AppendArgs(
            B_, cap, self.k.shape[0], self.new_k.data_ptr(),
            None if self.new_scale is None else self.new_scale.data_ptr(),
            self.new_kv.data_ptr(), self.new_host.data_ptr(), self.k.data_ptr(),
            None if self.k_scale is None else self.k_scale.data_ptr(),
            self.key_begin.data_ptr(), self.key_len.data_ptr(), self.req_to_host.data_ptr(),
            self.host_buf.dev_ptr, 0)
        self.ws = torch.empty(max(B.decode_workspace_bytes(self.args, self.n_gpu), 256),
                              dtype=torch.uint8, device=dev)
        self.ws_app = torch.empty(max(B.append_workspace_bytes(B_, self.n_gpu), 256),
                                  dtype=torch.uint8, device=dev)
        self.main = torch.cuda.Stream()
        self.step_dev = None
        self.graph = None
        if device_step:
            # advanced to the first step's stamp by the first replay
            first = int(m.steps[0]["step_id"]) if m.steps else int(m.pool.step_id)
            self.step_dev = torch.full((1,), first - 1, dtype=i32, device=dev)
            self.args.step_dev = self.app.step_dev = self.step_dev.data_ptr()

    def _enqueue_step(self, stream):
        if self.step_dev is not None:
            B.step_advance(self.step_dev, stream)
        B.decode_append(self.app, self.pool, self.new_slot, self.ws_app, stream)
        B.decode_select(self.args, self.pool, self.out, self.ws, stream)

    def capture(self):
        assert self.step_dev is not None, "a replayable step needs the stamp on the device"
        self.torch.cuda.synchronize()
        self.graph = B.CapturedGraph(self._enqueue_step, self.main)
        return self.graph

    def replay_step(self, st):
        self.load_step(st)
        self.graph.launch(self.main)

    def load_step(self, st):
        t = self.torch
        with t.cuda.stream(self.main):
            self.q.copy_(t.from_numpy(np.ascontiguousarray(st["q"])))
            self.w.copy_(t.from_numpy(np.ascontiguousarray(st["w"])))
            self.new_k.copy_(t.from_numpy(np.ascontiguousarray(st["new_k"])))
            if self.new_scale is not None:
                self.new_scale.copy_(t.from_numpy(np.ascontiguousarray(st["new_scale"])))
            self.new_kv.copy_(t.from_numpy(np.ascontiguousarray(st["new_kv"]).view(np.int16)))
            self.new_host.copy_(t.from_numpy(np.ascontiguousarray(st["new_host"], np.int32)))

    def run_step(self, st):
        self.load_step(st)
        self.app.step_id = self.args.step_id = int(st["step_id"])
        self._enqueue_step(self.main)

    def results(self):
        self.torch.cuda.synchronize()
        h = lambda t: t.cpu().numpy()
        return dict(scores=h(self.scores), topk_idx=h(self.topk_idx), topk_slot=h(self.topk_slot),
                    miss_host=h(self.miss_host), miss_slot=h(self.miss_slot),
                    counters=h(self.counters), kth=h(self.kth), theta=h(self.theta),
                    new_slot=h(self.new_slot), status=int(h(self.status)[0]),
                    key_len=h(self.key_len), k=h(self.k), req_to_host=h(self.req_to_host),
                    k_scale=None if self.k_scale is None else h(self.k_scale),
                    pool={n: h(t) for n, t in self.live.items()},
                    host_kv=self.host_kv.copy())

    def close(self):
        if self.graph is not None:
            self.graph.close()
            self.graph = None
        self.host_buf.close()


class PrefillChunkRunner:
    """Device buffers of one request's chunked prefill with its KV offloaded (the inter-query
    prefetch of the ECHO page's §6.2): all query rows, keys and the token -> host map, the pool
    with its pinned host backup, and per-chunk scores, subsets, unions and pool-step outputs.
    run_chunk(c) enqueues, on one stream: the chunk's causal scores; with prefetch, the
    approximate subsets under the current shift, their union and its prefetch gather; the
    exact top-k, its union and the guaranteed residency (lookup / evict / allocate + recall);
    then the shift update from the k-th score of the chunk's last row.  No arithmetic of the
    method lives here."""

    def __init__(self, q, w, k, req_to_host, pool, host_kv, chunk, topk, prefetch=False,
                 alpha=0.5):
        import torch
        self.torch = torch
        n = q.shape[0]
        self.n, self.chunk, self.topk, self.prefetch, self.alpha = n, chunk, topk, prefetch, alpha
        self.q, self.w, self.k = _dev(q), _dev(w), _dev(k)
        self.req_to_host = _dev(req_to_host)
        names = ("free", "priority", "to_host", "host_to_gpu", "indices_buf", "gpu_kv")
        self.live = {nm: _dev(getattr(pool, nm)) for nm in names}
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.host_buf = B.HostBuffer(host_kv.nbytes)
        self.host_buf.array.view(np.uint16).reshape(host_kv.shape)[...] = host_kv
        self.n_gpu, self.n_host = len(pool.free), len(pool.host_to_gpu)
        L = self.live
        self.pool = B.make_pool(self.n_gpu, self.n_host, L["free"], L["priority"], L["to_host"],
                                L["host_to_gpu"], L["indices_buf"], L["gpu_kv"],
                                self.host_buf.dev_ptr, self.status)
        i32, f32, dev = torch.int32, torch.float32, "cuda"
        self.n_seg = max(1, -(-n // 4096))
        self.scores = torch.empty((chunk, n), dtype=f32, device=dev)
        self.lens = torch.empty(chunk, dtype=i32, device=dev)
        self.subset = torch.empty((chunk, topk), dtype=i32, device=dev)
        self.subset_cnt = torch.empty(chunk, dtype=i32, device=dev)
        self.thr_cnt = torch.empty(chunk, dtype=i32, device=dev)
        self.idx = torch.empty((chunk, topk), dtype=i32, device=dev)
        self.pre = torch.empty((self.n_seg, 4096), dtype=i32, device=dev)
        self.pre_cnt = torch.empty(self.n_seg, dtype=i32, device=dev)
        self.uni = torch.empty((self.n_seg, 4096), dtype=i32, device=dev)
        self.uni_cnt = torch.empty(self.n_seg, dtype=i32, device=dev)
        self.seg_begin = torch.zeros(self.n_seg, dtype=torch.int64, device=dev)
        self.slot = torch.empty((self.n_seg, 4096), dtype=i32, device=dev)
        self.miss_host = torch.empty(self.n_seg * 4096, dtype=i32, device=dev)
        self.miss_slot = torch.empty(self.n_seg * 4096, dtype=i32, device=dev)
        self.n_miss = torch.zeros(1, dtype=i32, device=dev)
        self.free_list = torch.empty(self.n_gpu, dtype=i32, device=dev)
        self.free_count = torch.zeros(2, dtype=i32, device=dev)
        self.n_prefetched = torch.zeros(1, dtype=i32, device=dev)
        self.theta = torch.full((1,), float("nan"), dtype=f32, device=dev)
        self.kth = torch.empty(1, dtype=f32, device=dev)
        self.ws_union = torch.empty(max(B.union_workspace_bytes(n), 256), dtype=torch.uint8, device=dev)
        self.ws_topk = torch.empty(max(B.topk_workspace_bytes(chunk, n), 256), dtype=torch.uint8, device=dev)
        self.ws_pool = torch.empty(max(B.pool_workspace_bytes(self.n_seg, 4096, self.n_gpu), 256),
                                   dtype=torch.uint8, device=dev)
        self.main = torch.cuda.Stream()

    def run_chunk(self, c, step_id):
        t = self.torch
        t0 = c * self.chunk
        t1 = min(self.n, t0 + self.chunk)
        rows = t1 - t0
        st = self.main
        with t.cuda.stream(st):
            self.lens[:rows].copy_(t.arange(t0 + 1, t1 + 1, dtype=t.int32))
            self.n_prefetched.zero_()
        sc = self.scores[:rows]
        B.index_scores_prefill(self.q[t0:t1], self.w[t0:t1], self.k[:t1], sc, q_pos0=t0,
                               ld=self.n, stream=st)
        lens = self.lens[:rows]
        if self.prefetch:
            B.topk_subset(sc, lens, t1, self.topk, self.theta, self.subset[:rows],
                          self.subset_cnt[:rows], self.thr_cnt[:rows], ld=self.n, stream=st)
            B.union_rows(self.subset[:rows], t1, self.pre, self.pre_cnt, self.ws_union, stream=st)
            B.prefetch_begin(self.pool, self.free_list, self.free_count, stream=st)
            B.prefetch_gather(self.pool, self.seg_begin, self.req_to_host, self.pre, self.pre_cnt,
                              4096, self.free_list, self.free_count, self.n_prefetched, stream=st)
        B.topk(sc, lens, t1, self.topk, self.idx[:rows], self.ws_topk, ld=self.n, stream=st)
        B.union_rows(self.idx[:rows], t1, self.uni, self.uni_cnt, self.ws_union, stream=st)
        B.pool_lookup_alloc(self.pool, self.uni, self.seg_begin, self.req_to_host, step_id,
                            self.slot, self.miss_host, self.miss_slot, self.n_miss, self.ws_pool,
                            stream=st)
        B.recall(self.pool, self.miss_host, self.miss_slot, self.n_miss, self.n_seg * 4096,
                 stream=st)
        B.threshold_ema(sc[rows - 1:rows], self.idx[rows - 1:rows], self.alpha, self.theta,
                        self.kth, ld=self.n, stream=st)
        return rows

    def results(self, rows):
        self.torch.cuda.synchronize()
        h = lambda x: x.cpu().numpy()
        return dict(scores=h(self.scores[:rows]), subset=h(self.subset[:rows]),
                    subset_cnt=h(self.subset_cnt[:rows]), thr_cnt=h(self.thr_cnt[:rows]),
                    idx=h(self.idx[:rows]), pre=h(self.pre), pre_cnt=h(self.pre_cnt),
                    uni=h(self.uni), uni_cnt=h(self.uni_cnt), slot=h(self.slot),
                    n_miss=int(h(self.n_miss)[0]), n_prefetched=int(h(self.n_prefetched)[0]),
                    theta=float(h(self.theta)[0]), kth=float(h(self.kth)[0]),
                    status=int(h(self.status)[0]),
                    pool={nm: h(x) for nm, x in self.live.items()})

    def close(self):
        self.host_buf.close()
