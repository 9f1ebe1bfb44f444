// The whole decode step (ECHO review page §4): indexer scores -> exact top-k -> residency
// lookup / eviction / allocation (§5.2) -> recall gather -> priorities, with optional
// threshold prefetch (§6.1).  Every call only enqueues work, so the step can be captured into
// one hipGraph (§2: graph execution forbids host control and dynamically sized tensors inside
// the step).
//
// One stream.  Kernel boundaries on one queue cost next to nothing, while dependencies between
// queues inside a graph cost microseconds each, so work that can overlap the critical path
// rides along in the same launches as extra workgroups instead of on a second stream:
//
//   zero -> score (+ top-k histogram) -> top-k split + early lookup of the sure selections
//        (+ pool statistics) -> top-k finish + lookup of the rest (+ staging of the split's misses
//        from host memory)
//        -> evict-1 (+ staging of the finish's misses) -> evict-2 + allocate -> recall scatter
//
// With ranged prefetch, scoring is split into n_chunks token ranges: the launch of range c also
// gathers range c-1's candidates, and a gather launch for the last range precedes the split.
// With fused prefetch (§6.3), one launch scores and gathers: every workgroup has a wave that
// moves its range's over-threshold rows from host memory while the other waves score; the
// pool statistics then run ahead of it, with the free-slot list.
// With the EMA threshold (§6.1) a last small launch takes each request's k-th score and updates
// the caller's estimate for the next step.
#include <algorithm>
#include <new>

#include "internal.hpp"

namespace echo {

static size_t al(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

struct DecodeWs {
  uint32_t *hist0;     // [n_rows][2048] digit-0 histograms of the top-k keys   (zeroed)
  int32_t *cand_cnt;   // [n_chunks][n_rows]                                     (zeroed)
  int32_t *total_cnt;  // [n_rows]                                               (zeroed)
  PoolFastWs pool;     // starts with its zeroed region
  int64_t zero_words;  // hist0 .. end of the pool's zeroed region
  void *split;
  float *theta;        // [n_rows]
  int32_t *cand;       // [n_chunks][n_rows][cap]
  int32_t *free_list;  // [n_gpu]
  int32_t *free_count; // [2]
  uint16_t *stage;     // [n_rows * topk][ROW] recalled rows before they go to their slots
  FusedWs fz;          // fused prefetch
};

static size_t decode_ws_layout(const echo_decode_args *a, int32_t n_gpu, void *base, DecodeWs *w) {
  const bool pf = a->prefetch == ECHO_PREFETCH_RANGED, fz = a->prefetch == ECHO_PREFETCH_FUSED;
  const size_t nr = static_cast<size_t>(a->n_rows), nc = pf ? static_cast<size_t>(a->n_chunks) : 0;
  size_t off = 0;
  auto take = [&](size_t b) { size_t o = off; off += al(b); return o; };
  const size_t o_h = take(nr * 2048 * 4), o_cc = take(nc * nr * 4), o_tc = take(nr * 4);
  PoolFastWs pw;
  size_t pbytes;
  pool_fast_ws_layout(a->n_rows, a->topk, n_gpu, nullptr, &pw, &pbytes);
  const size_t o_pool = take(pbytes);
  const size_t zero_end = o_pool + static_cast<size_t>(pw.zero_words) * 4;
  const size_t o_split = take(topk_split_ws_bytes(a->n_rows, a->max_key_len, a->topk));
  const size_t o_st = take(nr * static_cast<size_t>(a->topk) * ROW * 2);
  size_t o_th = 0, o_c = 0, o_fl = 0, o_fc = 0, o_fz = 0;
  if (pf || fz) o_th = take(nr * 4);
  if (fz) o_fz = take(fused_ws_layout(a->n_rows, n_gpu, nullptr, nullptr));
  if (pf) {
    o_c = take(nc * nr * static_cast<size_t>(a->cap) * 4);
    o_fl = take(static_cast<size_t>(n_gpu) * 4);
    o_fc = take(2 * 4);
  }
  if (w && base) {
    char *b = static_cast<char *>(base);
    w->hist0 = reinterpret_cast<uint32_t *>(b + o_h);
    w->cand_cnt = reinterpret_cast<int32_t *>(b + o_cc);
    w->total_cnt = reinterpret_cast<int32_t *>(b + o_tc);
    pool_fast_ws_layout(a->n_rows, a->topk, n_gpu, b + o_pool, &w->pool, &pbytes);
    w->zero_words = static_cast<int64_t>(zero_end / 4);
    w->split = b + o_split;
    w->stage = reinterpret_cast<uint16_t *>(b + o_st);
    w->theta = reinterpret_cast<float *>(b + o_th);
    w->cand = reinterpret_cast<int32_t *>(b + o_c);
    w->free_list = reinterpret_cast<int32_t *>(b + o_fl);
    w->free_count = reinterpret_cast<int32_t *>(b + o_fc);
    if (fz) fused_ws_layout(a->n_rows, n_gpu, b + o_fz, &w->fz);
  }
  return off;
}

static int validate(const echo_decode_args *a, const echo_pool *pool, const echo_decode_out *o) {
  if (!a || !pool || !o) return fail(ECHO_EINVAL, "echo_decode_select: NULL argument");
  if (a->n_rows < 1 || a->n_rows > 65535) return fail(ECHO_EUNSUPPORTED, "echo_decode_select: n_rows %d outside [1, 65535]", a->n_rows);
  if (a->max_key_len < 0) return fail(ECHO_EINVAL, "echo_decode_select: max_key_len < 0");
  if (a->max_key_len > (1 << 22)) return fail(ECHO_EUNSUPPORTED, "echo_decode_select: max_key_len above 4M");
  if (a->topk < 1 || a->topk > ECHO_MAX_TOPK) return fail(ECHO_EUNSUPPORTED, "echo_decode_select: topk %d outside [1, %d]", a->topk, ECHO_MAX_TOPK);
  if (static_cast<int64_t>(a->n_rows) * a->topk > (1LL << 30)) return fail(ECHO_EUNSUPPORTED, "echo_decode_select: too many selections");
  if (!a->q || !a->w || !a->key_begin || !a->key_len || !a->req_to_host || (a->max_key_len > 0 && !a->k))
    return fail(ECHO_EINVAL, "echo_decode_select: NULL input");
  if (!o->scores || !o->topk_idx || !o->topk_slot || !o->miss_host || !o->miss_slot || !o->counters)
    return fail(ECHO_EINVAL, "echo_decode_select: NULL output");
  if (pool->n_gpu < 1 || pool->n_host < 1 || !pool->gpu_free || !pool->gpu_priority || !pool->gpu_to_host ||
      !pool->host_to_gpu || !pool->indices_buf || !pool->gpu_kv || !pool->host_kv || !pool->status)
    return fail(ECHO_EINVAL, "echo_decode_select: incomplete pool");
  if (pool->n_gpu > (1 << 22)) return fail(ECHO_EUNSUPPORTED, "echo_decode_select: more than 4M GPU slots");
  if (a->prefetch < ECHO_PREFETCH_OFF || a->prefetch > ECHO_PREFETCH_FUSED)
    return fail(ECHO_EUNSUPPORTED, "echo_decode_select: prefetch mode %d", a->prefetch);
  if (a->prefetch == ECHO_PREFETCH_RANGED && (a->n_chunks < 1 || a->n_chunks > 16))
    return fail(ECHO_EUNSUPPORTED, "echo_decode_select: n_chunks %d outside [1, 16]", a->n_chunks);
  if (a->prefetch == ECHO_PREFETCH_FUSED && a->pf_range != 0 &&
      (a->pf_range % 128 != 0 || a->pf_range < 128 || a->pf_range > ECHO_FUSED_MAX_RANGE))
    return fail(ECHO_EUNSUPPORTED, "echo_decode_select: pf_range %d is not 0 or a multiple of 128 in [128, %d]",
                a->pf_range, ECHO_FUSED_MAX_RANGE);
  if (a->prefetch) {
    if (a->n_sample < 64 || a->n_sample > 4096 || (a->n_sample & (a->n_sample - 1)))
      return fail(ECHO_EUNSUPPORTED, "echo_decode_select: n_sample must be a power of two in [64, 4096]");
    if (!(a->percentile > 0.f && a->percentile <= 100.f)) return fail(ECHO_EINVAL, "echo_decode_select: percentile outside (0, 100]");
    if (a->cap < 1 || a->cap_div < 1) return fail(ECHO_EINVAL, "echo_decode_select: cap and cap_div must be >= 1");
  }
  if (a->theta_ema && !(a->ema_alpha >= 0.f && a->ema_alpha <= 1.f))
    return fail(ECHO_EINVAL, "echo_decode_select: ema_alpha outside [0, 1]");
  if (a->reserve_free < 0 || a->reserve_free > pool->n_gpu)
    return fail(ECHO_EINVAL, "echo_decode_select: reserve_free outside [0, n_gpu]");
  if (a->k_page_table) {
    KeyPages kp;
    int rc = key_pages_of(a->k_page_table, a->k_page_size, a->k_max_pages, a->max_key_len,
                          "echo_decode_select", &kp);
    if (rc) return rc;
    if (a->prefetch == ECHO_PREFETCH_FUSED)
      return fail(ECHO_EUNSUPPORTED, "echo_decode_select: the fused prefetch reads a contiguous key cache only");
  }
  return ECHO_OK;
}

static int decode_select_impl(const echo_decode_args *a, const echo_pool *pool,
                              const echo_decode_out *o, void *ws, size_t ws_bytes, hipStream_t m) {
  int rc = validate(a, pool, o);
  if (rc) return rc;
  DecodeWs W{};
  const size_t need = decode_ws_layout(a, pool->n_gpu, ws, &W);
  if (!ws || ws_bytes < need) return fail(ECHO_EWORKSPACE, "echo_decode_select: workspace %zu < %zu", ws_bytes, need);
  W.pool.reserve = static_cast<uint32_t>(a->reserve_free);
  const int32_t n_ent = a->n_rows * a->topk;
  const bool pf = a->prefetch == ECHO_PREFETCH_RANGED, fz = a->prefetch == ECHO_PREFETCH_FUSED;
  const int nc = pf ? a->n_chunks : 1;

  if ((rc = launch_zero2_i32(o->counters, 8, reinterpret_cast<int32_t *>(W.hist0), W.zero_words, m))) return rc;
  const Stamp stamp{a->step_id, a->step_dev};
  KeyPages pages{nullptr, 0, 0};
  if (a->k_page_table &&
      (rc = key_pages_of(a->k_page_table, a->k_page_size, a->k_max_pages, a->max_key_len,
                         "echo_decode_select", &pages)))
    return rc;
  const KeyPages *kp = a->k_page_table ? &pages : nullptr;
  SideWork side{};
  side.P = PoolArgs{pool->gpu_free, pool->gpu_priority, pool->gpu_to_host, pool->host_to_gpu,
                    pool->indices_buf, pool->status, pool->n_gpu, pool->n_host};
  side.W = W.pool;
  side.stamp = stamp;
  // the pool statistics ride in the top-k split launch (fused prefetch: ahead of its kernel)
  SideWork stats_side = side;
  stats_side.n_stats = fz ? 0 : W.pool.n_chunks;
  side.n_stats = 0;
  // prefetch threshold: the caller's EMA estimate (§6.1), or a sample percentile of this
  // step's scores when there is no history
  const float *theta = a->theta_ema ? a->theta_ema : W.theta;
  if ((pf || fz) && !a->theta_ema &&
      (rc = launch_prefetch_threshold(a->q, a->w, a->k, a->k_scale, a->key_begin, a->key_len,
                                      a->n_rows, a->max_key_len, a->n_sample, a->percentile,
                                      W.theta, kp, m)))
    return rc;
  if (fz) {
    const int32_t range = fused_range(static_cast<int64_t>(a->n_rows) * a->max_key_len, a->max_key_len,
                                      a->pf_range);
    if ((rc = launch_fused_prefetch(a->q, a->w, a->k, a->k_scale, a->key_begin, a->key_len, a->n_rows,
                                    a->max_key_len, o->scores, a->max_key_len, theta, a->req_to_host,
                                    pool, a->cap, a->cap_div, range, W.fz, W.hist0, &W.pool, stamp,
                                    o->counters + 1, o->counters + 2, m)))
      return rc;
  } else if (pf) {
    if ((rc = launch_prefetch_begin(pool, W.free_list, W.free_count, m))) return rc;
    const int32_t span = (a->max_key_len + nc - 1) / nc;
    for (int c = 0; c < nc; ++c) {
      if (c > 0) {                                   // gather range c-1's candidates
        side.n_gather = a->n_rows;
        // no statistics to keep current: they are taken after the gathers, in the split
        side.G = make_gather_args(pool, a->key_begin, a->req_to_host,
                                  W.cand + static_cast<int64_t>(c - 1) * a->n_rows * a->cap,
                                  W.cand_cnt + static_cast<int64_t>(c - 1) * a->n_rows, a->cap,
                                  W.free_list, W.free_count, o->counters + 2, nullptr, stamp);
      }
      const int32_t lo = c * span, hi = (c + 1 == nc) ? a->max_key_len : (c + 1) * span;
      PrefetchArgs P{theta, a->req_to_host, pool->host_to_gpu,
                     W.cand + static_cast<int64_t>(c) * a->n_rows * a->cap,
                     W.cand_cnt + static_cast<int64_t>(c) * a->n_rows, W.total_cnt, a->cap, a->cap_div,
                     pool->n_host, c, nc, W.cand_cnt, a->n_rows};
      if ((rc = launch_score_decode(a->q, a->w, a->k, a->k_scale, a->key_begin, a->key_len, a->n_rows,
                                    a->max_key_len, lo, hi, o->scores, a->max_key_len, &P, W.hist0,
                                    &side, kp, m)))
        return rc;
    }
    // the last range's gather must finish before the top-k split looks selections up
    const int64_t last = static_cast<int64_t>(nc - 1) * a->n_rows;
    if ((rc = launch_prefetch_gather(pool, a->key_begin, a->req_to_host, W.cand + last * a->cap,
                                     W.cand_cnt + last, a->n_rows, a->cap, W.free_list, W.free_count,
                                     o->counters + 2, nullptr, stamp, m)))
      return rc;
  } else {
    if ((rc = launch_score_decode(a->q, a->w, a->k, a->k_scale, a->key_begin, a->key_len, a->n_rows,
                                  a->max_key_len, 0, a->max_key_len, o->scores, a->max_key_len,
                                  nullptr, W.hist0, nullptr, kp, m)))
      return rc;
  }
  if ((rc = launch_topk_split(o->scores, a->max_key_len, a->key_len, a->n_rows, a->max_key_len,
                              a->topk, W.hist0, W.split, pool, &W.pool, a->key_begin, a->req_to_host,
                              stamp, &stats_side, m)))
    return rc;
  if ((rc = launch_topk_finish(o->scores, a->max_key_len, a->key_len, a->n_rows, a->max_key_len,
                               a->topk, W.hist0, W.split, o->topk_idx, pool, &W.pool, a->key_begin,
                               a->req_to_host, stamp, o->topk_slot, true, W.stage, m)))
    return rc;
  if ((rc = launch_pool_evict(pool, W.pool, o->topk_idx, a->n_rows, a->topk, stamp, o->topk_slot,
                              o->miss_host, o->miss_slot, o->counters + 0, W.stage, m)))
    return rc;
  if ((rc = launch_recall_scatter(pool, W.pool, o->miss_host, o->miss_slot, o->counters + 0, n_ent,
                                  W.stage, m)))
    return rc;
  if (pf && (rc = launch_sum_i32(W.total_cnt, a->n_rows, o->counters + 1, m))) return rc;
  return launch_kth_ema(o->scores, a->max_key_len, o->topk_idx, a->n_rows, a->topk, a->ema_alpha,
                        a->theta_ema, o->kth, m);
}

struct GraphHandle {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

}  // namespace echo

using namespace echo;

struct echo_graph_s : GraphHandle {};

extern "C" size_t echo_decode_workspace_bytes(const echo_decode_args *a, int32_t n_gpu) {
  if (!a || n_gpu < 0 || a->n_rows < 0 || a->topk < 0 || a->max_key_len < 0) return 0;
  if (a->prefetch == ECHO_PREFETCH_RANGED && (a->n_chunks < 1 || a->cap < 0)) return 0;
  return decode_ws_layout(a, n_gpu, nullptr, nullptr);
}

extern "C" int echo_decode_select(const echo_decode_args *a, const echo_pool *pool,
                                  const echo_decode_out *out, void *ws, size_t ws_bytes,
                                  void *main_stream, void *side_stream) {
  (void)side_stream;                       // reserved: the step runs on main_stream
  return decode_select_impl(a, pool, out, ws, ws_bytes, S(main_stream));
}

extern "C" int echo_graph_capture_decode(const echo_decode_args *a, const echo_pool *pool,
                                         const echo_decode_out *out, void *ws, size_t ws_bytes,
                                         void *main_stream, void *side_stream, echo_graph *graph) {
  if (!graph) return fail(ECHO_EINVAL, "echo_graph_capture_decode: NULL graph");
  *graph = nullptr;
  if (!main_stream) return fail(ECHO_EINVAL, "echo_graph_capture_decode: capture needs a non-null main stream");
  (void)side_stream;                       // reserved: the step runs on main_stream
  int rc = validate(a, pool, out);
  if (rc) return rc;
  hipStream_t m = S(main_stream);
  hipError_t e = hipStreamBeginCapture(m, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return fail(ECHO_EHIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
  rc = decode_select_impl(a, pool, out, ws, ws_bytes, m);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(m, &g);
  if (rc) {
    if (g) (void)hipGraphDestroy(g);
    return rc;
  }
  if (e != hipSuccess) return fail(ECHO_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return fail(ECHO_EHIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  }
  echo_graph_s *h = new (std::nothrow) echo_graph_s;
  if (!h) {
    (void)hipGraphExecDestroy(ex);
    (void)hipGraphDestroy(g);
    return fail(ECHO_EHIP, "echo_graph_capture_decode: out of host memory");
  }
  h->graph = g;
  h->exec = ex;
  *graph = h;
  return ECHO_OK;
}

extern "C" int echo_graph_begin(void *stream) {
  if (!stream) return fail(ECHO_EINVAL, "echo_graph_begin: capture needs a non-null stream");
  hipError_t e = hipStreamBeginCapture(S(stream), hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return fail(ECHO_EHIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
  return ECHO_OK;
}

extern "C" int echo_graph_end(void *stream, echo_graph *graph) {
  if (graph) *graph = nullptr;
  if (!stream) return fail(ECHO_EINVAL, "echo_graph_end: NULL stream");
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(S(stream), &g);
  if (e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return fail(ECHO_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  }
  if (!graph) {
    (void)hipGraphDestroy(g);
    return fail(ECHO_EINVAL, "echo_graph_end: NULL graph");
  }
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return fail(ECHO_EHIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  }
  echo_graph_s *h = new (std::nothrow) echo_graph_s;
  if (!h) {
    (void)hipGraphExecDestroy(ex);
    (void)hipGraphDestroy(g);
    return fail(ECHO_EHIP, "echo_graph_end: out of host memory");
  }
  h->graph = g;
  h->exec = ex;
  *graph = h;
  return ECHO_OK;
}

extern "C" int echo_graph_launch(echo_graph graph, void *stream) {
  if (!graph) return fail(ECHO_EINVAL, "echo_graph_launch: NULL graph");
  hipError_t e = hipGraphLaunch(graph->exec, S(stream));
  if (e != hipSuccess) return fail(ECHO_EHIP, "hipGraphLaunch: %s", hipGetErrorString(e));
  return ECHO_OK;
}

extern "C" int echo_graph_destroy(echo_graph graph) {
  if (!graph) return ECHO_OK;
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipGraphDestroy(graph->graph);
  delete graph;
  return ECHO_OK;
}
