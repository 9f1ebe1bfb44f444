// Guaranteed residency of the selected tokens in the GPU pool (ECHO review page §5.1
// metadata, §5.2 free / allocate / recall lookup), as fixed-grid kernels with every count on
// the device, so the step can be captured into a hipGraph.
//
// Order of one call (all on one stream):
//   lookup     per selected entry: host index, HostTokenToGPU lookup; hit slots are protected
//              (free byte 2 for the duration of the call); misses counted per workgroup
//   compact    misses listed in (request, token) order by a prefix over workgroup counts
//   evict x5   need = max(0, #miss - #free); the `need` occupied unprotected slots with the
//              smallest (priority, slot) are evicted: three radix-histogram passes over the
//              slots' priorities, a count pass, an apply pass (metadata only, rows untouched);
//              the apply pass also counts the free slots of its chunk afterwards
//   alloc      the i-th miss takes the i-th free slot in ascending order (prefix over chunk
//              free counts): maps, priority = step, indices buffer, per-entry slot
//   finalize   priority = step for every selected slot, protection cleared, duplicate-host
//              check, indices buffer padding
// Data-dependent failures set status bits; every later kernel then leaves the pool alone.
#include <algorithm>

#include "internal.hpp"
#include "select.cuh"

namespace echo {

constexpr int PL_THREADS = 256;

struct PoolWs {
  uint32_t *hist;        // [3][2048]
  uint32_t *chunk_lt;    // [n_chunks]
  uint32_t *chunk_eq;    // [n_chunks]
  uint32_t *chunk_free;  // [n_chunks]
  uint32_t *wg_miss;     // [n_lookup_wg]
  int32_t *ent_host;     // [n_ent] host index of a missed entry, -1 otherwise
  int32_t *miss_entry;   // [n_ent] entry of the i-th miss
  int32_t *counters;     // [8]: 0 n_miss, 1 n_free
  int32_t n_chunks;
  int32_t n_lookup_wg;
};

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

static void pool_ws_layout(int32_t n_rows, int32_t k, int32_t n_gpu, void *base, PoolWs *w,
                           size_t *bytes) {
  const int64_t n_ent = static_cast<int64_t>(n_rows) * k;
  const int32_t n_chunks = std::max(1, (n_gpu + SEL_CHUNK - 1) / SEL_CHUNK);
  const int32_t n_lwg = static_cast<int32_t>(std::max<int64_t>(1, (n_ent + PL_THREADS - 1) / PL_THREADS));
  size_t off = 0;
  auto take = [&](size_t b) { size_t o = off; off += align256(b); return o; };
  const size_t o_hist = take(3 * SEL_BINS * 4), o_lt = take(n_chunks * 4), o_eq = take(n_chunks * 4),
               o_free = take(n_chunks * 4), o_wg = take(n_lwg * 4), o_eh = take(n_ent * 4),
               o_me = take(n_ent * 4), o_cnt = take(8 * 4);
  *bytes = off;
  if (w && base) {
    char *b = static_cast<char *>(base);
    w->hist = reinterpret_cast<uint32_t *>(b + o_hist);
    w->chunk_lt = reinterpret_cast<uint32_t *>(b + o_lt);
    w->chunk_eq = reinterpret_cast<uint32_t *>(b + o_eq);
    w->chunk_free = reinterpret_cast<uint32_t *>(b + o_free);
    w->wg_miss = reinterpret_cast<uint32_t *>(b + o_wg);
    w->ent_host = reinterpret_cast<int32_t *>(b + o_eh);
    w->miss_entry = reinterpret_cast<int32_t *>(b + o_me);
    w->counters = reinterpret_cast<int32_t *>(b + o_cnt);
    w->n_chunks = n_chunks;
    w->n_lookup_wg = n_lwg;
  }
}

size_t pool_ws_bytes(int32_t n_rows, int32_t k, int32_t n_gpu) {
  size_t b;
  pool_ws_layout(n_rows, k, n_gpu, nullptr, nullptr, &b);
  return b;
}

// ------------------------------------------------------------------ lookup + protection
__global__ __launch_bounds__(PL_THREADS) void pool_lookup_kernel(
    PoolArgs P, PoolWs W, const int32_t *__restrict__ idx, const int64_t *__restrict__ key_begin,
    const int32_t *__restrict__ req_to_host, int64_t n_k, int32_t n_rows, int32_t k,
    int32_t *__restrict__ topk_slot) {
  __shared__ uint32_t tmp[48];
  const int64_t n_ent = static_cast<int64_t>(n_rows) * k;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * PL_THREADS + threadIdx.x;
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < SEL_BINS; i += PL_THREADS) W.hist[i] = 0;  // digit-0 histogram
    if (threadIdx.x < 8) W.counters[threadIdx.x] = 0;
  }
  uint32_t miss = 0;
  if (e < n_ent) {
    const int32_t s = idx[e];
    int32_t slot_out = -1, h_miss = -1;
    if (s >= 0) {
      const int64_t tok = key_begin[e / k] + s;
      if (tok < 0 || tok >= n_k) {
        atomicOr(P.status, ECHO_ST_BAD_HOST);
      } else {
        const int32_t h = req_to_host[tok];
        if (h < 0 || h >= P.n_host) {
          atomicOr(P.status, ECHO_ST_BAD_HOST);
        } else {
          const int32_t slot = P.host_to_gpu[h];
          if (slot == INF) {
            miss = 1;
            h_miss = h;
          } else if (slot < 0 || slot >= P.n_gpu) {
            atomicOr(P.status, ECHO_ST_BAD_HOST);
          } else {
            slot_out = slot;
            P.free_[slot] = 2;   // protected for this call
          }
        }
      }
    }
    topk_slot[e] = slot_out;
    W.ent_host[e] = h_miss;
  }
  const uint32_t tot = block_sum<PL_THREADS>(miss, tmp);
  if (threadIdx.x == 0) W.wg_miss[blockIdx.x] = tot;
}

// ------------------------------------------------------------------ ordered miss list
__global__ __launch_bounds__(PL_THREADS) void pool_compact_kernel(
    PoolArgs P, PoolWs W, int32_t n_rows, int32_t k, int32_t *__restrict__ miss_host,
    int32_t *__restrict__ miss_slot, int32_t *__restrict__ n_miss_out) {
  __shared__ uint32_t tmp[48];
  const int64_t n_ent = static_cast<int64_t>(n_rows) * k;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * PL_THREADS + threadIdx.x;
  uint32_t before = 0, total = 0;
  for (int b = threadIdx.x; b < W.n_lookup_wg; b += PL_THREADS) {
    const uint32_t c = W.wg_miss[b];
    total += c;
    if (b < static_cast<int>(blockIdx.x)) before += c;
  }
  before = block_sum<PL_THREADS>(before, tmp);
  total = block_sum<PL_THREADS>(total, tmp);
  const int32_t h = (e < n_ent) ? W.ent_host[e] : -1;
  uint32_t t_all;
  const uint32_t rank = before + block_excl_scan<PL_THREADS>(h >= 0 ? 1u : 0u, tmp, &t_all);
  if (h >= 0) {
    miss_host[rank] = h;
    W.miss_entry[rank] = static_cast<int32_t>(e);
  }
  if (e < n_ent && e >= static_cast<int64_t>(total)) {
    miss_host[e] = -1;
    miss_slot[e] = -1;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    W.counters[0] = static_cast<int32_t>(total);
    *n_miss_out = static_cast<int32_t>(total);
  }
}

// ------------------------------------------------------------------ eviction (radix select)
struct EvictSrc {
  const uint8_t *free_;
  const int32_t *priority;
  int32_t n_gpu;
  ECHO_DEV int32_t n(int) const { return n_gpu; }
  ECHO_DEV bool get(int, int32_t e, uint32_t &key) const {
    if (free_[e] != 0) return false;      // free (1) or protected (2)
    key = i32_key(priority[e]);
    return true;
  }
};

// need = max(0, n_miss - n_free); 0 once any status bit is set.  Returns the number of slots
// to evict, or -1 (after flagging EXHAUSTED from workgroup 0) when too few are evictable.
ECHO_DEV int32_t evict_need(const PoolArgs &P, const PoolWs &W, SelWs &sw, uint32_t *tmp) {
  if (*(volatile int32_t *)P.status) return 0;
  const int32_t need = max(0, W.counters[0] - W.counters[1]);
  uint32_t local = 0;
  for (int b = threadIdx.x; b < SEL_BINS; b += SEL_THREADS) local += sw.h(0, 0)[b];
  const uint32_t evictable = block_sum<SEL_THREADS>(local, tmp);
  if (static_cast<uint32_t>(need) > evictable) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(P.status, ECHO_ST_EXHAUSTED);
    return -1;
  }
  return need;
}

ECHO_DEV SelWs evict_selws(const PoolWs &W) {
  SelWs s;
  s.hist = W.hist;
  s.chunk_lt = W.chunk_lt;
  s.chunk_eq = W.chunk_eq;
  s.n_chunks = W.n_chunks;
  return s;
}

template <int DIG>
__global__ __launch_bounds__(SEL_THREADS) void evict_hist_kernel(PoolArgs P, PoolWs W) {
  __shared__ uint32_t hl[SEL_COPIES * SEL_BINS];
  __shared__ uint32_t tmp[48];
  SelWs sw = evict_selws(W);
  const int chunk = blockIdx.x;
  if (chunk == 0 && DIG < 2) sel_zero_hist(sw, 0, DIG + 1);
  EvictSrc src{P.free_, P.priority, P.n_gpu};
  if (DIG == 0) {
    if (*(volatile int32_t *)P.status) return;
    // free slots of this chunk (before eviction)
    uint32_t nf = 0;
    for (int e = 0; e < SEL_PER_THREAD; ++e) {
      const int32_t i = chunk * SEL_CHUNK + e * SEL_THREADS + threadIdx.x;
      if (i < P.n_gpu) nf += (P.free_[i] == 1);
    }
    nf = block_sum<SEL_THREADS>(nf, tmp);
    if (threadIdx.x == 0 && nf) atomicAdd(&W.counters[1], static_cast<int32_t>(nf));
    sel_hist_chunk(src, sw, 0, chunk, 0, Pick{0u, 0u, 0u, 0, 0}, hl);
    return;
  }
  const int32_t need = evict_need(P, W, sw, tmp);
  if (need <= 0) return;
  const Pick p = sel_pick(sw, 0, DIG, static_cast<uint32_t>(need), tmp);
  if (p.none || p.all) return;
  sel_hist_chunk(src, sw, 0, chunk, DIG, p, hl);
}

__global__ __launch_bounds__(SEL_THREADS) void evict_count_kernel(PoolArgs P, PoolWs W) {
  __shared__ uint32_t tmp[48];
  SelWs sw = evict_selws(W);
  const int32_t need = evict_need(P, W, sw, tmp);
  if (need <= 0) return;
  const Pick p = sel_pick(sw, 0, 3, static_cast<uint32_t>(need), tmp);
  EvictSrc src{P.free_, P.priority, P.n_gpu};
  uint32_t lt = 0, eq = 0;
  for (int e = 0; e < SEL_PER_THREAD; ++e) {
    const int32_t i = blockIdx.x * SEL_CHUNK + e * SEL_THREADS + threadIdx.x;
    if (i < P.n_gpu) {
      const int c = sel_class(src, 0, i, p);
      lt += (c == 1);
      eq += (c == 2);
    }
  }
  lt = block_sum<SEL_THREADS>(lt, tmp);
  eq = block_sum<SEL_THREADS>(eq, tmp);
  if (threadIdx.x == 0) {
    W.chunk_lt[blockIdx.x] = lt;
    W.chunk_eq[blockIdx.x] = eq;
  }
}

__global__ __launch_bounds__(SEL_THREADS) void evict_apply_kernel(PoolArgs P, PoolWs W) {
  __shared__ uint32_t tmp[48];
  __shared__ uint8_t cls_lds[SEL_THREADS * (SEL_PER_THREAD + 1)];
  SelWs sw = evict_selws(W);
  const int chunk = blockIdx.x;
  const int32_t base = chunk * SEL_CHUNK;
  if (*(volatile int32_t *)P.status) return;
  const int32_t need = evict_need(P, W, sw, tmp);
  if (need < 0) return;
  if (need > 0) {
    const Pick p = sel_pick(sw, 0, 3, static_cast<uint32_t>(need), tmp);
    EvictSrc src{P.free_, P.priority, P.n_gpu};
    uint32_t lt_before = 0, eq_before = 0;
    {
      uint32_t lt = 0, eq = 0;
      for (int c = threadIdx.x; c < chunk; c += SEL_THREADS) {
        lt += W.chunk_lt[c];
        eq += W.chunk_eq[c];
      }
      lt_before = block_sum<SEL_THREADS>(lt, tmp);
      eq_before = block_sum<SEL_THREADS>(eq, tmp);
    }
    for (int e = 0; e < SEL_PER_THREAD; ++e) {
      const int li = e * SEL_THREADS + threadIdx.x;
      const int32_t i = base + li;
      const int c = (i < P.n_gpu) ? sel_class(src, 0, i, p) : 0;
      cls_lds[(li >> 4) * (SEL_PER_THREAD + 1) + (li & 15)] = static_cast<uint8_t>(c);
    }
    __syncthreads();
    const uint8_t *mine = cls_lds + threadIdx.x * (SEL_PER_THREAD + 1);
    uint32_t n_eq = 0;
    for (int e = 0; e < SEL_PER_THREAD; ++e) n_eq += (mine[e] == 2);
    uint32_t tot;
    uint32_t r = eq_before + block_excl_scan<SEL_THREADS>(n_eq, tmp, &tot);
    (void)lt_before;
    const int32_t i0 = base + threadIdx.x * SEL_PER_THREAD;
    for (int e = 0; e < SEL_PER_THREAD; ++e) {
      const int c = mine[e];
      bool take = (c == 1);
      if (c == 2) { take = r < p.k_rem; ++r; }
      if (take) {
        const int32_t slot = i0 + e;
        const int32_t h = P.to_host[slot];
        if (h >= 0 && h < P.n_host) P.host_to_gpu[h] = INF;
        P.to_host[slot] = INF;
        P.priority[slot] = -1;
        P.free_[slot] = 1;   // the row stays where it is: the host holds the backup
      }
    }
    __syncthreads();
  }
  // free slots of this chunk after eviction (feeds the ascending allocation)
  uint32_t nf = 0;
  for (int e = 0; e < SEL_PER_THREAD; ++e) {
    const int32_t i = base + e * SEL_THREADS + threadIdx.x;
    if (i < P.n_gpu) nf += (P.free_[i] == 1);
  }
  nf = block_sum<SEL_THREADS>(nf, tmp);
  if (threadIdx.x == 0) W.chunk_free[chunk] = nf;
}

// ------------------------------------------------------------------ ascending allocation
__global__ __launch_bounds__(SEL_THREADS) void pool_alloc_kernel(
    PoolArgs P, PoolWs W, int32_t step_id, int32_t *__restrict__ miss_host,
    int32_t *__restrict__ miss_slot, int32_t *__restrict__ topk_slot) {
  __shared__ uint32_t tmp[48];
  if (*(volatile int32_t *)P.status) return;
  const int32_t n_miss = W.counters[0];
  if (n_miss == 0) return;
  const int chunk = blockIdx.x;
  uint32_t before = 0;
  for (int c = threadIdx.x; c < chunk; c += SEL_THREADS) before += W.chunk_free[c];
  before = block_sum<SEL_THREADS>(before, tmp);
  if (before >= static_cast<uint32_t>(n_miss)) return;
  const int32_t i0 = chunk * SEL_CHUNK + threadIdx.x * SEL_PER_THREAD;
  uint32_t nf = 0;
  for (int e = 0; e < SEL_PER_THREAD; ++e) {
    const int32_t i = i0 + e;
    if (i < P.n_gpu) nf += (P.free_[i] == 1);
  }
  uint32_t tot;
  uint32_t rank = before + block_excl_scan<SEL_THREADS>(nf, tmp, &tot);
  for (int e = 0; e < SEL_PER_THREAD && rank < static_cast<uint32_t>(n_miss); ++e) {
    const int32_t slot = i0 + e;
    if (slot >= P.n_gpu || P.free_[slot] != 1) continue;
    const int32_t h = miss_host[rank];
    P.free_[slot] = 0;
    P.to_host[slot] = h;
    P.host_to_gpu[h] = slot;
    P.priority[slot] = step_id;
    if (rank < static_cast<uint32_t>(P.n_gpu)) P.indices_buf[rank] = slot;
    miss_slot[rank] = slot;
    topk_slot[W.miss_entry[rank]] = slot;
    ++rank;
  }
}

// ------------------------------------------------------------------ finalize
__global__ __launch_bounds__(PL_THREADS) void pool_finalize_kernel(
    PoolArgs P, PoolWs W, const int32_t *__restrict__ idx, int32_t n_rows, int32_t k,
    int32_t step_id, const int32_t *__restrict__ topk_slot) {
  const int64_t n_ent = static_cast<int64_t>(n_rows) * k;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * PL_THREADS + threadIdx.x;
  const int32_t st = *(volatile int32_t *)P.status;
  const bool abort = (st & (ECHO_ST_EXHAUSTED | ECHO_ST_BAD_HOST)) != 0;
  if (e < n_ent && idx[e] >= 0) {
    const int32_t h = W.ent_host[e];   // >= 0 for a miss
    const int32_t slot = topk_slot[e];
    if (h < 0) {
      if (slot >= 0 && slot < P.n_gpu) {
        P.free_[slot] = 0;                           // clear the protection mark
        if (!abort) P.priority[slot] = step_id;
      }
    } else if (!abort) {
      if (slot < 0 || slot >= P.n_gpu || P.host_to_gpu[h] != slot)
        atomicOr(P.status, ECHO_ST_DUP_HOST);
      else
        P.priority[slot] = step_id;
    }
  }
  if (!abort) {
    const int64_t lim = min<int64_t>(P.n_gpu, n_ent);
    const int64_t j = W.counters[0] + e;
    if (j < lim) P.indices_buf[j] = -1;
  }
}

int launch_pool_lookup_alloc(const echo_pool *pool, const int32_t *idx, const int64_t *key_begin,
                             const int32_t *req_to_host, int64_t n_k, int32_t n_rows, int32_t k,
                             int32_t step_id, int32_t *topk_slot, int32_t *miss_host,
                             int32_t *miss_slot, int32_t *n_miss, void *ws, size_t ws_bytes,
                             hipStream_t st) {
  PoolWs W;
  size_t need;
  pool_ws_layout(n_rows, k, pool->n_gpu, ws, &W, &need);
  if (ws_bytes < need) return fail(ECHO_EWORKSPACE, "echo_pool_lookup_alloc: workspace %zu < %zu", ws_bytes, need);
  if (pool_small_fits(pool->n_gpu))
    return launch_pool_small(pool, W.miss_entry, idx, key_begin, req_to_host, n_k, n_rows, k,
                             step_id, topk_slot, miss_host, miss_slot, n_miss, st);
  PoolArgs P{pool->gpu_free, pool->gpu_priority, pool->gpu_to_host, pool->host_to_gpu,
             pool->indices_buf, pool->status, pool->n_gpu, pool->n_host};
  const int64_t n_ent = static_cast<int64_t>(n_rows) * k;
  const unsigned lwg = static_cast<unsigned>(W.n_lookup_wg);
  pool_lookup_kernel<<<lwg, PL_THREADS, 0, st>>>(P, W, idx, key_begin, req_to_host, n_k, n_rows, k, topk_slot);
  pool_compact_kernel<<<lwg, PL_THREADS, 0, st>>>(P, W, n_rows, k, miss_host, miss_slot, n_miss);
  const unsigned sg = static_cast<unsigned>(W.n_chunks);
  evict_hist_kernel<0><<<sg, SEL_THREADS, 0, st>>>(P, W);
  evict_hist_kernel<1><<<sg, SEL_THREADS, 0, st>>>(P, W);
  evict_hist_kernel<2><<<sg, SEL_THREADS, 0, st>>>(P, W);
  evict_count_kernel<<<sg, SEL_THREADS, 0, st>>>(P, W);
  evict_apply_kernel<<<sg, SEL_THREADS, 0, st>>>(P, W);
  pool_alloc_kernel<<<sg, SEL_THREADS, 0, st>>>(P, W, step_id, miss_host, miss_slot, topk_slot);
  const int64_t fin = std::max<int64_t>(n_ent, 1);
  pool_finalize_kernel<<<static_cast<unsigned>((fin + PL_THREADS - 1) / PL_THREADS), PL_THREADS, 0, st>>>(
      P, W, idx, n_rows, k, step_id, topk_slot);
  (void)n_ent;
  return check_launch("pool_lookup_alloc");
}

// ------------------------------------------------------------------ pool init / status
__global__ void pool_init_kernel(PoolArgs P) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < P.n_gpu; i += stride) {
    P.free_[i] = 1;
    P.priority[i] = -1;
    P.to_host[i] = INF;
    P.indices_buf[i] = -1;
  }
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < P.n_host; i += stride)
    P.host_to_gpu[i] = INF;
  if (blockIdx.x == 0 && threadIdx.x == 0) *P.status = 0;
}

__global__ void status_clear_kernel(int32_t *s) { *s = 0; }

}  // namespace echo

using namespace echo;

static int check_pool(const echo_pool *pool, const char *fn) {
  if (!pool) return fail(ECHO_EINVAL, "%s: NULL pool", fn);
  if (pool->n_gpu < 1 || pool->n_host < 1) return fail(ECHO_EINVAL, "%s: pool sizes must be >= 1", fn);
  if (!pool->gpu_free || !pool->gpu_priority || !pool->gpu_to_host || !pool->host_to_gpu ||
      !pool->indices_buf || !pool->status)
    return fail(ECHO_EINVAL, "%s: NULL pool member", fn);
  return ECHO_OK;
}

extern "C" size_t echo_pool_workspace_bytes(int32_t n_rows, int32_t k, int32_t n_gpu) {
  if (n_rows < 0 || k < 0 || n_gpu < 0) return 0;
  return pool_ws_bytes(n_rows, k, n_gpu);
}

extern "C" int echo_pool_lookup_alloc(const echo_pool *pool, const int32_t *idx,
                                      const int64_t *key_begin, const int32_t *req_to_host,
                                      int64_t n_k, int32_t n_rows, int32_t k, int32_t step_id,
                                      int32_t *topk_slot, int32_t *miss_host, int32_t *miss_slot,
                                      int32_t *n_miss, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_pool(pool, "echo_pool_lookup_alloc");
  if (rc) return rc;
  if (n_rows < 0 || k < 1 || n_k < 0) return fail(ECHO_EINVAL, "echo_pool_lookup_alloc: bad n_rows/k/n_k");
  if (static_cast<int64_t>(n_rows) * k > (1LL << 30)) return fail(ECHO_EUNSUPPORTED, "echo_pool_lookup_alloc: too many entries");
  if (!idx || !key_begin || !req_to_host || !topk_slot || !miss_host || !miss_slot || !n_miss || !ws)
    return fail(ECHO_EINVAL, "echo_pool_lookup_alloc: NULL pointer");
  return launch_pool_lookup_alloc(pool, idx, key_begin, req_to_host, n_k, n_rows, k, step_id,
                                  topk_slot, miss_host, miss_slot, n_miss, ws, ws_bytes, S(stream));
}

extern "C" int echo_pool_init(echo_pool *pool, void *stream) {
  int rc = check_pool(pool, "echo_pool_init");
  if (rc) return rc;
  PoolArgs P{pool->gpu_free, pool->gpu_priority, pool->gpu_to_host, pool->host_to_gpu,
             pool->indices_buf, pool->status, pool->n_gpu, pool->n_host};
  pool_init_kernel<<<1024, 256, 0, S(stream)>>>(P);
  return check_launch("pool_init");
}

extern "C" int echo_status_clear(int32_t *status, void *stream) {
  if (!status) return fail(ECHO_EINVAL, "echo_status_clear: NULL");
  status_clear_kernel<<<1, 1, 0, S(stream)>>>(status);
  return check_launch("status_clear");
}
