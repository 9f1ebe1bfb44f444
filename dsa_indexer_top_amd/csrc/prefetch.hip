// Threshold prefetch (ECHO review page §6.1): turn the top-k into a "score above a predicted
// threshold" test that can be applied while scores are still being produced, and start moving
// those rows from host memory before the exact top-k is known.  Prefetch only decides what
// moves early; the guaranteed recall after the exact top-k fills every gap, so the selected
// set and the attended rows are the same with or without it.
//
//   threshold  per request, the nearest-rank percentile of the scores of a fixed, evenly
//              spaced sample of its tokens (a single step has no history for the page's EMA
//              of the k-th score).  One workgroup per request scores the sample with the same
//              MFMA tile as the main scoring kernel, then bitonic-sorts it in LDS.
//   begin      lists the free slots of the pool (in no particular order) for prefetch to take.
//   gather     for the candidates one scoring call appended: take free slots (never evict),
//              set both maps, priority 0 (first to go if space is short later), and copy the
//              rows from mapped pinned host memory.  Runs on a side stream while the next
//              scoring call runs on the main stream: the two touch disjoint host indices.
#include <algorithm>
#include <cmath>

#include "internal.hpp"
#include "pool_common.cuh"
#include "score_tile.cuh"

namespace echo {

constexpr int PT_THREADS = 256;
constexpr int PT_MAX_SAMPLE = 4096;

__global__ __launch_bounds__(PT_THREADS) void prefetch_threshold_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ w, const uint8_t *__restrict__ k,
    const float *__restrict__ k_scale, const int64_t *__restrict__ key_begin,
    const int32_t *__restrict__ key_len, int32_t n_sample, int32_t rank, float *__restrict__ theta) {
  __shared__ float smp[PT_MAX_SAMPLE];
  const int r = blockIdx.x;
  const int32_t L = key_len[r];
  if (L <= 0) {
    if (threadIdx.x == 0) theta[r] = INFINITY;
    return;
  }
  const int64_t kb = key_begin[r];
  QOperand qo;
  load_q_operand(q, w, r, qo);
  const int l = lane_id(), j = l & 15, g = l >> 4, wv = threadIdx.x >> 6;
  const int per_wave = n_sample / (PT_THREADS / 64);
  for (int i0 = wv * per_wave; i0 < (wv + 1) * per_wave; i0 += 16) {
    const int i = i0 + j;
    const int64_t pos = (static_cast<int64_t>(i) * L) / n_sample;     // sample position
    const int4 *kp = reinterpret_cast<const int4 *>(k + (kb + pos) * D + 32 * g);
    const int4 b0 = kp[0], b1 = kp[1];
    float s = reduce_groups(score_tile_partial(qo, v8i{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w}));
    if (k_scale) s *= k_scale[kb + pos];
    if (g == 0) smp[i] = s;
  }
  __syncthreads();
  // bitonic sort, ascending
  for (int size = 2; size <= n_sample; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n_sample; i += PT_THREADS) {
        const int p = i ^ stride;
        if (p > i) {
          const bool up = (i & size) == 0;
          const float a = smp[i], b = smp[p];
          if ((a > b) == up) {
            smp[i] = b;
            smp[p] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) theta[r] = smp[rank - 1];
}

int launch_prefetch_threshold(const uint8_t *q, const float *w, const uint8_t *k,
                              const float *k_scale, const int64_t *key_begin,
                              const int32_t *key_len, int32_t n_q, int32_t n_sample,
                              float percentile, float *theta, hipStream_t st) {
  if (n_q == 0) return ECHO_OK;
  int32_t rank = static_cast<int32_t>(std::ceil(static_cast<double>(percentile) / 100.0 * n_sample));
  rank = std::min(std::max(rank, 1), n_sample);
  prefetch_threshold_kernel<<<n_q, PT_THREADS, 0, st>>>(q, w, k, k_scale, key_begin, key_len,
                                                        n_sample, rank, theta);
  return check_launch("prefetch_threshold");
}

// ------------------------------------------------------------------ free-slot list
// free_count[0] = number listed, free_count[1] = number taken by prefetch (both zeroed here).
__global__ void prefetch_count_reset_kernel(int32_t *free_count) {
  free_count[0] = 0;
  free_count[1] = 0;
}

__global__ __launch_bounds__(256) void prefetch_free_list_kernel(const uint8_t *__restrict__ free_,
                                                                 int32_t n_gpu, int32_t *free_list,
                                                                 int32_t *free_count) {
  __shared__ uint32_t tmp[48];
  __shared__ int32_t base;
  for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * 256; c0 < n_gpu; c0 += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t i = c0 + threadIdx.x;
    const uint32_t f = (i < n_gpu && free_[i] == 1) ? 1u : 0u;
    uint32_t tot;
    const uint32_t off = block_excl_scan<256>(f, tmp, &tot);
    if (threadIdx.x == 0) base = tot ? atomicAdd(free_count, static_cast<int32_t>(tot)) : 0;
    __syncthreads();
    if (f) free_list[base + off] = static_cast<int32_t>(i);
    __syncthreads();
  }
}

int launch_prefetch_begin(const echo_pool *pool, int32_t *free_list, int32_t *free_count,
                          hipStream_t st) {
  prefetch_count_reset_kernel<<<1, 1, 0, st>>>(free_count);
  const int blocks = std::min(1024, (pool->n_gpu + 255) / 256);
  prefetch_free_list_kernel<<<std::max(blocks, 1), 256, 0, st>>>(pool->gpu_free, pool->n_gpu, free_list, free_count);
  return check_launch("prefetch_begin");
}

// ------------------------------------------------------------------ prefetch gather
__global__ __launch_bounds__(PG_THREADS) void prefetch_gather_kernel(GatherArgs G) {
  __shared__ uint32_t lds[PG_LDS_WORDS];
  gather_request(G, blockIdx.x, lds);
}

GatherArgs make_gather_args(const echo_pool *pool, const int64_t *key_begin,
                            const int32_t *req_to_host, const int32_t *cand,
                            const int32_t *cand_cnt, int32_t cap, const int32_t *free_list,
                            int32_t *free_count, int32_t *n_prefetched, const PoolFastWs *pw,
                            Stamp stamp) {
  return GatherArgs{pool->host_kv, pool->gpu_kv, pool->gpu_free, pool->gpu_priority,
                    pool->gpu_to_host, pool->host_to_gpu, pool->status, pool->n_gpu, pool->n_host,
                    key_begin, req_to_host, cand, cand_cnt, cap, free_list, free_count,
                    n_prefetched, pw ? pw->counters : nullptr, pw ? pw->fine : nullptr,
                    pw ? pw->coarse : nullptr, stamp};
}

int launch_prefetch_gather(const echo_pool *pool, const int64_t *key_begin,
                           const int32_t *req_to_host, const int32_t *cand,
                           const int32_t *cand_cnt, int32_t n_q, int32_t cap,
                           const int32_t *free_list, int32_t *free_count, int32_t *n_prefetched,
                           const PoolFastWs *pw, Stamp stamp, hipStream_t st) {
  if (n_q == 0 || cap == 0) return ECHO_OK;
  prefetch_gather_kernel<<<n_q, PG_THREADS, 0, st>>>(make_gather_args(
      pool, key_begin, req_to_host, cand, cand_cnt, cap, free_list, free_count, n_prefetched, pw, stamp));
  return check_launch("prefetch_gather");
}

__global__ __launch_bounds__(256) void sum_i32_kernel(const int32_t *v, int32_t n, int32_t *out) {
  __shared__ uint32_t tmp[48];
  uint32_t s = 0;
  for (int i = threadIdx.x; i < n; i += 256) s += static_cast<uint32_t>(v[i]);
  s = block_sum<256>(s, tmp);
  if (threadIdx.x == 0) *out = static_cast<int32_t>(s);
}

int launch_sum_i32(const int32_t *v, int32_t n, int32_t *out, hipStream_t st) {
  sum_i32_kernel<<<1, 256, 0, st>>>(v, n, out);
  return check_launch("sum");
}

}  // namespace echo

using namespace echo;

extern "C" int echo_prefetch_threshold(const uint8_t *q, const float *w, const uint8_t *k,
                                       const float *k_scale, const int64_t *key_begin,
                                       const int32_t *key_len, int32_t n_q, int32_t n_sample,
                                       float percentile, float *theta, void *stream) {
  if (n_q < 0) return fail(ECHO_EINVAL, "echo_prefetch_threshold: n_q < 0");
  if (n_sample < 64 || n_sample > PT_MAX_SAMPLE || (n_sample & (n_sample - 1)))
    return fail(ECHO_EUNSUPPORTED, "echo_prefetch_threshold: n_sample must be a power of two in [64, 4096]");
  if (!(percentile > 0.f && percentile <= 100.f)) return fail(ECHO_EINVAL, "echo_prefetch_threshold: percentile outside (0, 100]");
  if (n_q > 0 && (!q || !w || !k || !key_begin || !key_len || !theta))
    return fail(ECHO_EINVAL, "echo_prefetch_threshold: NULL pointer");
  return launch_prefetch_threshold(q, w, k, k_scale, key_begin, key_len, n_q, n_sample, percentile, theta, S(stream));
}

extern "C" int echo_prefetch_begin(const echo_pool *pool, int32_t *free_list, int32_t *free_count,
                                   void *stream) {
  if (!pool || !pool->gpu_free || pool->n_gpu < 1 || !free_list || !free_count)
    return fail(ECHO_EINVAL, "echo_prefetch_begin: NULL or empty pool");
  return launch_prefetch_begin(pool, free_list, free_count, S(stream));
}

extern "C" int echo_prefetch_gather(const echo_pool *pool, const int64_t *key_begin,
                                    const int32_t *req_to_host, const int32_t *cand,
                                    const int32_t *cand_cnt, int32_t n_q, int32_t cap,
                                    const int32_t *free_list, int32_t *free_count,
                                    int32_t *n_prefetched, void *stream) {
  if (!pool || !pool->gpu_kv || !pool->host_kv || !pool->status || !pool->gpu_free || !pool->gpu_priority ||
      !pool->gpu_to_host || !pool->host_to_gpu)
    return fail(ECHO_EINVAL, "echo_prefetch_gather: NULL pool member");
  if (pool->n_gpu < 1 || pool->n_host < 1) return fail(ECHO_EINVAL, "echo_prefetch_gather: empty pool");
  if (n_q < 0 || cap < 0) return fail(ECHO_EINVAL, "echo_prefetch_gather: negative size");
  if (n_q > 0 && cap > 0 && (!key_begin || !req_to_host || !cand || !cand_cnt || !free_list || !free_count || !n_prefetched))
    return fail(ECHO_EINVAL, "echo_prefetch_gather: NULL pointer");
  return launch_prefetch_gather(pool, key_begin, req_to_host, cand, cand_cnt, n_q, cap, free_list,
                                free_count, n_prefetched, nullptr, Stamp{0, nullptr}, S(stream));
}
