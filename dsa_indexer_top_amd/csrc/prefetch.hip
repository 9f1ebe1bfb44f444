// Threshold prefetch (ECHO review page §6.1): turn the top-k into a "score above a predicted
// threshold" test that can be applied while scores are still being produced, and start moving
// those rows from host memory before the exact top-k is known.  Prefetch only decides what
// moves early; the guaranteed recall after the exact top-k fills every gap, so the selected
// set and the attended rows are the same with or without it.
//
//   threshold  per request, the nearest-rank percentile of the scores of a fixed, evenly
//              spaced sample of its tokens (a single step has no history for the page's EMA
//              of the k-th score).  One 1024-thread workgroup per request: its 16 waves score
//              the sample with the same MFMA tile as the main scoring kernel (four tiles' key
//              loads in flight at a time), and a three-pass radix select (11 + 11 + 10 bits of
//              the order key, LDS histograms) finds the sampled score of the wanted rank.
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

constexpr int PT_THREADS = 1024;
constexpr int PT_WAVES = PT_THREADS / 64;
constexpr int PT_MAX_SAMPLE = 4096;
constexpr int PT_BATCH = 4;                       // sample tiles whose key loads are in flight

// Float with order key `key` (the inverse of f32_key on its image).
ECHO_DEV float key_f32(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__global__ __launch_bounds__(PT_THREADS) void prefetch_threshold_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ w, const uint8_t *__restrict__ k,
    const float *__restrict__ k_scale, const int64_t *__restrict__ key_begin,
    const int32_t *__restrict__ key_len, int32_t max_len, int32_t n_sample, int32_t rank,
    float *__restrict__ theta, KeyPages kp) {
  __shared__ uint32_t skey[PT_MAX_SAMPLE];        // order keys of the sampled scores
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t tmp[48];
  const int r = blockIdx.x;
  const int32_t L = min(max(key_len[r], 0), max_len);
  if (L <= 0) {
    if (threadIdx.x == 0) theta[r] = INFINITY;
    return;
  }
  const int64_t kb = key_begin ? key_begin[r] : 0;
  const int l = lane_id(), j = l & 15, g = l >> 4, wv = threadIdx.x >> 6;
  const int n_tiles = n_sample / 16;              // >= 4; wave wv takes tiles wv, wv + 16, ...
  if (wv < n_tiles) {                              // uniform per wave
    QOperand qo;
    load_q_operand(q, w, r, qo);
    for (int t0 = wv; t0 < n_tiles; t0 += PT_WAVES * PT_BATCH) {
      int4 b0[PT_BATCH], b1[PT_BATCH];
      float sc[PT_BATCH];
#pragma unroll
      for (int u = 0; u < PT_BATCH; ++u) {            // every load of the batch before any use
        const int tile = t0 + u * PT_WAVES;
        const int i = (tile < n_tiles ? tile : t0) * 16 + j;
        const int32_t pos = static_cast<int32_t>((static_cast<int64_t>(i) * L) / n_sample);  // < L
        const int64_t row = key_row(kp, r, kb, pos);
        const int4 *kr = reinterpret_cast<const int4 *>(k + row * D + 32 * g);
        b0[u] = kr[0];
        b1[u] = kr[1];
        sc[u] = k_scale ? k_scale[row] : 1.f;
      }
#pragma unroll
      for (int u = 0; u < PT_BATCH; ++u) {
        const int tile = t0 + u * PT_WAVES;
        if (tile >= n_tiles) break;                // uniform
        float s = reduce_groups(score_tile_partial(
            qo, v8i{b0[u].x, b0[u].y, b0[u].z, b0[u].w, b1[u].x, b1[u].y, b1[u].z, b1[u].w}));
        if (k_scale) s *= sc[u];
        if (g == 0) skey[tile * 16 + j] = f32_key(s);
      }
    }
  }
  // radix select of the rank-th smallest key: top 11 bits, next 11, last 10
  uint32_t want = static_cast<uint32_t>(rank), prefix = 0, mask = 0;
  for (int d = 0; d < 3; ++d) {
    const int sh = d == 0 ? 21 : (d == 1 ? 10 : 0);
    const uint32_t dm = d == 2 ? 0x3FFu : 0x7FFu;
    for (int b = threadIdx.x; b < 2048; b += PT_THREADS) hist[b] = 0;
    __syncthreads();                                // also orders the sample stores above
    for (int i0 = 0; i0 < PT_MAX_SAMPLE; i0 += PT_THREADS) {      // uniform trip count
      const int i = i0 + threadIdx.x;
      const uint32_t kk = i < n_sample ? skey[i] : 0u;
      hist_add_peeled(hist, (kk >> sh) & dm, i < n_sample && (kk & mask) == prefix);
    }
    __syncthreads();
    uint32_t bin, below, count;
    pick2048<PT_THREADS>(hist, want, tmp, bin, below, count);
    want -= below;
    prefix |= bin << sh;
    mask |= dm << sh;
  }
  if (threadIdx.x == 0) theta[r] = key_f32(prefix);
}

int launch_prefetch_threshold(const uint8_t *q, const float *w, const uint8_t *k,
                              const float *k_scale, const int64_t *key_begin,
                              const int32_t *key_len, int32_t n_q, int32_t max_len,
                              int32_t n_sample, float percentile, float *theta, const KeyPages *kp,
                              hipStream_t st) {
  if (n_q == 0) return ECHO_OK;
  int32_t rank = static_cast<int32_t>(std::ceil(static_cast<double>(percentile) / 100.0 * n_sample));
  rank = std::min(std::max(rank, 1), n_sample);
  prefetch_threshold_kernel<<<n_q, PT_THREADS, 0, st>>>(q, w, k, k_scale, key_begin, key_len,
                                                        max_len, n_sample, rank, theta,
                                                        kp ? *kp : KeyPages{nullptr, 0, 0});
  return check_launch("prefetch_threshold");
}

// ------------------------------------------------------------------ free-slot list
// free_count[0] = number listed, free_count[1] = number taken by prefetch (both zeroed here).
__global__ void prefetch_count_reset_kernel(int32_t *free_count) {
  free_count[0] = 0;
  free_count[1] = 0;
}

// One workgroup per 4096-slot chunk, 16 slots per thread; one global atomic per workgroup.
constexpr int FL_T = 256, FL_CH = 4096;
__global__ __launch_bounds__(FL_T) void prefetch_free_list_kernel(const uint8_t *__restrict__ free_,
                                                                  int32_t n_gpu, int32_t *free_list,
                                                                  int32_t *free_count) {
  __shared__ uint32_t tmp[48];
  const int t = threadIdx.x;
  uint32_t fw[4], nf = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t s0 = static_cast<int64_t>(blockIdx.x) * FL_CH + j * 4 * FL_T + t * 4;
    if (s0 + 3 < n_gpu) {
      fw[j] = *reinterpret_cast<const uint32_t *>(free_ + s0);
    } else {
      fw[j] = 0;
      for (int e = 0; e < 4; ++e)
        if (s0 + e < n_gpu) fw[j] |= static_cast<uint32_t>(free_[s0 + e]) << (8 * e);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) nf += ((fw[j] >> (8 * e)) & 0xFFu) == 1u;
  }
  uint32_t tot;
  const uint32_t off = block_excl_scan<FL_T>(nf, tmp, &tot);
  if (t == 0) tmp[44] = tot ? static_cast<uint32_t>(atomicAdd(free_count, static_cast<int32_t>(tot))) : 0u;
  __syncthreads();
  uint32_t pos = tmp[44] + off;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (((fw[j] >> (8 * e)) & 0xFFu) == 1u)
        free_list[pos++] = static_cast<int32_t>(static_cast<int64_t>(blockIdx.x) * FL_CH + j * 4 * FL_T + t * 4 + e);
}

int launch_prefetch_begin(const echo_pool *pool, int32_t *free_list, int32_t *free_count,
                          hipStream_t st) {
  prefetch_count_reset_kernel<<<1, 1, 0, st>>>(free_count);
  const int blocks = (pool->n_gpu + FL_CH - 1) / FL_CH;
  prefetch_free_list_kernel<<<std::max(blocks, 1), FL_T, 0, st>>>(pool->gpu_free, pool->n_gpu, free_list, free_count);
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
                                       const int32_t *key_len, int32_t n_q, int32_t max_key_len,
                                       int32_t n_sample, float percentile, float *theta,
                                       void *stream) {
  if (n_q < 0 || max_key_len < 0) return fail(ECHO_EINVAL, "echo_prefetch_threshold: n_q or max_key_len < 0");
  if (n_q > 65535) return fail(ECHO_EUNSUPPORTED, "echo_prefetch_threshold: n_q %d > 65535", n_q);
  if (n_sample < 64 || n_sample > PT_MAX_SAMPLE || (n_sample & (n_sample - 1)))
    return fail(ECHO_EUNSUPPORTED, "echo_prefetch_threshold: n_sample must be a power of two in [64, 4096]");
  if (!(percentile > 0.f && percentile <= 100.f)) return fail(ECHO_EINVAL, "echo_prefetch_threshold: percentile outside (0, 100]");
  if (n_q > 0 && (!q || !w || !k || !key_begin || !key_len || !theta))
    return fail(ECHO_EINVAL, "echo_prefetch_threshold: NULL pointer");
  return launch_prefetch_threshold(q, w, k, k_scale, key_begin, key_len, n_q, max_key_len, n_sample,
                                   percentile, theta, nullptr, S(stream));
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
