// Launch helpers shared between the library's translation units (host side).
#pragma once

#include "common.hpp"

namespace echo {

struct PrefetchArgs {
  const float *theta;        // [n_q]
  const int32_t *req_to_host;// [n_k]
  const int32_t *host_to_gpu;// [n_host]
  int32_t *cand;             // [n_q, cap] this call's list
  int32_t *cand_cnt;         // [n_q] this call's list lengths
  int32_t *total_cnt;        // [n_q] over-threshold non-resident tokens of the step so far
  int32_t cap;
  int32_t cap_div;
};

struct PoolArgs {
  uint8_t *free_;
  int32_t *priority;
  int32_t *to_host;
  int32_t *host_to_gpu;
  int32_t *indices_buf;
  int32_t *status;
  int32_t n_gpu, n_host;
};

// hist0 (optional, [n_q][2048]): digit-0 histogram of the top-k keys of the scores, added to
int launch_score_decode(const uint8_t *q, const float *w, const uint8_t *k, const float *k_scale,
                        const int64_t *key_begin, const int32_t *key_len, int32_t n_q,
                        int32_t max_len, int32_t tok_lo, int32_t tok_hi, float *scores,
                        int64_t ld, const PrefetchArgs *pf, uint32_t *hist0, hipStream_t st);

size_t topk_ws_bytes(int32_t n_rows, int32_t max_len);
// hist0: optional digit-0 histograms from launch_score_decode
int launch_topk_rows(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                     int32_t max_len, int32_t k, const uint32_t *hist0, int32_t *idx,
                     hipStream_t st);
int launch_topk(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                int32_t max_len, int32_t k, int32_t *idx, void *ws, size_t ws_bytes,
                hipStream_t st);

// Workspace of the multi-workgroup pool step (pool_fast.hip).  The first zero_words 32-bit
// words (counters, priority histograms, protection bitmap) must be zeroed before each step.
struct PoolFastWs {
  int32_t *counters;      // [16]: 0 free slots (stats; prefetch decrements)
  uint32_t *fine;         // [65536] occupied, unprotected slots per priority bin
  uint32_t *coarse;       // [2048]  the same, 32 fine bins per coarse bin
  uint32_t *prot;         // [ceil(n_gpu/32)] protection bitmap (slots holding a selected token)
  uint32_t *row_miss_cnt; // [n_rows]
  int32_t *row_miss_h;    // [n_rows * k] ordered misses of each request: host index
  int32_t *row_miss_j;    // [n_rows * k] ... and column in the request's selection
  uint32_t *chunk_free;   // [n_chunks] free slots per 4096-slot chunk after the first evictions
  uint32_t *chunk_cand;   // [n_chunks] threshold-bin slots per chunk
  uint64_t *cand;         // [n_chunks * 4096] (priority key << 32 | slot), per chunk in slot order
  int32_t *miss_entry;    // [n_rows * k] entry (r*k + j) of the i-th miss
  void *base;
  int32_t n_chunks;
  int64_t zero_words;
};
void pool_fast_ws_layout(int32_t n_rows, int32_t k, int32_t n_gpu, void *base, PoolFastWs *w,
                         size_t *bytes);
size_t pool_fast_ws_bytes(int32_t n_rows, int32_t k, int32_t n_gpu);
int launch_pool_stats(const echo_pool *pool, const PoolFastWs &W, int32_t step_id, hipStream_t st);
int launch_pool_lookup_rows(const echo_pool *pool, const PoolFastWs &W, const int32_t *idx,
                            const int64_t *key_begin, const int32_t *req_to_host, int64_t n_k,
                            int32_t n_rows, int32_t k, int32_t step_id, int32_t *topk_slot,
                            hipStream_t st);
int launch_pool_evict(const echo_pool *pool, const PoolFastWs &W, const int32_t *idx, int32_t n_rows,
                      int32_t k, int32_t step_id, int32_t *topk_slot, int32_t *miss_host,
                      int32_t *miss_slot, int32_t *n_miss, hipStream_t st);

int launch_pool_step(const echo_pool *pool, const int32_t *idx, const int64_t *key_begin,
                     const int32_t *req_to_host, int64_t n_k, int32_t n_rows, int32_t k,
                     int32_t step_id, int32_t *topk_slot, int32_t *miss_host, int32_t *miss_slot,
                     int32_t *n_miss, void *ws, size_t ws_bytes, hipStream_t st);

// Decode top-k: split (multi-workgroup) then finish (one workgroup per request); when pool is
// not NULL the finish also performs the residency lookup into *pw (whose zeroed region and
// statistics must be ready).
size_t topk_split_ws_bytes(int32_t n_rows, int32_t max_len, int32_t k);
int launch_topk_split(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                      int32_t max_len, int32_t k, const uint32_t *hist0, void *split_ws,
                      hipStream_t st);
int launch_topk_finish(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                       int32_t max_len, int32_t k, const uint32_t *hist0, void *split_ws,
                       int32_t *idx, const echo_pool *pool, const PoolFastWs *pw,
                       const int64_t *key_begin, const int32_t *req_to_host, int32_t step_id,
                       int32_t *topk_slot, hipStream_t st);

int launch_recall_gather(const echo_pool *pool, const int32_t *miss_host, const int32_t *miss_slot,
                         const int32_t *n_miss, int32_t max_miss, hipStream_t st);

int launch_prefetch_threshold(const uint8_t *q, const float *w, const uint8_t *k,
                              const float *k_scale, const int64_t *key_begin,
                              const int32_t *key_len, int32_t n_q, int32_t n_sample,
                              float percentile, float *theta, hipStream_t st);
int launch_prefetch_begin(const echo_pool *pool, int32_t *free_list, int32_t *free_count,
                          hipStream_t st);
// pw (optional): pool-step statistics kept consistent with the allocations (free count, and
// the priority histogram for the new slots' priority 0 relative to step_id)
int launch_prefetch_gather(const echo_pool *pool, const int64_t *key_begin,
                           const int32_t *req_to_host, const int32_t *cand,
                           const int32_t *cand_cnt, int32_t n_q, int32_t cap,
                           const int32_t *free_list, int32_t *free_count, int32_t *n_prefetched,
                           const PoolFastWs *pw, int32_t step_id, hipStream_t st);
int launch_zero_i32(int32_t *p, int64_t n, hipStream_t st);
int launch_zero2_i32(int32_t *p, int64_t n, int32_t *q, int64_t m, hipStream_t st);
int launch_sum_i32(const int32_t *v, int32_t n, int32_t *out, hipStream_t st);

}  // namespace echo
