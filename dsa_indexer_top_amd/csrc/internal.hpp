// Launch helpers shared between the library's translation units (host side).
#pragma once

#include "common.hpp"

namespace echo {

// The step stamp, the priority given to the slots a step selects or fills: a host value, or a
// device word that the caller advances between steps, so that one captured graph can serve every
// step.  Kernels read it once at their start.
struct Stamp {
  int32_t value;
  const int32_t *dev;        // nullptr: use value
};
ECHO_DEV int32_t stamp_of(const Stamp &s) { return s.dev ? *s.dev : s.value; }

// Paged indexer-K cache: token t of request r lives at row (table[r * max_pages + t / P] * P +
// t % P) of k and k_scale, P = 1 << shift tokens per page; table == nullptr for the contiguous
// layout (row key_begin[r] + t).
struct KeyPages {
  const int32_t *table;
  int32_t shift;
  int32_t max_pages;
};
ECHO_DEV int64_t key_row(const KeyPages &kp, int r, int64_t kb, int32_t t) {
  if (!kp.table) return kb + t;
  const int64_t page = kp.table[static_cast<int64_t>(r) * kp.max_pages + (t >> kp.shift)];
  return (page << kp.shift) | (t & ((1 << kp.shift) - 1));
}

// Page arguments of a paged key cache, checked (page size a power of two in [16, 65536],
// max_pages * page_size >= max_key_len); fn names the entry point in the error text.
int key_pages_of(const int32_t *page_table, int32_t page_size, int32_t max_pages, int32_t max_key_len,
                 const char *fn, KeyPages *kp);

struct PrefetchArgs {
  const float *theta;        // [n_q]
  const int32_t *req_to_host;// [n_k]
  const int32_t *host_to_gpu;// [n_host]
  int32_t *cand;             // [n_q, cap] this call's list
  int32_t *cand_cnt;         // [n_q] this call's list lengths
  int32_t *total_cnt;        // [n_q] over-threshold non-resident tokens of the step so far
  int32_t cap;
  int32_t cap_div;
  int32_t n_host;            // host indices outside [0, n_host) never qualify
  int32_t call, n_calls;     // the calls of a step share cap_r: calls 0..c together list at
                             // most floor(cap_r (c+1) / n), so an early call cannot take the
                             // whole cap and a share left unused passes on to later calls
  const int32_t *before_cnt; // [call][ld_before] the list lengths of the step's earlier calls
  int32_t ld_before;
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
// side (optional): pool work carried by the same launch as leading workgroups
int launch_score_decode(const uint8_t *q, const float *w, const uint8_t *k, const float *k_scale,
                        const int64_t *key_begin, const int32_t *key_len, int32_t n_q,
                        int32_t max_len, int32_t tok_lo, int32_t tok_hi, float *scores,
                        int64_t ld, const PrefetchArgs *pf, uint32_t *hist0, const struct SideWork *side,
                        const KeyPages *kp, hipStream_t st);

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
  int32_t *counters;      // [16]: 0 free slots, 2 threshold fine bin, 3 evictable slots below it
  uint32_t *fine;         // [32768] occupied, unprotected slots per priority bin (spread layout)
  uint32_t *coarse;       // [32768 words, 1024 used] the same, 32 fine bins per coarse bin
  uint32_t *prot;         // [ceil(n_gpu/32)] protection bitmap (slots holding a selected token)
  uint32_t *stage_a;      // [n_rows] (zeroed) misses found by the early lookup in the top-k split
  uint32_t *row_miss_cnt; // [n_rows]
  int32_t *row_miss_h;    // [n_rows * k] ordered misses of each request: host index
  int32_t *row_miss_j;    // [n_rows * k] ... column in the request's selection
  int32_t *row_miss_s;    // [n_rows * k] ... and staging row
  uint32_t *stage_b;      // [n_rows] misses found by the top-k finish (staging rows r*k + stage_a[r] ...)
  int32_t *stage_h;       // [n_rows * k] host index of each staging row r*k + i
  uint32_t *chunk_free;   // [n_chunks] free slots per 4096-slot chunk after the first evictions
  uint32_t *chunk_cand;   // [n_chunks] threshold-bin slots per chunk
  uint64_t *cand;         // [n_chunks * 4096] (priority key << 32 | slot), per chunk in slot order
  int32_t *miss_entry;    // [n_rows * k] entry (r*k + j) of the i-th miss
  int32_t *miss_stage;    // [n_rows * k] staging row of the i-th miss
  void *base;
  int32_t n_chunks;
  int64_t zero_words;
  uint32_t reserve;       // free slots the eviction leaves after allocation (prefetch room)
};
// Prefetch gather of one scoring range's candidates (one workgroup per request).
struct GatherArgs {
  const uint16_t *host_kv;
  uint16_t *gpu_kv;
  uint8_t *free_;
  int32_t *priority, *to_host, *host_to_gpu;
  const int32_t *status;
  int32_t n_gpu, n_host;
  const int64_t *key_begin;
  const int32_t *req_to_host;
  const int32_t *cand;        // [n_q, cap] token indices of one scoring range's candidates
  const int32_t *cand_cnt;    // [n_q]
  int32_t cap;
  const int32_t *free_list;   // free slots in ascending order
  int32_t *free_count;        // [2]: free slots listed, slots taken so far
  int32_t *n_prefetched;
  int32_t *st_free;           // optional pool-step statistics to keep current
  uint32_t *st_fine, *st_coarse;
  Stamp stamp;
};
GatherArgs make_gather_args(const echo_pool *pool, const int64_t *key_begin,
                            const int32_t *req_to_host, const int32_t *cand,
                            const int32_t *cand_cnt, int32_t cap, const int32_t *free_list,
                            int32_t *free_count, int32_t *n_prefetched, const PoolFastWs *pw,
                            Stamp stamp);

// Work that rides along in another kernel's launch as extra leading workgroups of 256 threads:
// n_stats pool-statistics chunks (every occupied slot), then n_gather prefetch-gather requests.
struct SideWork {
  PoolArgs P;
  PoolFastWs W;
  Stamp stamp;
  int32_t n_stats;
  int32_t n_gather;
  GatherArgs G;
};
void pool_fast_ws_layout(int32_t n_rows, int32_t k, int32_t n_gpu, void *base, PoolFastWs *w,
                         size_t *bytes);
size_t pool_fast_ws_bytes(int32_t n_rows, int32_t k, int32_t n_gpu);
// excl_prot: histogram only unprotected slots (after the lookup); otherwise all occupied
// slots, and the lookup subtracts what it protects.
int launch_pool_stats(const echo_pool *pool, const PoolFastWs &W, Stamp stamp, bool excl_prot,
                      hipStream_t st);
int launch_pool_lookup_rows(const echo_pool *pool, const PoolFastWs &W, const int32_t *idx,
                            const int64_t *key_begin, const int32_t *req_to_host, int64_t n_k,
                            int32_t n_rows, int32_t k, Stamp stamp, int32_t *topk_slot,
                            hipStream_t st);
// Missed rows copied into a staging area by workgroups riding along in the eviction launches.
struct StageArgs {
  const uint16_t *host_kv;
  uint16_t *stage;            // [n_rows * k][ROW]; NULL: no staging
};
// stage (optional): evict-1 and evict-2 also read their shares of the staging rows (the
// stage_cut_f / stage_cut_e split of r*k + [0, stage_a[r] + stage_b[r])) from host memory;
// the caller then runs launch_recall_scatter.
int launch_pool_evict(const echo_pool *pool, const PoolFastWs &W, const int32_t *idx, int32_t n_rows,
                      int32_t k, Stamp stamp, int32_t *topk_slot, int32_t *miss_host,
                      int32_t *miss_slot, int32_t *n_miss, uint16_t *stage, hipStream_t st);

int launch_pool_step(const echo_pool *pool, const int32_t *idx, const int64_t *key_begin,
                     const int32_t *req_to_host, int64_t n_k, int32_t n_rows, int32_t k,
                     Stamp stamp, int32_t *topk_slot, int32_t *miss_host, int32_t *miss_slot,
                     int32_t *n_miss, void *ws, size_t ws_bytes, hipStream_t st);

// Decode top-k: split (multi-workgroup) then finish (one workgroup per request).  With a pool,
// the split looks the sure selections up early (protection, priority-histogram removal,
// misses queued at staging rows r*k + [0, stage_a[r])), and the finish looks up the rest,
// lists every request's misses in order and queues its own misses after the split's; with a
// staging area the finish launch also reads the split's queued misses from host memory.  The
// pool workspace's zeroed region must be ready and its histograms must hold every occupied
// slot.
size_t topk_split_ws_bytes(int32_t n_rows, int32_t max_len, int32_t k);
// side (optional, with a pool): pool-statistics workgroups riding along (n_stats leading ones).
int launch_topk_split(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                      int32_t max_len, int32_t k, const uint32_t *hist0, void *split_ws,
                      const echo_pool *pool, const PoolFastWs *pw, const int64_t *key_begin,
                      const int32_t *req_to_host, Stamp stamp, const SideWork *side,
                      hipStream_t st);
int launch_topk_finish(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                       int32_t max_len, int32_t k, const uint32_t *hist0, void *split_ws,
                       int32_t *idx, const echo_pool *pool, const PoolFastWs *pw,
                       const int64_t *key_begin, const int32_t *req_to_host, Stamp stamp,
                       int32_t *topk_slot, bool early, uint16_t *stage, hipStream_t st);

int launch_recall_gather(const echo_pool *pool, const int32_t *miss_host, const int32_t *miss_slot,
                         const int32_t *n_miss, int32_t max_miss, hipStream_t st);
// Staged recall, second half: moves staged rows (stage[miss_stage[rank]]) to their allocated
// slots once allocation is done.
int launch_recall_scatter(const echo_pool *pool, const PoolFastWs &W, const int32_t *miss_host,
                          const int32_t *miss_slot, const int32_t *n_miss, int32_t max_miss,
                          const uint16_t *stage, hipStream_t st);

int launch_prefetch_threshold(const uint8_t *q, const float *w, const uint8_t *k,
                              const float *k_scale, const int64_t *key_begin,
                              const int32_t *key_len, int32_t n_q, int32_t max_len,
                              int32_t n_sample, float percentile, float *theta, const KeyPages *kp,
                              hipStream_t st);
int launch_prefetch_begin(const echo_pool *pool, int32_t *free_list, int32_t *free_count,
                          hipStream_t st);
// pw (optional): pool-step statistics (free count, priority histograms) updated for the slots
// this call fills (priority 0 relative to the step stamp)
int launch_prefetch_gather(const echo_pool *pool, const int64_t *key_begin,
                           const int32_t *req_to_host, const int32_t *cand,
                           const int32_t *cand_cnt, int32_t n_q, int32_t cap,
                           const int32_t *free_list, int32_t *free_count, int32_t *n_prefetched,
                           const PoolFastWs *pw, Stamp stamp, hipStream_t st);
// Scoring with the prefetch in the same kernel (score_fused.hip).  Workspace: counts and the
// ascending list of free slots, slice offsets and per-request totals.
struct FusedWs {
  int32_t *chunk_free;   // [ceil(n_gpu / 4096)] free slots per chunk
  int32_t *free_list;    // [n_gpu] ascending
  int32_t *slice_off;    // [n_q] first free_list entry of each request's places
  int32_t *counts;       // [2]: 0 length of free_list
  int32_t *demand;       // [n_q] tokens above the threshold and not resident
  int32_t *taken;        // [n_q] rows prefetched
  int32_t *cap_eff;      // [n_q] places of each request (its cap, scaled to the free slots)
  int32_t *claimed;      // [n_q] places claimed so far
};
size_t fused_ws_layout(int32_t n_q, int32_t n_gpu, void *base, FusedWs *w);
// Tokens per range (one workgroup each): pf_range when nonzero, else enough workgroups to put
// several on every CU.
int32_t fused_range(int64_t total_tokens, int32_t max_len, int32_t pf_range);
// hist0 (optional): the top-k digit-0 histograms, as launch_score_decode; stats (optional): the
// pool-step statistics, computed ahead of the kernel and kept current for the slots it fills;
// demand_out / taken_out (optional): the step's totals.
int launch_fused_prefetch(const uint8_t *q, const float *w, const uint8_t *k, const float *k_scale,
                          const int64_t *key_begin, const int32_t *key_len, int32_t n_q,
                          int32_t max_len, float *scores, int64_t ld, const float *theta,
                          const int32_t *req_to_host, const echo_pool *pool, int32_t cap,
                          int32_t cap_div, int32_t range, const FusedWs &Z, uint32_t *hist0,
                          const PoolFastWs *stats, Stamp stamp, int32_t *demand_out,
                          int32_t *taken_out, hipStream_t st);
int launch_zero_i32(int32_t *p, int64_t n, hipStream_t st);
int launch_zero2_i32(int32_t *p, int64_t n, int32_t *q, int64_t m, hipStream_t st);
int launch_sum_i32(const int32_t *v, int32_t n, int32_t *out, hipStream_t st);
// kth[r] = smallest score among row r's selections (NaN if none); theta (optional) updated by
// the EMA of the k-th score
int launch_kth_ema(const float *scores, int64_t ld, const int32_t *idx, int32_t n_rows, int32_t k,
                   float alpha, float *theta, float *kth, hipStream_t st);

}  // namespace echo
