/*
 * echo.h — C ABI of the MI355X (gfx950) DSA-indexer + top-k + pool-residency decode step.
 *
 * What the library computes follows the ECHO review page ("OSDI'26 | ECHO：稀疏 attention
 * 省了算力，却把 HBM 撑爆了"):
 *   §2    the lightning-indexer score of a cached token s for query t is the sum over the
 *         64 indexer heads of w[h,t] * ReLU(q[h,t] . k[s]) (d = 128, FP8 q/k, one key per
 *         token shared by all heads), followed by an exact top-k;
 *   §5.1  the pool metadata (free bitmap, per-slot eviction priority, fixed-length result
 *         buffer, the two slot<->host maps with an infinity sentinel);
 *   §5.2  the in-graph allocate / free / recall operations, with the recall copying rows
 *         straight out of host memory from a GPU kernel;
 *   §6.1  threshold prefetch during scoring, made lossless by the guaranteed recall;
 *   §6.3  the indexer kernel whose threshold test feeds a queue that a copy stage in the same
 *         kernel drains from host memory.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns every buffer and
 *     stream; no entry point allocates device memory, frees it, or synchronises, except
 *     echo_recall in ECHO_RECALL_MEMCPY mode and the echo_graph_* / echo_host_* helpers,
 *     which say so.  Everything else only enqueues work on the given stream(s), so it can be
 *     captured into a hipGraph.
 *   - Streams are hipStream_t passed as void* (NULL = the null stream).
 *   - FP8 = OCP E4M3FN bytes.  H = 64 heads and D = 128 are fixed.
 *   - Return codes: ECHO_OK, or a negative ECHO_E* code when an argument is rejected on the
 *     host (nothing is enqueued then) or a launch fails; echo_last_error() gives the text
 *     (thread-local).  Failures that depend on device data (pool exhausted, bad host index,
 *     duplicate host index) never trap: they OR bits into the pool's device status word.
 *   - "inf" in the pool maps is INT32_MAX (ECHO_INF).
 */
#ifndef ECHO_H
#define ECHO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ECHO_H_INDEX 64
#define ECHO_D_INDEX 128
#define ECHO_ROW_ELEMS 576 /* MLA latent row: 512 compressed + 64 RoPE values (bf16 bits) */
#define ECHO_INF 0x7FFFFFFF
#define ECHO_MAX_TOPK 4096
#define ECHO_FUSED_MAX_RANGE 8192      /* tokens per range of the fused prefetch, at most */
#define ECHO_FUSED_MAX_PER_RANGE 128   /* rows one range of the fused prefetch moves, at most */

/* Prefetch modes (echo_decode_args.prefetch). */
enum {
  ECHO_PREFETCH_OFF = 0,
  ECHO_PREFETCH_RANGED = 1, /* scoring split into n_chunks launches; each also gathers the
                               candidates of the range before it */
  ECHO_PREFETCH_FUSED = 2   /* one launch: scoring waves and a host-gather wave per workgroup
                               (echo_index_scores_fused) */
};

enum {
  ECHO_OK = 0,
  ECHO_EINVAL = -1,      /* bad argument or shape; nothing enqueued */
  ECHO_EUNSUPPORTED = -2,/* outside the supported range; nothing enqueued */
  ECHO_EHIP = -3,        /* a HIP call or kernel launch failed */
  ECHO_EWORKSPACE = -4   /* workspace smaller than the matching *_workspace_bytes() */
};

/* Sticky device status bits (pool->status). */
enum {
  ECHO_ST_EXHAUSTED = 1, /* the misses need more slots than free + evictable; pool untouched */
  ECHO_ST_BAD_HOST = 2,  /* a selected token maps to a host index outside [0, n_host); pool untouched */
  ECHO_ST_DUP_HOST = 4,  /* two selected misses share a host index (caller precondition broken);
                            pool state afterwards is unspecified */
  ECHO_ST_CACHE_FULL = 8 /* echo_decode_append: a request's key range is full; its token was not
                            appended */
};

/* Recall modes for echo_recall. */
enum {
  ECHO_RECALL_GATHER = 0, /* GPU kernel reads mapped pinned host memory; graph-capturable */
  ECHO_RECALL_MEMCPY = 1  /* host reads the miss list (synchronises the stream) and issues one
                             hipMemcpyAsync per row; NOT graph-capturable */
};

/*
 * GPU pool of one layer plus its host backup (§5.1).  All members are device pointers the
 * caller allocated; sizes: gpu_free/gpu_priority/gpu_to_host/indices_buf [n_gpu],
 * host_to_gpu [n_host], gpu_kv [n_gpu * 576], host_kv [n_host * 576], status [1].
 *   gpu_free      1 = slot free, 0 = occupied (GPUTokenFree)
 *   gpu_priority  eviction priority, lowest evicted first, -1 for a free slot (GPUTokenPriority)
 *   gpu_to_host   host index held by the slot, ECHO_INF when empty (GPUTokenToHost)
 *   host_to_gpu   slot holding the host index, ECHO_INF when not resident (HostTokenToGPU)
 *   indices_buf   fixed-length result list: slot given to the i-th miss, -1 after the last
 *                 (GPUIndicesBuffer); see echo_pool_lookup_alloc for how far it is written
 *   gpu_kv        latent rows of the slots, bf16 bits, 1152 bytes per row
 *   host_kv       the host backup: a DEVICE-ACCESSIBLE pointer to pinned, mapped host
 *                 memory (echo_host_alloc gives one), read by GPU kernels over the host link
 *   status        sticky ECHO_ST_* bits; cleared only by echo_pool_init / echo_status_clear
 */
typedef struct {
  int32_t n_gpu;
  int32_t n_host;
  uint8_t *gpu_free;
  int32_t *gpu_priority;
  int32_t *gpu_to_host;
  int32_t *host_to_gpu;
  int32_t *indices_buf;
  uint16_t *gpu_kv;
  const uint16_t *host_kv;
  int32_t *status;
} echo_pool;

/* Bytes of pool metadata: 4*n_host + 13*n_gpu (§5.1). */
size_t echo_pool_metadata_bytes(int32_t n_host, int32_t n_gpu);

/* Resets a pool to empty: free = 1, priority = -1, both maps = ECHO_INF, indices_buf = -1,
 * status = 0.  Rows are left as they are.  Enqueued on `stream`. */
int echo_pool_init(echo_pool *pool, void *stream);

/* Sets *status = 0 (enqueued). */
int echo_status_clear(int32_t *status, void *stream);

/*
 * Decode indexer scores (§2).  For every query (request) r in [0, n_q) and key s in
 * [0, key_len[r]):
 *     scores[r*ld + s] = sum_h w[r*64 + h] * ReLU(scale(s) * (q[r,h,:] . k[key_begin[r] + s, :]))
 * with scale(s) = k_scale[key_begin[r] + s] when k_scale != NULL, else 1 (k_scale dequantises
 * the FP8 key; the library applies it after the head sum, which is equal in exact arithmetic
 * because scale > 0).  Products are exact, sums are fp32.
 *   q        [n_q, 64, 128] FP8 bytes     w       [n_q, 64] fp32
 *   k        [n_k, 128] FP8 bytes, 128-byte rows; request r owns rows key_begin[r] .. +key_len[r]
 *   k_scale  [n_k] fp32 > 0, or NULL
 *   key_begin [n_q] int64, key_len [n_q] int32 (0 <= key_len[r] <= max_key_len)
 *   scores   [n_q, ld] fp32, ld >= max_key_len; entries s >= key_len[r] are not written.
 * Errors: EINVAL for n_q < 0, max_key_len < 0, ld < max_key_len or NULL pointers.
 * Device-side lengths above max_key_len are clamped to max_key_len (never read out of range).
 */
int echo_index_scores(const uint8_t *q, const float *w, const uint8_t *k, const float *k_scale,
                      const int64_t *key_begin, const int32_t *key_len, int32_t n_q,
                      int32_t max_key_len, float *scores, int64_t ld, void *stream);

/*
 * echo_index_scores over a paged key cache (§5.1: per-layer caches in fixed-size pages): the key
 * (and key scale) of token s of request r is row page_table[r * max_pages + s / page_size] *
 * page_size + s % page_size of k_pages (k_scale_pages; NULL = scale 1).  Same scores as
 * echo_index_scores over the same keys laid out contiguously.  page_size is a power of two in
 * [16, 65536]; max_pages * page_size >= max_key_len.  Errors as echo_index_scores, EINVAL for a
 * NULL page table or too few pages, EUNSUPPORTED for a bad page size.
 */
int echo_index_scores_paged(const uint8_t *q, const float *w, const uint8_t *k_pages,
                            const float *k_scale_pages, const int32_t *page_table,
                            int32_t page_size, int32_t max_pages, const int32_t *key_len,
                            int32_t n_q, int32_t max_key_len, float *scores, int64_t ld,
                            void *stream);

/*
 * echo_index_scores plus, in the same launch, the first radix pass of the exact top-k (§2):
 * hist[r*2048 + b] += the number of tokens s < key_len[r] of request r whose score's order key
 * has top 11 bits b, where the order key is ~key(score) and key(x) maps a float to uint32 in
 * increasing order (-0 counted as +0): bin 0 holds the highest scores.  hist [n_q, 2048] is
 * accumulated (zero it first).  The decode step's scoring launch is this one.  Errors as
 * echo_index_scores, and EINVAL for a NULL hist.
 */
int echo_index_scores_hist(const uint8_t *q, const float *w, const uint8_t *k,
                           const float *k_scale, const int64_t *key_begin, const int32_t *key_len,
                           int32_t n_q, int32_t max_key_len, float *scores, int64_t ld,
                           uint32_t *hist, void *stream);

/*
 * Threshold prefetch fused into scoring (§6.1).  Scores tokens [tok_lo, tok_hi) of every
 * request exactly as echo_index_scores does, and in addition lists scored tokens s with
 * score > theta[r] whose host index h = req_to_host[key_begin[r] + s] lies in [0, n_host) and is
 * not resident (host_to_gpu[h] == ECHO_INF) in this call's list cand[r*cap + j],
 * j < cand_cnt[r].  Every such token counts in the step-wide per-request counter total_cnt[r]
 * (the demand); listed tokens are bounded by cap_r = min(cap, ceil(key_len[r] / cap_div)) over
 * the step (the page's global prefetch counter, bounded in proportion to the context length).
 * Each workgroup (a run of at most 4096 tokens of one request) collects its qualifying tokens
 * (at most 1024 of them for listing; any further ones are counted only) and, at its end, adds
 * their number to total_cnt[r] and lists as many as cap_r still allows, reserving places in
 * the list with an atomic add on cand_cnt[r] and giving back those past the cap (so cand_cnt[r]
 * may run past the count while the call runs; after it, it is the number listed).  Which
 * qualifying tokens are listed, and in which order, depends on timing; the scores never do.  Because each call has its own list, a
 * consumer that waits for this call sees a complete list (echo_prefetch_gather).
 *   theta [n_q] fp32; req_to_host [n_k] int32; host_to_gpu [n_host]; cand [n_q, cap] int32;
 *   cand_cnt [n_q] (zeroed by the caller before this call); total_cnt [n_q] (zeroed once per
 *   step).
 */
int echo_index_scores_prefetch(const uint8_t *q, const float *w, const uint8_t *k,
                               const float *k_scale, const int64_t *key_begin,
                               const int32_t *key_len, int32_t n_q, int32_t max_key_len,
                               int32_t tok_lo, int32_t tok_hi, float *scores, int64_t ld,
                               const float *theta, const int32_t *req_to_host,
                               const int32_t *host_to_gpu, int32_t n_host, int32_t *cand,
                               int32_t *cand_cnt, int32_t *total_cnt, int32_t cap,
                               int32_t cap_div, void *stream);

/*
 * Scoring and threshold prefetch in one kernel (§6.3, with the §6.1 threshold and the §5.2
 * allocate and zero-copy row reads).  Scores every request exactly as echo_index_scores does
 * (same values), and moves rows of tokens scoring above theta[r] into free GPU slots while the
 * later keys are still being scored.
 *   Ranges.  Request r's tokens are cut into ranges of `range` tokens (one workgroup each;
 *   range = 0 picks one; else a multiple of 128 in [128, ECHO_FUSED_MAX_RANGE]).
 *   Which rows.  The tokens s with score > theta[r] (fp32, strict; NaN never passes) whose host
 *   index h = req_to_host[key_begin[r] + s] is in [0, n_host) and not resident
 *   (host_to_gpu[h] == ECHO_INF when the call starts) qualify.  Each range asks for places for
 *   its first ECHO_FUSED_MAX_PER_RANGE qualifying tokens in token order (its candidates).
 *   Cap and places.  Request r may move c_r = min(cap, ceil(key_len[r] / cap_div), n_gpu) rows,
 *   scaled to floor(c_r * F / C) when the caps add up to C > F, the pool's free slots at the
 *   start.  Those free slots, ascending, form a list; request r owns c_r entries of it, after
 *   those of requests < r.  Its ranges claim them first come, first served (one counter per
 *   request): min(#candidates, c_r) rows move, each range's a token-order prefix of its
 *   candidates in ascending slots, into the request's first entries.  So when a request's
 *   candidates fit its cap, all of them move; which of the request's slots each one gets
 *   depends on timing.
 *   Each moved token: free = 0, gpu_to_host = h, host_to_gpu[h] = slot, priority 0, and its
 *   row copied from host_kv.  Nothing is evicted; nothing moves when the status word is
 *   nonzero.
 *   Outputs: *n_prefetched = rows moved; *demand (or NULL) = qualifying tokens, before caps.
 *   Workspace: echo_fused_workspace_bytes(n_q, pool->n_gpu) bytes.  Host indices are unique
 *   across requests (caller precondition).
 * Errors: EINVAL for negative sizes, ld < max_key_len, cap < 0, cap_div < 1, NULL pointers or
 * an incomplete pool; EUNSUPPORTED for n_q > 65535, max_key_len or n_gpu above 2^22, or a bad
 * range; EWORKSPACE for a short workspace.
 */
size_t echo_fused_workspace_bytes(int32_t n_q, int32_t n_gpu);
int echo_index_scores_fused(const uint8_t *q, const float *w, const uint8_t *k,
                            const float *k_scale, const int64_t *key_begin,
                            const int32_t *key_len, int32_t n_q, int32_t max_key_len,
                            float *scores, int64_t ld, const float *theta,
                            const int32_t *req_to_host, const echo_pool *pool, int32_t cap,
                            int32_t cap_div, int32_t range, int32_t *n_prefetched,
                            int32_t *demand, void *ws, size_t ws_bytes, void *stream);

/*
 * Per-request prefetch threshold: theta[r] = the nearest-rank `percentile` of the scores of
 * request r at the n_sample positions floor(i * L_r / n_sample), i < n_sample, with
 * L_r = min(key_len[r], max_key_len) (the stand-in for the page's per-layer EMA prediction of
 * the k-th score, §6.1, on a single step with no history).  theta[r] = +inf when L_r <= 0.
 * n_sample must be a power of two in [64, 4096].  Computes the sampled scores itself from q, w,
 * k, k_scale (as echo_index_scores does).  Errors: EINVAL for negative n_q or max_key_len, a
 * percentile outside (0, 100] or NULL pointers; EUNSUPPORTED for n_sample outside the range or
 * n_q > 65535.
 */
int echo_prefetch_threshold(const uint8_t *q, const float *w, const uint8_t *k,
                            const float *k_scale, const int64_t *key_begin,
                            const int32_t *key_len, int32_t n_q, int32_t max_key_len,
                            int32_t n_sample, float percentile, float *theta, void *stream);

/*
 * Prefill (causal) indexer scores (§3.4: quadratic in the context).  Query rows t in
 * [0, n_q) sit at absolute positions q_pos0 + t and see keys s in [0, min(n_k, q_pos0+t+1)):
 *     scores[t*ld + s] = sum_h w[t*64+h] * ReLU(q[t,h,:] . k[s,:])
 *   q [n_q, 64, 128] FP8; w [n_q, 64] fp32; k [n_k, 128] FP8; scores [n_q, ld] fp32,
 *   ld >= n_k; entries past a row's causal length are not written.
 */
int echo_index_scores_prefill(const uint8_t *q, const float *w, const uint8_t *k, int32_t n_q,
                              int32_t n_k, int32_t q_pos0, float *scores, int64_t ld,
                              void *stream);

/*
 * Exact top-k per row (§2).  Row r holds len[r] scores at scores[r*ld ...].  Selects the
 * min(k, len[r]) highest scores; ties go to the lower index; -0.0 equals +0.0.  Writes
 * idx[r*k + j], the selected token indices in ascending order, -1 padded to k.
 * NaN scores are outside the contract.  1 <= k <= ECHO_MAX_TOPK.
 *   ws: device workspace of at least echo_topk_workspace_bytes(n_rows, max_len) bytes.
 * len[r] above max_len is clamped to max_len.
 */
size_t echo_topk_workspace_bytes(int32_t n_rows, int32_t max_len);
int echo_topk(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
              int32_t max_len, int32_t k, int32_t *idx, void *ws, size_t ws_bytes,
              void *stream);

/*
 * Approximate top-k subset per row for the inter-query prefetch of a chunked prefill (§6.2).
 * Every score of row r (scores[r*ld + s], s < len[r]) is shifted, x = fl32(score - shift), and
 * mapped by the top 8 bits of its order key (sign-flipped, -0 as +0) to one of 256 bins.  The
 * highest bins whose total stays <= k are taken whole and the next bin down is the threshold
 * bin.  subset[r*k + j] lists the tokens of the taken bins in ascending order, -1 padded to k;
 * subset_cnt[r] is their number (<= k, and > k - the threshold bin's size when there is one);
 * thr_cnt[r] (optional) is the threshold bin's size (0 when every bin fits).  The subset lies
 * inside the row's exact top-k.  shift [1] is a device float, the prediction of the k-th score
 * (NULL or NaN = 0: no prediction yet).  len[r] above max_len is clamped; ld >= max_len.
 * 1 <= k <= ECHO_MAX_TOPK.  ECHO_EINVAL for negative sizes, ld < max_len or NULL pointers
 * (thr_cnt and shift may be NULL); ECHO_EUNSUPPORTED for k outside the range.
 */
int echo_topk_subset(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                     int32_t max_len, int32_t k, const float *shift, int32_t *subset,
                     int32_t *subset_cnt, int32_t *thr_cnt, void *stream);

/*
 * Union of index lists (§6.2: a query block's prefetch set is the union of its rows' subsets, and
 * its guaranteed recall covers the union of its rows' exact top-k).  Entries of idx [n_rows, k]
 * in [0, n_keys) are collected (others, -1 included, are ignored) and listed in ascending order
 * in segments of 4096 consecutive keys: out[s*4096 + j] for the union's keys in
 * [4096 s, 4096 s + 4096), -1 padded; out_cnt[s] their number; n_seg = ceil(n_keys / 4096)
 * (1 when n_keys = 0).  The segments are 4096-wide selection rows with key_begin 0 for
 * echo_pool_lookup_alloc (k = 4096) and candidate rows for echo_prefetch_gather (cap = 4096).
 * ws: echo_union_workspace_bytes(n_keys) bytes (a bitmap, cleared by the call).  ECHO_EINVAL
 * for negative sizes or NULL pointers, ECHO_EWORKSPACE for a short workspace,
 * ECHO_EUNSUPPORTED above 2^30 keys.
 */
size_t echo_union_workspace_bytes(int32_t n_keys);
int echo_union_rows(const int32_t *idx, int32_t n_rows, int32_t k, int32_t n_keys, int32_t *out,
                    int32_t *out_cnt, void *ws, size_t ws_bytes, void *stream);

/*
 * k-th score and its EMA (§6.1, §6.2): for each row r, kth[r] = the smallest score among the
 * selected tokens idx[r*k + j] >= 0 (NaN when there is none), and theta[r] = kth[r] if theta[r]
 * is NaN, else fmaf(alpha, theta[r], (1 - alpha) * kth[r]); a row with no selection keeps theta.
 * Either output may be NULL (not both).  0 <= alpha <= 1.
 */
int echo_threshold_ema(const float *scores, int64_t ld, const int32_t *idx, int32_t n_rows,
                       int32_t k, float alpha, float *theta, float *kth, void *stream);

/*
 * Residency lookup + eviction + allocation for the selected tokens (§5.2 free/allocate and
 * the lookup half of recall), without the row copy.  For the entries idx[r*k + j] >= 0 taken
 * in (r, j) order: h = req_to_host[key_begin[r] + idx]; hit iff host_to_gpu[h] != ECHO_INF.
 *   - every hit slot is protected for this call (a bitmap in the workspace);
 *   - need = max(0, n_miss - #free); the `need` unprotected occupied slots with the smallest
 *     (priority, slot index) are evicted: free = 1, priority = -1, both maps = ECHO_INF; their
 *     rows are not touched (the host holds the backup);
 *   - the i-th miss gets the i-th free slot in ascending slot order: free = 0, maps set,
 *     priority = step_id; miss_host[i] = h, miss_slot[i] = slot, indices_buf[i] = slot;
 *     miss_host/miss_slot entries past n_miss and indices_buf entries [n_miss,
 *     min(n_gpu, n_rows*k)) are -1;
 *   - every selected slot's priority = step_id; topk_slot[r*k + j] = its slot (-1 where
 *     idx is -1); *n_miss = number of misses.
 * req_to_host has n_k entries; a token index key_begin[r] + idx outside [0, n_k), a host index
 * outside [0, n_host) or a HostTokenToGPU entry outside [0, n_gpu) sets ECHO_ST_BAD_HOST.
 * On ECHO_ST_EXHAUSTED or ECHO_ST_BAD_HOST the pool is left untouched and topk_slot,
 * miss_*, n_miss are unspecified.  Rows of missed tokens still have to be copied by
 * echo_recall.  step_id must exceed every priority already in the pool for the policy to be
 * least-recently-selected-first (not checked).  1 <= k <= ECHO_MAX_TOPK; n_gpu <= 2^22.
 *   ws: device workspace of at least echo_pool_workspace_bytes(n_rows, k, pool->n_gpu).
 */
size_t echo_pool_workspace_bytes(int32_t n_rows, int32_t k, int32_t n_gpu);
int echo_pool_lookup_alloc(const echo_pool *pool, const int32_t *idx, const int64_t *key_begin,
                           const int32_t *req_to_host, int64_t n_k, int32_t n_rows, int32_t k,
                           int32_t step_id, int32_t *topk_slot, int32_t *miss_host,
                           int32_t *miss_slot, int32_t *n_miss, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * echo_pool_lookup_alloc without a workspace argument, for callers that cannot allocate
 * (code under hipGraph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and errors as echo_pool_lookup_alloc; its workspace is a fixed device array
 * of ECHO_STATIC_SCRATCH_BYTES inside the library, one per GPU, held until the process ends.
 * Sizes whose echo_pool_workspace_bytes(n_rows, k, pool->n_gpu) exceeds that are rejected with
 * ECHO_EUNSUPPORTED (nothing enqueued).  Allocates nothing; launch on a stream of the current
 * device.  Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (other streams, other threads) race and give undefined results.  Each call clears what must
 * start at zero itself.
 */
#define ECHO_STATIC_SCRATCH_BYTES (16u << 20)
int echo_pool_lookup_alloc_static(const echo_pool *pool, const int32_t *idx,
                                  const int64_t *key_begin, const int32_t *req_to_host, int64_t n_k,
                                  int32_t n_rows, int32_t k, int32_t step_id, int32_t *topk_slot,
                                  int32_t *miss_host, int32_t *miss_slot, int32_t *n_miss,
                                  void *stream);

/*
 * Recall (§5.2): gpu_kv[miss_slot[i]] = host_kv[miss_host[i]] bitwise (1152 bytes) for
 * i < *n_miss (n_miss is read on the device; max_miss bounds it).
 *   ECHO_RECALL_GATHER: one kernel reads the rows straight from mapped pinned host memory.
 *   ECHO_RECALL_MEMCPY: synchronises `stream`, reads n_miss and the lists to the host and
 *     issues one hipMemcpyAsync (host -> device) per row on `stream`; returns after enqueueing.
 * Skipped entirely when the pool status word is nonzero.  ECHO_EINVAL for a pool with a
 * NULL gpu_kv, host_kv, host_to_gpu or status, or with n_gpu or n_host below 1.
 */
int echo_recall(const echo_pool *pool, const int32_t *miss_host, const int32_t *miss_slot,
                const int32_t *n_miss, int32_t max_miss, int32_t mode, void *stream);

/*
 * Prefetch side of the overlap (§6.1 with the §5.2 allocate and UVM copy).
 * echo_prefetch_begin lists the pool's free slots (in no particular order) into free_list
 * [n_gpu] and sets free_count[0] = their number, free_count[1] = 0 (taken so far).
 * echo_prefetch_gather takes the candidates of one echo_index_scores_prefetch call (cand,
 * cand_cnt), gives each a slot from free_list (counter free_count[1]; never evicts: candidates
 * beyond the free slots are dropped), sets both maps, gives the slot priority 0 (first to go
 * when space is short later), copies the row from host memory, and adds the number of rows it
 * moved to *n_prefetched.  Skipped when the pool status word is nonzero.  Both reject a pool
 * with NULL members it uses or n_gpu (n_host) below 1 with ECHO_EINVAL.
 */
int echo_prefetch_begin(const echo_pool *pool, int32_t *free_list, int32_t *free_count,
                        void *stream);
int echo_prefetch_gather(const echo_pool *pool, const int64_t *key_begin,
                         const int32_t *req_to_host, const int32_t *cand,
                         const int32_t *cand_cnt, int32_t n_q, int32_t cap,
                         const int32_t *free_list, int32_t *free_count, int32_t *n_prefetched,
                         void *stream);

/*
 * The whole decode step (§4): scores -> [threshold prefetch] -> exact top-k -> lookup /
 * evict / allocate -> recall -> priorities.  Pure enqueue on `main_stream`, so the call can be
 * captured into one hipGraph (echo_graph_capture_decode).  Work that overlaps the critical
 * path (the pool's priority histogram, prefetch gathers, reading missed rows from host memory
 * into a staging area of the workspace) rides along as extra workgroups of the same launches.
 * Prefetch (§6.1): ECHO_PREFETCH_RANGED scores in n_chunks launches, each of which also gathers
 * the candidates of the range before it (which candidates win the cap depends on timing);
 * ECHO_PREFETCH_FUSED scores in one launch with a host-gather wave per workgroup, with the
 * rows and slots of echo_index_scores_fused (§6.3).  Either way the
 * threshold is theta_ema when given, else the sample percentile, and the selection and the
 * selected rows are those of the step without prefetch.  With prefetch on, the rest of the
 * pool is not reproducible from run to run: which unselected candidates move, the free slot
 * each takes, and so the slots the guaranteed recall then finds free and the contents of
 * topk_slot / miss_slot / indices_buf, depend on the order in which workgroups finish.  The
 * pool invariants (maps a bijection, every resident row equal to its host row) always hold.
 * `side_stream` is reserved and ignored (pass NULL or main_stream).  Workspace:
 * echo_decode_workspace_bytes(a, pool->n_gpu) bytes (it includes n_rows * topk staged rows of
 * ECHO_ROW_ELEMS bf16 values).
 */
typedef struct {
  const uint8_t *q;          /* [n_rows, 64, 128] FP8 */
  const float *w;            /* [n_rows, 64] */
  const uint8_t *k;          /* [n_k, 128] FP8 */
  const float *k_scale;      /* [n_k] or NULL */
  const int64_t *key_begin;  /* [n_rows] */
  const int32_t *key_len;    /* [n_rows] */
  const int32_t *req_to_host;/* [n_k] host index of every cached token */
  int32_t n_rows;
  int32_t max_key_len;
  int32_t topk;
  int32_t step_id;
  /* prefetch: ECHO_PREFETCH_OFF, _RANGED or _FUSED */
  int32_t prefetch;
  int32_t n_chunks;          /* RANGED: scoring split into this many token ranges (1..16); ranges
                                0..c together list at most floor(cap_r (c+1) / n) of a request's
                                cap (a share left unused passes on), so the gathers spread over
                                the later launches */
  int32_t n_sample;          /* threshold sample size (power of two, 64..4096) */
  float percentile;          /* threshold percentile, e.g. 95 */
  int32_t cap;               /* per-request candidate cap bound */
  int32_t cap_div;           /* cap_r = min(cap, ceil(L_r / cap_div)) */
  /* EMA threshold (§6.1; off when theta_ema == NULL).  theta_ema [n_rows] is the caller's
     per-request estimate of the k-th largest score, kept from step to step.  With prefetch on
     it replaces the sample percentile as the threshold (NaN = no estimate yet: nothing is
     prefetched).  At the end of the step it is updated from this step's k-th score kth (the
     smallest selected score): theta = kth if theta is NaN, else
     fmaf(ema_alpha, theta, (1 - ema_alpha) * kth); a request with no selection keeps it. */
  float *theta_ema;
  float ema_alpha;           /* the page uses 0.5 */
  /* [1] or NULL: when given, the step stamp is read on the device from *step_dev instead of
     step_id, so that one captured graph can serve every step (echo_step_advance moves it on) */
  const int32_t *step_dev;
  /* Free slots the guaranteed recall leaves after its allocation, as room for the next step's
     prefetch (which only takes free slots): it evicts further down the same (priority, slot)
     order until reserve_free slots stay free, as far as unprotected slots allow.  0 = evict
     only what the misses need.  0 <= reserve_free <= n_gpu. */
  int32_t reserve_free;
  /* FUSED: tokens per range (0 = the library picks; else as echo_index_scores_fused) */
  int32_t pf_range;
  /* Paged indexer-K cache (§5.1: the caches are kept per layer in fixed-size pages; NULL = the
     contiguous layout).  With a page table, token s of request r has its key at row
     k_page_table[r * k_max_pages + s / k_page_size] * k_page_size + s % k_page_size of k (and
     k_scale); key_begin then only offsets req_to_host.  k_page_size is a power of two in
     [16, 65536], k_max_pages * k_page_size >= max_key_len.  Not with ECHO_PREFETCH_FUSED
     (EUNSUPPORTED). */
  const int32_t *k_page_table;
  int32_t k_page_size;
  int32_t k_max_pages;
} echo_decode_args;

typedef struct {             /* device outputs of one step */
  float *scores;             /* [n_rows, max_key_len] */
  int32_t *topk_idx;         /* [n_rows, topk] */
  int32_t *topk_slot;        /* [n_rows, topk] */
  int32_t *miss_host;        /* [n_rows * topk] */
  int32_t *miss_slot;        /* [n_rows * topk] */
  int32_t *counters;         /* [8]: 0 n_miss (guaranteed recall), 1 prefetch demand (tokens
                                above threshold and not resident, summed over requests),
                                2 rows prefetched, 3..7 reserved (zero) */
  float *kth;                /* [n_rows] or NULL: smallest selected score per request (the k-th
                                largest when key_len >= topk; NaN when nothing is selected) */
} echo_decode_out;

size_t echo_decode_workspace_bytes(const echo_decode_args *a, int32_t n_gpu);
int echo_decode_select(const echo_decode_args *a, const echo_pool *pool,
                       const echo_decode_out *out, void *ws, size_t ws_bytes, void *main_stream,
                       void *side_stream);

/*
 * One new token per request, before its query is scored (§2: a token's latent row is backed up
 * to host memory when it is generated, so eviction never moves data; §5.2: allocate serves
 * newly generated KV as well as recalled tokens).  For every request r with
 * p = key_len[r] < capacity and key_begin[r] + p < n_k:
 *   k[key_begin[r] + p] = new_k[r] (128 FP8 bytes); k_scale[...] = new_scale[r] when given;
 *   req_to_host[key_begin[r] + p] = new_host[r]; key_len[r] = p + 1 (on the device);
 *   host_kv_w[new_host[r]] = new_kv[r] (576 bf16 values written through the host link);
 * a request at capacity appends nothing and sets ECHO_ST_CACHE_FULL.  Then the appended tokens,
 * in request order, get GPU slots exactly as misses of echo_pool_lookup_alloc with k = 1
 * (nothing protected, eviction of the lowest (priority, slot) when no slot is free, priority
 * step_id), and their rows are copied from new_kv into those slots.  new_slot[r] receives the
 * slot (-1 for a request that appended nothing); it is unspecified when the pool status word
 * is nonzero afterwards.  new_host[r] must lie in [0, n_host), be distinct and not be resident
 * (ECHO_ST_BAD_HOST / ECHO_ST_DUP_HOST otherwise; the pool is then left untouched, the key
 * cache and host rows are still written).  Pure enqueue on `stream`; workspace:
 * echo_append_workspace_bytes(n_rows, pool->n_gpu).  Argument errors (nothing enqueued):
 * ECHO_EINVAL for NULL inputs, an incomplete pool, capacity or n_k below 1, or k_scale and
 * new_scale not both given or both NULL; ECHO_EUNSUPPORTED for n_rows outside [1, 65535] or more
 * than 2^22 GPU slots; ECHO_EWORKSPACE for a short workspace.
 */
typedef struct {
  int32_t n_rows;
  int32_t capacity;          /* key rows reserved per request (key_len never exceeds it) */
  int64_t n_k;               /* rows of k, k_scale and req_to_host */
  const uint8_t *new_k;      /* [n_rows, 128] FP8 */
  const float *new_scale;    /* [n_rows], or NULL when k_scale is NULL */
  const uint16_t *new_kv;    /* [n_rows, 576] bf16 bits, device memory */
  const int32_t *new_host;   /* [n_rows] host row of each new token */
  uint8_t *k;                /* [n_k, 128] the indexer K cache */
  float *k_scale;            /* [n_k] or NULL */
  const int64_t *key_begin;  /* [n_rows] */
  int32_t *key_len;          /* [n_rows], incremented */
  int32_t *req_to_host;      /* [n_k] */
  uint16_t *host_kv_w;       /* WRITABLE device-mapped pointer to the pool's host backup
                                (the same memory as echo_pool.host_kv) */
  int32_t step_id;
  const int32_t *step_dev;   /* [1] or NULL: the step stamp read on the device (as in
                                echo_decode_args) */
} echo_append_args;
size_t echo_append_workspace_bytes(int32_t n_rows, int32_t n_gpu);
int echo_decode_append(const echo_append_args *a, const echo_pool *pool, int32_t *new_slot,
                       void *ws, size_t ws_bytes, void *stream);

/* *step_dev += 1, enqueued on `stream` (one thread).  With the stamp on the device, a captured
 * sequence echo_step_advance -> echo_decode_append -> echo_decode_select is one whole decode
 * step that can be replayed for every step (the caller refreshes the step's query and new
 * tokens in the same device buffers between replays).  ECHO_EINVAL for NULL. */
int echo_step_advance(int32_t *step_dev, void *stream);

/* Graph helpers (host side; they create HIP objects).  Capture one echo_decode_select into a
 * hipGraph on `main_stream`, instantiate it, and replay it.  The graph
 * reads and writes the buffers that were passed at capture time. */
typedef struct echo_graph_s *echo_graph;
int echo_graph_capture_decode(const echo_decode_args *a, const echo_pool *pool,
                              const echo_decode_out *out, void *ws, size_t ws_bytes,
                              void *main_stream, void *side_stream, echo_graph *graph);
int echo_graph_launch(echo_graph graph, void *stream);
int echo_graph_destroy(echo_graph graph);

/* Capture of any sequence of echo_* calls enqueued on `stream` between the two calls (host side;
 * they create HIP objects): echo_graph_begin starts a stream capture, echo_graph_end ends it and
 * instantiates the graph (launch with echo_graph_launch, free with echo_graph_destroy).  Calls
 * that synchronise (echo_recall in ECHO_RECALL_MEMCPY mode) cannot be captured.  A failed
 * echo_graph_end leaves *graph NULL and the stream no longer capturing. */
int echo_graph_begin(void *stream);
int echo_graph_end(void *stream, echo_graph *graph);

/* Pinned, device-mapped host memory for the host backup (hipHostMalloc, mapped; coherent when
 * `coherent` != 0).  *host receives the host pointer, *dev the device-side pointer to pass as
 * echo_pool.host_kv.  Free with echo_host_free. */
int echo_host_alloc(size_t bytes, int coherent, void **host, void **dev);
int echo_host_free(void *host);

/* Text of the last error on this thread ("" if none). */
const char *echo_last_error(void);

/* Library version string. */
const char *echo_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ECHO_H */
