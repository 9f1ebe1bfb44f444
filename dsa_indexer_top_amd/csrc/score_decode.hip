// Decode lightning-indexer scores on gfx950 (ECHO review page, §2: score of cached token s =
// sum over the 64 indexer heads of w[h] * ReLU(q[h] . k[s]); FP8 q/k, one 128-byte key per
// token shared by every head).  Optional fused threshold prefetch (§6.1): tokens scoring above
// a per-request threshold that are not resident are appended to a capped candidate list.
//
// Work split: grid (token range, request).  A workgroup of 4 waves streams its token range in
// chunks of 256 tokens (32 KB).  Each thread fetches 8 x 16 B of the chunk with fully
// coalesced global loads (the next chunk is fetched into registers while the current one is
// computed), and writes them into an LDS double buffer whose 16-byte segments are XOR-swizzled
// by token so the MFMA-layout reads below are bank-conflict free.  Each wave scores one
// 64-token group of the chunk.
//
// Contraction (score_tile.cuh): v_mfma_f32_16x16x128_f8f6f4, A = q of 16 heads held in VGPRs
// for the whole kernel, B = k of 16 tokens read from LDS; four MFMAs cover the 64 heads (issued
// before their epilogue) and the ReLU * w head reduction is 16 FMAs per lane.  The four tiles'
// partials of a group are summed over the lane groups by a butterfly of three lane swaps, after
// which every lane holds one token's score, so the whole wave writes 64 scores at once.
// Measured on MI355X at 8 x 65536 tokens against the former 128-token stages with one
// cross-lane sum per tile: 12.6 us instead of 13.1 us for the scoring alone.
//
// Prefetch candidates: each call appends to its own list (cand, cand_cnt), so a later kernel
// sees a complete list, and the calls of a step share each request's cap cumulatively.  A
// workgroup collects its over-threshold tokens in LDS (one LDS atomic per wave and chunk) and
// looks their residency up only at its end, with all of those loads in flight together, so the
// streaming loop never waits on a lookup (measured on MI355X at 64 x 131072 tokens: per-chunk
// lookups made each ranged scoring launch about twice as long as plain scoring).  The eligible
// ones are then published with one atomic for the demand and one atomic add that reserves
// places on the call's list, so the step's counters see one update per workgroup instead of
// one per token.
//
// Side work (SIDE): the launch may carry extra leading workgroups that do independent pool
// work (priority statistics, a previous range's prefetch gather) while the scoring workgroups
// stream keys; the grid is one-dimensional and block b >= n_side scores (token block
// (b - n_side) % gx of request (b - n_side) / gx).
#include "internal.hpp"
#include "pool_common.cuh"
#include "score_tile.cuh"

namespace echo {

constexpr int SD_THREADS = 256;
constexpr int SD_CHUNK = 256;                                    // tokens per LDS stage
constexpr int SD_UNITS = SD_CHUNK * D / 16;                      // 16-byte units per chunk
constexpr int SD_LOADS = SD_UNITS / SD_THREADS;                  // per thread per chunk = 8
static_assert(SD_CHUNK == 64 * (SD_THREADS / 64), "one 64-token group per wave per chunk");

ECHO_DEV int swz(int tok, int seg) { return tok * 128 + ((seg ^ ((tok >> 1) & 7)) << 4); }

constexpr int SD_SCORE_WORDS = 2 * SD_CHUNK * D / 4;               // the LDS double buffer
constexpr int SD_PF_OVER = 1024;         // over-threshold tokens a workgroup holds for lookup
constexpr int SD_PF_PER = SD_PF_OVER / SD_THREADS;
// LDS words of the prefetch list: over-threshold tokens, then their count, the count of
// eligible tokens past the list, the compacted count and the claim (count, base)
constexpr int SD_PF_WORDS = SD_PF_OVER + 5;

template <bool HAS_SCALE, bool PREFETCH, bool HIST, bool SIDE, bool PAGED>
__global__ __launch_bounds__(SD_THREADS, 2) void score_decode_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ w, const uint8_t *__restrict__ k,
    const float *__restrict__ k_scale, const int64_t *__restrict__ key_begin,
    const int32_t *__restrict__ key_len, int32_t max_len, int32_t tok_lo, int32_t tok_hi,
    int32_t tokens_per_wg, int32_t gx, float *__restrict__ scores, int64_t ld, PrefetchArgs pf,
    uint32_t *__restrict__ hist0, SideWork side, KeyPages kp) {
  constexpr int WORDS = SD_SCORE_WORDS + (HIST ? 2048 : 0);
  constexpr int ALL = SIDE && SIDE_LDS_WORDS > WORDS ? SIDE_LDS_WORDS : WORDS;
  __shared__ __attribute__((aligned(16))) uint32_t smem[ALL];
  __shared__ int32_t pf_list[PREFETCH ? SD_PF_WORDS : 1];
  int b = blockIdx.x;
  if constexpr (SIDE) {
    if (side_work(side, b, smem)) return;
    b -= side.n_stats + side.n_gather;
  }
  const int r = b / gx;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int j = l & 15, g = l >> 4;
  const int tsel = group_tile_sel();              // the tile whose score this lane ends up with
  // the request's length and key offset, and its q operand, all requested before the first
  // wait, so their latencies overlap (the q loads of a workgroup with no tokens are wasted)
  const int32_t len_r = key_len[r];
  const int64_t kb = key_begin ? key_begin[r] : 0;   // no key_begin for a paged key cache
  QOperand qo;
  load_q_operand(q, w, r, qo);
  const int32_t L = min(max(len_r, 0), max_len);
  const int32_t hi = min(L, tok_hi);
  const int32_t t_begin = tok_lo + (b % gx) * tokens_per_wg;
  if (t_begin >= hi) return;
  const int32_t t_end = min(hi, t_begin + tokens_per_wg);
  float *__restrict__ srow = scores + static_cast<int64_t>(r) * ld;

  uint8_t (*lds)[SD_CHUNK * D] = reinterpret_cast<uint8_t (*)[SD_CHUNK * D]>(smem);
  uint32_t *hl = smem + SD_SCORE_WORDS;

  float theta = 0.f;
  int32_t cap_r = 0;
  if constexpr (PREFETCH) {
    theta = pf.theta[r];
    cap_r = min(pf.cap, (L + pf.cap_div - 1) / pf.cap_div);
  }

  int4 pre[SD_LOADS];
  float pre_sc = 1.f;                  // the key scale of the token this lane scores, one chunk ahead
  auto fetch = [&](int32_t c0) {
#pragma unroll
    for (int m = 0; m < SD_LOADS; ++m) {
      const int e = tid + m * SD_THREADS;
      const int32_t t = c0 + (e >> 3);
      if (t < t_end)
        pre[m] = *reinterpret_cast<const int4 *>(k + (PAGED ? key_row(kp, r, kb, t) : kb + t) * D +
                                                 ((e & 7) << 4));
      else
        pre[m] = int4{0, 0, 0, 0};
    }
    if constexpr (HAS_SCALE) {
      // fetched with the keys, so the multiply never waits on a load of its own (a wait there
      // would also wait for the next chunk's keys)
      const int32_t t = c0 + wv * 64 + tsel * 16 + j;
      pre_sc = t < t_end ? k_scale[PAGED ? key_row(kp, r, kb, t) : kb + t] : 1.f;
    }
  };

  if constexpr (HIST)
    for (int b = threadIdx.x; b < 2048; b += SD_THREADS) hl[b] = 0;   // ordered by the first barrier
  if constexpr (PREFETCH)
    if (threadIdx.x < 3) pf_list[SD_PF_OVER + threadIdx.x] = 0;       // ordered by the first barrier
  fetch(t_begin);
  int buf = 0;
  for (int32_t c0 = t_begin; c0 < t_end; c0 += SD_CHUNK) {
    uint8_t *sb = lds[buf];
#pragma unroll
    for (int m = 0; m < SD_LOADS; ++m) {
      const int e = tid + m * SD_THREADS;
      *reinterpret_cast<int4 *>(sb + swz(e >> 3, e & 7)) = pre[m];
    }
    const float sc = pre_sc;
    __syncthreads();
    if (c0 + SD_CHUNK < t_end) fetch(c0 + SD_CHUNK);

    float part[4];
#pragma unroll
    for (int tile = 0; tile < 4; ++tile) {
      const int tt = wv * 64 + tile * 16 + j;
      const int4 b0 = *reinterpret_cast<const int4 *>(sb + swz(tt, 2 * g));
      const int4 b1 = *reinterpret_cast<const int4 *>(sb + swz(tt, 2 * g + 1));
      part[tile] = score_tile_partial_mf(qo, v8i{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w});
    }
    float s_out = butterfly4(part);
    const int32_t t_out = c0 + wv * 64 + tsel * 16 + j;
    const bool writer = t_out < t_end;
    if (writer) {
      if constexpr (HAS_SCALE) s_out *= sc;
      srow[t_out] = s_out;
    }
    if constexpr (PREFETCH) {
      // over-threshold tokens take consecutive places of the workgroup's LDS list; their
      // residency is looked up at the workgroup's end, all at once, so no chunk waits on it.
      // Past the list's end (more than SD_PF_OVER such tokens) a token is looked up here and
      // only counted towards the demand.
      const bool over = writer && s_out > theta;
      const uint64_t mo = __ballot(over);
      if (mo) {
        const int lead = __ffsll(static_cast<unsigned long long>(mo)) - 1;
        int32_t base = 0;
        if (l == lead) base = atomicAdd(&pf_list[SD_PF_OVER], static_cast<int32_t>(__popcll(mo)));
        base = __builtin_amdgcn_readlane(base, lead);
        const int at = base + static_cast<int>(__popcll(mo & ((1ull << l) - 1ull)));
        if (over) {
          if (at < SD_PF_OVER) {
            pf_list[at] = t_out;
          } else {
            const int32_t h = pf.req_to_host[kb + t_out];
            if (h >= 0 && h < pf.n_host && pf.host_to_gpu[h] == INF) atomicAdd(&pf_list[SD_PF_OVER + 1], 1);
          }
        }
      }
    }
    if constexpr (HIST) hist_add_peeled(hl, (~f32_key(s_out)) >> 21, writer);
    buf ^= 1;
  }
  if constexpr (HIST || PREFETCH) __syncthreads();
  if constexpr (HIST) {
    uint32_t *gh = hist0 + static_cast<int64_t>(r) * 2048;
    for (int b = threadIdx.x; b < 2048; b += SD_THREADS)
      if (hl[b]) atomicAdd(&gh[b], hl[b]);
  }
  if constexpr (PREFETCH) {
    // residency of the listed over-threshold tokens: every load in flight before the first use
    const int32_t n_over = min(pf_list[SD_PF_OVER], SD_PF_OVER);
    int32_t tok[SD_PF_PER], hh[SD_PF_PER];
#pragma unroll
    for (int i = 0; i < SD_PF_PER; ++i) {
      const int e = threadIdx.x + i * SD_THREADS;
      tok[i] = e < n_over ? pf_list[e] : -1;
    }
#pragma unroll
    for (int i = 0; i < SD_PF_PER; ++i) hh[i] = tok[i] >= 0 ? pf.req_to_host[kb + tok[i]] : -1;
    bool el[SD_PF_PER];
#pragma unroll
    for (int i = 0; i < SD_PF_PER; ++i) el[i] = hh[i] >= 0 && hh[i] < pf.n_host;
#pragma unroll
    for (int i = 0; i < SD_PF_PER; ++i) el[i] = el[i] && pf.host_to_gpu[hh[i]] == INF;
    __syncthreads();                                 // every list entry read before compaction
    // the eligible ones move to the front of the list (in no particular order)
#pragma unroll
    for (int i = 0; i < SD_PF_PER; ++i) {
      const uint64_t me = __ballot(el[i]);
      if (me) {
        const int lead = __ffsll(static_cast<unsigned long long>(me)) - 1;
        int32_t base = 0;
        if (l == lead) base = atomicAdd(&pf_list[SD_PF_OVER + 2], static_cast<int32_t>(__popcll(me)));
        base = __builtin_amdgcn_readlane(base, lead);
        if (el[i]) pf_list[base + static_cast<int>(__popcll(me & ((1ull << l) - 1ull)))] = tok[i];
      }
    }
    __syncthreads();
    // every eligible token counts towards the request's demand (total_cnt); the workgroup
    // lists as many of them as this call's share of the cap still allows (the cumulative
    // share less what the step's earlier calls listed).  It reserves places [pos, pos + want)
    // with one atomic add on the call's list count, fills those below the share and gives the
    // rest back.  The reserved runs are disjoint, so the places filled are exactly
    // [0, min(share, all wants)); a workgroup that reserves after the one crossing the share
    // gets pos >= share, since that one gives back only what lies past the share; and once
    // every workgroup is done the count is the number listed.  (A compare-and-swap loop here
    // made the request's workgroups, which end together, wait for one another: measured on
    // MI355X at 64 x 131072 tokens in four ranges with a 98.4th-percentile threshold, each
    // range's launch took about 66 us against 51 us with no token over the threshold.)
    if (threadIdx.x == 0) {
      const int32_t n_listed = pf_list[SD_PF_OVER + 2];
      const int32_t n_q = n_listed + pf_list[SD_PF_OVER + 1];
      int32_t take = 0, pos = 0;
      if (n_q > 0) {
        atomicAdd(&pf.total_cnt[r], n_q);
        int32_t share = static_cast<int32_t>(static_cast<int64_t>(cap_r) * (pf.call + 1) / pf.n_calls);
        for (int c = 0; c < pf.call; ++c) share -= pf.before_cnt[static_cast<int64_t>(c) * pf.ld_before + r];
        const int32_t want = n_listed;
        if (want > 0) {
          pos = atomicAdd(&pf.cand_cnt[r], want);
          take = max(0, min(want, share - pos));
          if (take < want) atomicSub(&pf.cand_cnt[r], want - take);
        }
      }
      pf_list[SD_PF_OVER + 3] = take;
      pf_list[SD_PF_OVER + 4] = pos;
    }
    __syncthreads();
    const int32_t take = pf_list[SD_PF_OVER + 3], pos = pf_list[SD_PF_OVER + 4];
    for (int i = threadIdx.x; i < take; i += SD_THREADS)
      pf.cand[static_cast<int64_t>(r) * pf.cap + pos + i] = pf_list[i];
  }
}

// Tokens per workgroup: about one workgroup per CU for small launches, and at most 2048 tokens
// (measured on MI355X, scoring alone: 8 x 65536 tokens 12.6 us with 2048 per workgroup against
// 12.8 with 1024 and 20.7 with 4096; 64 x 131072 207 us with 2048, 210 with 8192, 242 with
// 32768), whole chunks each.
static int32_t pick_tokens_per_wg(int64_t total_tokens, int32_t max_len, bool hist) {
  (void)hist;
  const int64_t target = total_tokens / 256;
  int32_t t = SD_CHUNK;
  while (t < target && t < 2048) t <<= 1;
  if (t > max_len) t = ((max_len + SD_CHUNK - 1) / SD_CHUNK) * SD_CHUNK;
  return t < SD_CHUNK ? SD_CHUNK : t;
}

int launch_score_decode(const uint8_t *q, const float *w, const uint8_t *k, const float *k_scale,
                        const int64_t *key_begin, const int32_t *key_len, int32_t n_q,
                        int32_t max_len, int32_t tok_lo, int32_t tok_hi, float *scores,
                        int64_t ld, const PrefetchArgs *pf, uint32_t *hist0, const SideWork *side,
                        const KeyPages *kp, hipStream_t st) {
  tok_hi = tok_hi < max_len ? tok_hi : max_len;
  const int n_side = side ? side->n_stats + side->n_gather : 0;
  const bool scoring = n_q > 0 && tok_hi > tok_lo;
  if (!scoring && n_side == 0) return ECHO_OK;
  const int32_t span = scoring ? tok_hi - tok_lo : 1;
  int32_t tpw = pick_tokens_per_wg(static_cast<int64_t>(n_q) * span, span, hist0 != nullptr);
  // a prefetching range launch of at least 512 x 4096 tokens runs one round of 4096-token
  // workgroups instead of two of 2048, so it has one tail, not two (64 x 131072 tokens in four
  // ranges, measured on MI355X: 1909 us per step against 1919)
  if (pf && tpw == 2048 && static_cast<int64_t>(n_q) * span >= 512 * 4096) tpw = 4096;
  const int32_t gx = (span + tpw - 1) / tpw;
  const int64_t blocks = static_cast<int64_t>(n_side) + (scoring ? static_cast<int64_t>(gx) * n_q : 0);
  if (blocks > 0x7FFFFFFF) return fail(ECHO_EUNSUPPORTED, "score_decode: grid too large");
  PrefetchArgs none{};
  const PrefetchArgs &p = pf ? *pf : none;
  SideWork no_side{};
  const SideWork &sw = side ? *side : no_side;
  const KeyPages pages = kp ? *kp : KeyPages{nullptr, 0, 0};
#define ECHO_SD(SC, PF, HI, SI)                                                                 \
  do {                                                                                          \
    if (pages.table)                                                                            \
      score_decode_kernel<SC, PF, HI, SI, true><<<static_cast<unsigned>(blocks), SD_THREADS, 0, st>>>( \
          q, w, k, k_scale, key_begin, key_len, max_len, tok_lo, scoring ? tok_hi : tok_lo, tpw, gx, \
          scores, ld, p, hist0, sw, pages);                                                     \
    else                                                                                        \
      score_decode_kernel<SC, PF, HI, SI, false><<<static_cast<unsigned>(blocks), SD_THREADS, 0, st>>>( \
          q, w, k, k_scale, key_begin, key_len, max_len, tok_lo, scoring ? tok_hi : tok_lo, tpw, gx, \
          scores, ld, p, hist0, sw, pages);                                                     \
  } while (0)
  const bool sc = k_scale != nullptr, pfo = pf != nullptr, hi = hist0 != nullptr, si = n_side > 0;
  if (si) {
    // side work rides only with the decode step's scoring (histogram on)
    if (!hi) return fail(ECHO_EINVAL, "score_decode: side work needs the top-k histogram");
    if (sc && pfo) ECHO_SD(true, true, true, true);
    else if (sc) ECHO_SD(true, false, true, true);
    else if (pfo) ECHO_SD(false, true, true, true);
    else ECHO_SD(false, false, true, true);
  } else if (sc && pfo && hi) ECHO_SD(true, true, true, false);
  else if (sc && pfo) ECHO_SD(true, true, false, false);
  else if (sc && hi) ECHO_SD(true, false, true, false);
  else if (sc) ECHO_SD(true, false, false, false);
  else if (pfo && hi) ECHO_SD(false, true, true, false);
  else if (pfo) ECHO_SD(false, true, false, false);
  else if (hi) ECHO_SD(false, false, true, false);
  else ECHO_SD(false, false, false, false);
#undef ECHO_SD
  return check_launch("score_decode");
}

}  // namespace echo

using namespace echo;

extern "C" int echo_index_scores(const uint8_t *q, const float *w, const uint8_t *k,
                                 const float *k_scale, const int64_t *key_begin,
                                 const int32_t *key_len, int32_t n_q, int32_t max_key_len,
                                 float *scores, int64_t ld, void *stream) {
  if (n_q < 0 || max_key_len < 0) return fail(ECHO_EINVAL, "echo_index_scores: negative n_q or max_key_len");
  if (ld < max_key_len) return fail(ECHO_EINVAL, "echo_index_scores: ld %lld < max_key_len %d", (long long)ld, max_key_len);
  if (n_q > 65535) return fail(ECHO_EUNSUPPORTED, "echo_index_scores: n_q %d > 65535", n_q);
  if (n_q > 0 && (!q || !w || !key_begin || !key_len || !scores || (max_key_len > 0 && !k)))
    return fail(ECHO_EINVAL, "echo_index_scores: NULL pointer");
  return launch_score_decode(q, w, k, k_scale, key_begin, key_len, n_q, max_key_len, 0,
                             max_key_len, scores, ld, nullptr, nullptr, nullptr, nullptr, S(stream));
}

// Checks the page arguments of a paged key cache and fills kp; EINVAL/EUNSUPPORTED on error.
int echo::key_pages_of(const int32_t *page_table, int32_t page_size, int32_t max_pages,
                       int32_t max_key_len, const char *fn, KeyPages *kp) {
  if (!page_table) return fail(ECHO_EINVAL, "%s: NULL page table", fn);
  if (page_size < 16 || page_size > (1 << 16) || (page_size & (page_size - 1)))
    return fail(ECHO_EUNSUPPORTED, "%s: page size %d is not a power of two in [16, 65536]", fn, page_size);
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  if (max_pages < 1 || static_cast<int64_t>(max_pages) * page_size < max_key_len)
    return fail(ECHO_EINVAL, "%s: %d pages of %d tokens cannot hold max_key_len %d", fn, max_pages,
                page_size, max_key_len);
  *kp = KeyPages{page_table, shift, max_pages};
  return ECHO_OK;
}

extern "C" int echo_index_scores_paged(const uint8_t *q, const float *w, const uint8_t *k_pages,
                                       const float *k_scale_pages, const int32_t *page_table,
                                       int32_t page_size, int32_t max_pages,
                                       const int32_t *key_len, int32_t n_q, int32_t max_key_len,
                                       float *scores, int64_t ld, void *stream) {
  static const char *fn = "echo_index_scores_paged";
  if (n_q < 0 || max_key_len < 0) return fail(ECHO_EINVAL, "%s: negative n_q or max_key_len", fn);
  if (ld < max_key_len) return fail(ECHO_EINVAL, "%s: ld %lld < max_key_len %d", fn, (long long)ld, max_key_len);
  if (n_q > 65535) return fail(ECHO_EUNSUPPORTED, "%s: n_q %d > 65535", fn, n_q);
  if (n_q > 0 && (!q || !w || !key_len || !scores || (max_key_len > 0 && !k_pages)))
    return fail(ECHO_EINVAL, "%s: NULL pointer", fn);
  KeyPages kp{};
  int rc = key_pages_of(page_table, page_size, max_pages, max_key_len, fn, &kp);
  if (rc) return rc;
  // a request's key rows come from its pages (no key_begin)
  return launch_score_decode(q, w, k_pages, k_scale_pages, nullptr, key_len, n_q, max_key_len, 0,
                             max_key_len, scores, ld, nullptr, nullptr, nullptr, &kp, S(stream));
}

extern "C" int echo_index_scores_hist(const uint8_t *q, const float *w, const uint8_t *k,
                                      const float *k_scale, const int64_t *key_begin,
                                      const int32_t *key_len, int32_t n_q, int32_t max_key_len,
                                      float *scores, int64_t ld, uint32_t *hist, void *stream) {
  if (n_q < 0 || max_key_len < 0) return fail(ECHO_EINVAL, "echo_index_scores_hist: negative n_q or max_key_len");
  if (ld < max_key_len) return fail(ECHO_EINVAL, "echo_index_scores_hist: ld %lld < max_key_len %d", (long long)ld, max_key_len);
  if (n_q > 65535) return fail(ECHO_EUNSUPPORTED, "echo_index_scores_hist: n_q %d > 65535", n_q);
  if (n_q > 0 && (!q || !w || !key_begin || !key_len || !scores || !hist || (max_key_len > 0 && !k)))
    return fail(ECHO_EINVAL, "echo_index_scores_hist: NULL pointer");
  return launch_score_decode(q, w, k, k_scale, key_begin, key_len, n_q, max_key_len, 0,
                             max_key_len, scores, ld, nullptr, hist, nullptr, nullptr, S(stream));
}

extern "C" int echo_index_scores_prefetch(const uint8_t *q, const float *w, const uint8_t *k,
                                          const float *k_scale, const int64_t *key_begin,
                                          const int32_t *key_len, int32_t n_q,
                                          int32_t max_key_len, int32_t tok_lo, int32_t tok_hi,
                                          float *scores, int64_t ld, const float *theta,
                                          const int32_t *req_to_host, const int32_t *host_to_gpu,
                                          int32_t n_host, int32_t *cand, int32_t *cand_cnt,
                                          int32_t *total_cnt, int32_t cap, int32_t cap_div,
                                          void *stream) {
  if (n_q < 0 || max_key_len < 0) return fail(ECHO_EINVAL, "echo_index_scores_prefetch: negative n_q or max_key_len");
  if (ld < max_key_len) return fail(ECHO_EINVAL, "echo_index_scores_prefetch: ld < max_key_len");
  if (n_q > 65535) return fail(ECHO_EUNSUPPORTED, "echo_index_scores_prefetch: n_q > 65535");
  if (tok_lo < 0 || tok_hi < tok_lo) return fail(ECHO_EINVAL, "echo_index_scores_prefetch: bad token range");
  if (cap < 0 || cap_div < 1) return fail(ECHO_EINVAL, "echo_index_scores_prefetch: cap < 0 or cap_div < 1");
  if (n_q > 0 && (!q || !w || !key_begin || !key_len || !scores || !theta || !req_to_host ||
                  !host_to_gpu || !cand_cnt || !total_cnt || (cap > 0 && !cand) || (max_key_len > 0 && !k)))
    return fail(ECHO_EINVAL, "echo_index_scores_prefetch: NULL pointer");
  if (n_host < 0) return fail(ECHO_EINVAL, "echo_index_scores_prefetch: n_host < 0");
  PrefetchArgs pf{theta, req_to_host, host_to_gpu, cand, cand_cnt, total_cnt, cap, cap_div, n_host, 0, 1,
                  nullptr, 0};
  return launch_score_decode(q, w, k, k_scale, key_begin, key_len, n_q, max_key_len, tok_lo,
                             tok_hi, scores, ld, &pf, nullptr, nullptr, nullptr, S(stream));
}
