// Exact top-k for the decode step, spread over many workgroups (ECHO review page §2: exact
// top-k of the indexer scores; ties go to the lower token index), followed by the residency
// lookup of the selected tokens (§5.2: recall starts with a lookup of the selected host
// indices in HostTokenToGPU).
//
//   split   grid (4096-score chunk, request): every workgroup re-derives the threshold bin b0
//           of the request from the digit-0 histogram the scoring kernel built, and writes the
//           indices of its chunk below b0 ("sure") and the (key, index) pairs in b0
//           ("candidates") into per-chunk segments, in index order.  In the decode step it
//           also looks the sure selections up in the pool right away (they are selected
//           whatever the remaining digits decide): hits are protected and leave the priority
//           histogram, misses are queued for staging from host memory, and each sure
//           selection's result goes to sure_code.
//   finish  one 1024-thread workgroup per request: concatenates the segments in chunk order
//           (so both lists are ascending), resolves the remaining key digits on the
//           candidates in LDS, takes the keys below the threshold key and the lowest-index
//           ties, merges the two ascending lists into the selection, writes it, and looks each
//           selected token up in the pool (the sure ones by their split result, the others
//           now), lists the misses in order and queues the new ones for staging.  Extra
//           workgroups of the same launch read the split's queued misses from host memory.
//           A threshold bin too large for LDS is resolved with passes over the request's
//           scores instead.
#include <algorithm>

#include "internal.hpp"
#include "pool_common.cuh"

namespace echo {

constexpr int TS_T = 256;                        // split workgroup
constexpr int TS_CH = 4096;                      // scores per chunk
constexpr int TF_T = 1024;                       // finish workgroup
constexpr int TF_CAP = 8192;                     // candidates resolved in LDS
constexpr int TF_J = 8;                          // overflow passes: groups per thread per batch
constexpr int TF_STEP = 4 * TF_T;
constexpr int TF_BATCH = TF_J * TF_STEP;
constexpr int TS_HW = 2048;                      // LDS histogram window of a split workgroup

ECHO_DEV uint32_t score_key(float x) { return ~f32_key(x); }   // ascending key = descending score

// Staging row named by an early-lookup code (-2 - row), or -1 when the code names none or a row
// outside the staging area [0, n_stage).  Computed in 64 bits, so no code value overflows.
ECHO_DEV int32_t staged_row(int32_t code, int64_t n_stage) {
  if (code > -2) return -1;
  const int64_t row = -2 - static_cast<int64_t>(code);
  return row < n_stage ? static_cast<int32_t>(row) : -1;
}

// keys of elements i0 .. i0+3 of a row (bit e of `valid` marks presence)
ECHO_DEV void row_load4(const float *row, bool vec, int32_t n, int32_t i0, uint32_t key[4], int &valid) {
  valid = 0;
  if (vec && i0 + 3 < n) {
    const float4 v = *reinterpret_cast<const float4 *>(row + i0);
    key[0] = score_key(v.x); key[1] = score_key(v.y); key[2] = score_key(v.z); key[3] = score_key(v.w);
    valid = 0xF;
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    key[e] = 0xFFFFFFFFu;
    if (i0 + e < n) { key[e] = score_key(row[i0 + e]); valid |= 1 << e; }
  }
}

template <int NT>
ECHO_DEV void pick_bins(const uint32_t *hist, int nb, uint32_t m, uint32_t *tmp, uint32_t &bin,
                        uint32_t &below) {
  const int per = nb / NT;
  const int t = threadIdx.x;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[t * per + i];
  uint32_t total;
  const uint32_t before = block_excl_scan<NT>(local, tmp, &total);
  if (before < m && m <= before + local) {
    uint32_t cum = before;
    for (int i = 0; i < per; ++i) {
      const uint32_t c = hist[t * per + i];
      if (cum < m && m <= cum + c) { tmp[40] = t * per + i; tmp[41] = cum; break; }
      cum += c;
    }
  }
  __syncthreads();
  bin = tmp[40];
  below = tmp[41];
  __syncthreads();
}

size_t topk_split_ws_bytes(int32_t n_rows, int32_t max_len, int32_t k) {
  const int64_t nch = std::max(1, (max_len + TS_CH - 1) / TS_CH);
  const int64_t segs = static_cast<int64_t>(n_rows) * nch;
  auto al = [](int64_t b) { return (b + 255) & ~static_cast<int64_t>(255); };
  return static_cast<size_t>(al(segs * 4) * 2 + al(segs * k * 4) * 2 + al(segs * TS_CH * 8));
}

struct SplitWs {
  uint32_t *sure_cnt;   // [n_rows * nch]
  uint32_t *cand_cnt;   // [n_rows * nch]
  int32_t *sure;        // [n_rows * nch * k]
  uint64_t *cand;       // [n_rows * nch * 4096]  (key << 32 | index)
  int32_t *sure_code;   // [n_rows * nch * k] early lookup: slot (hit), -2 - staging row (miss), -1 (bad)
  int32_t nch;
};

// Early residency lookup of the sure selections (decode step).
struct SplitLookup {
  PoolArgs P;
  PoolFastWs W;
  const int64_t *key_begin;
  const int32_t *req_to_host;
  Stamp stamp;
};

static SplitWs make_split_ws(void *base, int32_t n_rows, int32_t max_len, int32_t k) {
  const int64_t nch = std::max(1, (max_len + TS_CH - 1) / TS_CH);
  const int64_t segs = static_cast<int64_t>(n_rows) * nch;
  auto al = [](int64_t b) { return (b + 255) & ~static_cast<int64_t>(255); };
  char *b = static_cast<char *>(base);
  SplitWs w;
  w.sure_cnt = reinterpret_cast<uint32_t *>(b);
  w.cand_cnt = reinterpret_cast<uint32_t *>(b + al(segs * 4));
  w.sure = reinterpret_cast<int32_t *>(b + 2 * al(segs * 4));
  w.cand = reinterpret_cast<uint64_t *>(b + 2 * al(segs * 4) + al(segs * k * 4));
  w.sure_code = reinterpret_cast<int32_t *>(b + 2 * al(segs * 4) + al(segs * k * 4) + al(segs * TS_CH * 8));
  w.nch = static_cast<int32_t>(nch);
  return w;
}

// ---------------------------------------------------------------- split
// LOOKUP: the early residency lookup of the sure selections (see the file comment).
// Side work (decode step): n_stats leading workgroups compute the pool statistics of one
// 4096-slot chunk each (free count, priority histograms of every occupied slot) while the
// other workgroups split; the lookup's subtraction of protected slots commutes with them.
constexpr int TS_GSCAN = 4 * (TS_T / 64) + TS_T / 64 + 2;
constexpr int TS_SPLIT_WORDS = 48 + TS_GSCAN + ECHO_MAX_TOPK + TS_HW;
constexpr int TS_LDS_WORDS = TS_SPLIT_WORDS > STATS_LDS_WORDS ? TS_SPLIT_WORDS : STATS_LDS_WORDS;

template <bool LOOKUP>
__global__ __launch_bounds__(TS_T) void topk_split_kernel(const float *__restrict__ scores, int64_t ld,
                                                          const int32_t *__restrict__ len, int32_t max_len,
                                                          int32_t k, const uint32_t *__restrict__ hist0,
                                                          SplitWs W, SplitLookup L, SideWork side) {
  __shared__ uint32_t lds[LOOKUP ? TS_LDS_WORDS : 48 + TS_GSCAN];
  int blk = blockIdx.x;
  if constexpr (LOOKUP) {
    if (blk < side.n_stats) {
      stats_chunk<false>(side.P, side.W, stamp_of(side.stamp), blk, lds);
      return;
    }
    blk -= side.n_stats;
  }
  uint32_t *tmp = lds, *gscan = lds + 48;
  int32_t *sl = reinterpret_cast<int32_t *>(lds + 48 + TS_GSCAN);   // this chunk's sure indices, ascending
  uint32_t *hl = lds + 48 + TS_GSCAN + ECHO_MAX_TOPK;
  const int r = blk / W.nch, c = blk % W.nch, t = threadIdx.x;
  const int32_t n = min(max(len[r], 0), max_len);
  const int32_t m = min(k, n);
  if (m == n || c * TS_CH >= n) return;
  uint32_t b0, below0, c0;
  pick2048<TS_T>(hist0 + static_cast<int64_t>(r) * 2048, static_cast<uint32_t>(m), tmp, b0, below0, c0);
  const bool keep_cand = c0 <= TF_CAP;
  const float *row = scores + static_cast<int64_t>(r) * ld;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  uint32_t key[4][4];
  int valid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) row_load4(row, vec, n, c * TS_CH + j * 4 * TS_T + t * 4, key[j], valid[j]);
  uint32_t cnt[4], off[4], tot;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t cs = 0, cc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((valid[j] >> e) & 1) {
        const uint32_t b = key[j][e] >> 21;
        cs += b < b0;
        cc += b == b0 && keep_cand;
      }
    cnt[j] = cs | (cc << 16);
  }
  group_excl_scan<TS_T, 4>(cnt, off, gscan, &tot);
  const int64_t seg = static_cast<int64_t>(r) * W.nch + c;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t ps = off[j] & 0xFFFF, pc = off[j] >> 16;
    const int32_t i0 = c * TS_CH + j * 4 * TS_T + t * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((valid[j] >> e) & 1) {
        const uint32_t b = key[j][e] >> 21;
        if (b < b0) {
          if (ps < static_cast<uint32_t>(k)) {
            W.sure[seg * k + ps] = i0 + e;
            if (LOOKUP) sl[ps] = i0 + e;
          }
          ++ps;
        } else if (b == b0 && keep_cand) {
          W.cand[seg * TS_CH + pc] = (static_cast<uint64_t>(key[j][e]) << 32) | static_cast<uint32_t>(i0 + e);
          ++pc;
        }
      }
  }
  if (t == 0) {
    W.sure_cnt[seg] = tot & 0xFFFF;
    W.cand_cnt[seg] = tot >> 16;
  }
  if constexpr (LOOKUP) {
    if (L.P.n_gpu == 0) return;
    __syncthreads();
    const PoolArgs &P = L.P;
    const uint32_t n_s = min(tot & 0xFFFFu, static_cast<uint32_t>(k));
    const int64_t kb = L.key_begin[r];
    for (uint32_t base = 0; base < n_s; base += 4 * TS_T) {      // uniform
      int32_t h[4], slot[4], code[4], pr[4];
      uint32_t miss[4], old[4], bins[4];
      bool hit[4], bad = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t p = base + i * TS_T + t;
        h[i] = p < n_s ? L.req_to_host[kb + sl[p]] : -1;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t p = base + i * TS_T + t;
        slot[i] = (p < n_s && h[i] >= 0 && h[i] < P.n_host) ? P.host_to_gpu[h[i]] : -1;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t p = base + i * TS_T + t;
        hit[i] = false;
        miss[i] = 0;
        code[i] = -1;
        if (p < n_s) {
          if (h[i] < 0 || h[i] >= P.n_host) bad = true;
          else if (slot[i] == INF) miss[i] = 1;
          else if (slot[i] < 0 || slot[i] >= P.n_gpu) bad = true;
          else { hit[i] = true; code[i] = slot[i]; }
        }
      }
      if (bad) atomicOr(P.status, ECHO_ST_BAD_HOST);
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = hit[i] ? P.priority[slot[i]] : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        old[i] = hit[i] ? atomicOr(&L.W.prot[slot[i] >> 5], 1u << (slot[i] & 31)) : ~0u;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bins[i] = (hit[i] && !((old[i] >> (slot[i] & 31)) & 1u)) ? prio_bin(pr[i], stamp_of(L.stamp)) : 0xFFFFFFFFu;
      // misses: staging rows r*k + [stage_a[r], ...), reserved once per workgroup
      uint32_t mo[4], n_m;
      group_excl_scan<TS_T, 4>(miss, mo, gscan, &n_m);
      if (t == 0) tmp[44] = n_m ? atomicAdd(&L.W.stage_a[r], n_m) : 0u;
      __syncthreads();
      const uint32_t sbase = tmp[44];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t p = base + i * TS_T + t;
        if (miss[i]) {
          const int64_t srow = static_cast<int64_t>(r) * k + sbase + mo[i];
          L.W.stage_h[srow] = h[i];
          code[i] = -2 - static_cast<int32_t>(srow);
        }
        if (p < n_s) W.sure_code[seg * k + p] = code[i];
      }
      hist_flush_bins<TS_T, 4, true, TS_HW>(bins, hl, tmp, L.W.fine, L.W.coarse);
    }
  }
}

// ---------------------------------------------------------------- finish + lookup
__global__ __launch_bounds__(TF_T) void topk_finish_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ len, int32_t max_len,
    int32_t k, const uint32_t *__restrict__ hist0, SplitWs W, int32_t *__restrict__ idx,
    // lookup (skipped when pool.n_gpu == 0)
    PoolArgs P, PoolFastWs PW, const int64_t *__restrict__ key_begin,
    const int32_t *__restrict__ req_to_host, Stamp stamp, int32_t *__restrict__ topk_slot,
    bool sub_prot, bool early, int32_t n_rows, StageArgs SA) {
  if (static_cast<int>(blockIdx.x) >= n_rows) {
    // staging of (most of) the misses the split's early lookup found
    const int u = blockIdx.x - n_rows, per = (k + 127) / 128, rr = u / per;
    const int32_t hi = stage_cut_f(static_cast<int32_t>(PW.stage_a[rr]));
    stage_rows<TF_T, 128>(SA.host_kv, SA.stage, PW.stage_h, P.status, k, P.n_host, rr,
                          (u % per) * 128, 0, hi);
    return;
  }
  __shared__ uint32_t tmp[48];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t cbuf[2 * TF_CAP];               // candidates; later the lookup's histogram
  uint32_t *ckey = cbuf;
  int32_t *cidx = reinterpret_cast<int32_t *>(cbuf + TF_CAP);
  __shared__ int32_t sure[ECHO_MAX_TOPK];
  __shared__ int32_t scode[ECHO_MAX_TOPK];            // early-lookup result of each sure selection
  __shared__ int32_t sel[ECHO_MAX_TOPK];
  __shared__ int32_t fin[ECHO_MAX_TOPK];
  __shared__ uint32_t segoff[2][1024];
  __shared__ uint32_t gscan[TF_J * (TF_T / 64) + TF_T / 64 + 2];
  const int r = blockIdx.x, t = threadIdx.x;
  const int32_t n = min(max(len[r], 0), max_len);
  const int32_t m = min(k, n);
  const float *row = scores + static_cast<int64_t>(r) * ld;
  uint32_t n_sure_sel = 0;                           // sure selections listed in sure[]

  if (m == n) {
    for (int j = t; j < m; j += TF_T) fin[j] = j;
  } else {
    const int nch_r = (n + TS_CH - 1) / TS_CH;          // chunks of this request (<= 1024)
    const int64_t seg0 = static_cast<int64_t>(r) * W.nch;
    const uint32_t sc = t < nch_r ? W.sure_cnt[seg0 + t] : 0u;   // loaded with the histogram
    const uint32_t cc = t < nch_r ? W.cand_cnt[seg0 + t] : 0u;
    uint32_t b0, below0, c0;
    pick2048<TF_T>(hist0 + static_cast<int64_t>(r) * 2048, static_cast<uint32_t>(m), tmp, b0, below0, c0);
    uint32_t k_rem = static_cast<uint32_t>(m) - below0;
    uint32_t prefix = b0 << 21, mask = 0xFFE00000u;
    // segment offsets: exclusive prefixes over the request's chunks
    {
      uint32_t tot;
      const uint32_t so = block_excl_scan<TF_T>(sc, tmp, &tot);
      const uint32_t co = block_excl_scan<TF_T>(cc, tmp, &tot);
      segoff[0][t] = so;
      segoff[1][t] = co;
    }
    __syncthreads();
    // sure list, ascending: position p lives in the chunk whose offset range holds it (all
    // loads independent, issued together)
    auto seg_of = [&](int which, uint32_t p) {
      int lo = 0, hi = nch_r - 1;
      while (lo < hi) { const int md = (lo + hi + 1) >> 1; if (segoff[which][md] <= p) lo = md; else hi = md - 1; }
      return lo;
    };
    const uint32_t n_sure = min(below0, static_cast<uint32_t>(ECHO_MAX_TOPK));
    n_sure_sel = n_sure;
    for (uint32_t p = t; p < n_sure; p += TF_T) {
      const int q = seg_of(0, p);
      const int64_t at = (seg0 + q) * k + (p - segoff[0][q]);
      sure[p] = W.sure[at];
      if (early) scode[p] = W.sure_code[at];
    }
    if (c0 <= TF_CAP) {
      const uint32_t n_cand = c0;
      for (uint32_t p = t; p < n_cand; p += TF_T) {
        const int q = seg_of(1, p);
        const uint64_t v = W.cand[(seg0 + q) * TS_CH + (p - segoff[1][q])];
        ckey[p] = static_cast<uint32_t>(v >> 32);
        cidx[p] = static_cast<int32_t>(v & 0xFFFFFFFFu);
      }
      __syncthreads();
      for (int d = 1; d <= 2; ++d) {
        const int sh = d == 1 ? 10 : 0;
        const uint32_t dm = d == 1 ? 0x7FFu : 0x3FFu;
        for (int b = t; b < 2048; b += TF_T) hist[b] = 0;
        __syncthreads();
        for (uint32_t i0 = 0; i0 < n_cand; i0 += TF_T) {
          const uint32_t i = i0 + t;
          const uint32_t kk = i < n_cand ? ckey[i] : 0u;
          hist_add_peeled(hist, (kk >> sh) & dm, i < n_cand && (kk & mask) == prefix);
        }
        __syncthreads();
        uint32_t b, bl;
        pick_bins<TF_T>(hist, d == 1 ? 2048 : 1024, k_rem, tmp, b, bl);
        k_rem -= bl;
        prefix |= b << sh;
        mask |= dm << sh;
      }
      // candidates in index order: every key < K*, then the first k_rem keys == K*.  One scan
      // of the (less, equal) counts packed 16|16 (n_cand <= TF_CAP < 2^16) places them all:
      // a taken candidate goes to (less before) + min(equal before, k_rem).
      constexpr int SJ = TF_CAP / TF_T;
      uint32_t cnt[SJ], cbase[SJ], ctot;
#pragma unroll
      for (int j = 0; j < SJ; ++j) {
        const uint32_t i = j * TF_T + t;
        const uint32_t kk = i < n_cand ? ckey[i] : ~0u;
        cnt[j] = i < n_cand ? ((kk < prefix ? 1u : 0u) | (kk == prefix ? 0x10000u : 0u)) : 0u;
      }
      group_excl_scan<TF_T, SJ>(cnt, cbase, gscan, &ctot);
#pragma unroll
      for (int j = 0; j < SJ; ++j) {
        const uint32_t i = j * TF_T + t;
        const uint32_t lt_b = cbase[j] & 0xFFFFu, eq_b = cbase[j] >> 16;
        const bool take = (cnt[j] & 0xFFFFu) || ((cnt[j] >> 16) && eq_b < k_rem);
        if (take) {
          const uint32_t pos = lt_b + min(eq_b, k_rem);
          if (pos < ECHO_MAX_TOPK) sel[pos] = cidx[i];
        }
      }
      __syncthreads();
      const uint32_t n_sel = min((ctot & 0xFFFFu) + min(ctot >> 16, k_rem), static_cast<uint32_t>(ECHO_MAX_TOPK));
      for (uint32_t a = t; a < n_sure; a += TF_T) {
        const int32_t v = sure[a];
        uint32_t lo = 0, hi = n_sel;
        while (lo < hi) { const uint32_t md = (lo + hi) >> 1; if (sel[md] < v) lo = md + 1; else hi = md; }
        if (a + lo < ECHO_MAX_TOPK) fin[a + lo] = v;
      }
      for (uint32_t b = t; b < n_sel; b += TF_T) {
        const int32_t v = sel[b];
        uint32_t lo = 0, hi = n_sure;
        while (lo < hi) { const uint32_t md = (lo + hi) >> 1; if (sure[md] < v) lo = md + 1; else hi = md; }
        if (b + lo < ECHO_MAX_TOPK) fin[b + lo] = v;
      }
    } else {
      // overflow: remaining digits and the ordered output by passes over the row's scores
      const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
      uint32_t key[TF_J][4];
      int valid[TF_J];
      for (int d = 1; d <= 2; ++d) {
        const int sh = d == 1 ? 10 : 0;
        const uint32_t dm = d == 1 ? 0x7FFu : 0x3FFu;
        for (int b = t; b < 2048; b += TF_T) hist[b] = 0;
        __syncthreads();
        for (int32_t base = 0; base < n; base += TF_BATCH) {
#pragma unroll
          for (int j = 0; j < TF_J; ++j) row_load4(row, vec, n, base + j * TF_STEP + t * 4, key[j], valid[j]);
#pragma unroll
          for (int j = 0; j < TF_J; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              hist_add_peeled(hist, (key[j][e] >> sh) & dm, ((valid[j] >> e) & 1) && (key[j][e] & mask) == prefix);
        }
        __syncthreads();
        uint32_t b, bl;
        pick_bins<TF_T>(hist, d == 1 ? 2048 : 1024, k_rem, tmp, b, bl);
        k_rem -= bl;
        prefix |= b << sh;
        mask |= dm << sh;
      }
      uint32_t n_out = 0, eq_seen = 0;
      for (int32_t base = 0; base < n; base += TF_BATCH) {
#pragma unroll
        for (int j = 0; j < TF_J; ++j) row_load4(row, vec, n, base + j * TF_STEP + t * 4, key[j], valid[j]);
        uint32_t eqc[TF_J], eqo[TF_J], tot;
#pragma unroll
        for (int j = 0; j < TF_J; ++j) {
          eqc[j] = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) eqc[j] += ((valid[j] >> e) & 1) && key[j][e] == prefix;
        }
        group_excl_scan<TF_T, TF_J>(eqc, eqo, gscan, &tot);
        uint32_t tk[TF_J], po[TF_J], tot2;
#pragma unroll
        for (int j = 0; j < TF_J; ++j) {
          uint32_t er = eq_seen + eqo[j];
          tk[j] = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((valid[j] >> e) & 1) {
              if (key[j][e] < prefix) ++tk[j];
              else if (key[j][e] == prefix) { if (er < k_rem) ++tk[j]; ++er; }
            }
        }
        group_excl_scan<TF_T, TF_J>(tk, po, gscan, &tot2);
#pragma unroll
        for (int j = 0; j < TF_J; ++j) {
          uint32_t er = eq_seen + eqo[j], pos = n_out + po[j];
          const int32_t i0 = base + j * TF_STEP + t * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((valid[j] >> e) & 1) {
              bool take = key[j][e] < prefix;
              if (key[j][e] == prefix) { take = er < k_rem; ++er; }
              if (take) {
                if (pos < ECHO_MAX_TOPK) fin[pos] = i0 + e;
                ++pos;
              }
            }
        }
        n_out += tot2;
        eq_seen += tot;
      }
    }
  }
  __syncthreads();
  int32_t *out = idx + static_cast<int64_t>(r) * k;
  for (int j = t; j < k; j += TF_T) out[j] = j < m ? fin[j] : -1;

  // ---- residency lookup of the selection, misses listed in order
  if (P.n_gpu == 0) return;
  int32_t *slot_out = topk_slot + static_cast<int64_t>(r) * k;
  const int64_t kb = key_begin[r];
  const uint32_t sa = early ? PW.stage_a[r] : 0u;
  constexpr int LJ = ECHO_MAX_TOPK / TF_T;          // entries per thread: j = t + TF_T * i
  int32_t h[LJ], slot[LJ], res[LJ], srow[LJ], code[LJ], early_row[LJ];
  bool cand[LJ], hit[LJ];
  const int64_t n_stage = static_cast<int64_t>(n_rows) * k;
  // a sure selection carries the split's result; the others are looked up here
#pragma unroll
  for (int i = 0; i < LJ; ++i) {
    const int32_t j = t + TF_T * i;
    cand[i] = j < m;
    code[i] = -1;
    if (early && j < m && n_sure_sel > 0) {
      const int32_t tok = fin[j];
      uint32_t lo = 0, hi = n_sure_sel;
      while (lo < hi) { const uint32_t md = (lo + hi) >> 1; if (sure[md] < tok) lo = md + 1; else hi = md; }
      if (lo < n_sure_sel && sure[lo] == tok) { cand[i] = false; code[i] = scode[lo]; }
    }
  }
#pragma unroll
  for (int i = 0; i < LJ; ++i) {
    const int32_t j = t + TF_T * i;
    early_row[i] = staged_row(code[i], n_stage);
    h[i] = cand[i] ? req_to_host[kb + fin[j]] : (early_row[i] >= 0 ? PW.stage_h[early_row[i]] : -1);
  }
#pragma unroll
  for (int i = 0; i < LJ; ++i)
    slot[i] = (cand[i] && h[i] >= 0 && h[i] < P.n_host) ? P.host_to_gpu[h[i]] : -1;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < LJ; ++i) {
    const int32_t j = t + TF_T * i;
    hit[i] = false;
    res[i] = -1;
    srow[i] = -1;
    if (cand[i]) {
      if (h[i] < 0 || h[i] >= P.n_host) bad = true;
      else if (slot[i] == INF) res[i] = INF;
      else if (slot[i] < 0 || slot[i] >= P.n_gpu) bad = true;
      else { hit[i] = true; res[i] = slot[i]; }
    } else if (j < m) {
      if (code[i] >= 0) res[i] = code[i];                        // hit, protected by the split
      else if (early_row[i] >= 0) { res[i] = INF; srow[i] = early_row[i]; }   // miss, already queued
      else if (code[i] <= -2) bad = true;                         // no such staging row
    }
  }
  if (bad) atomicOr(P.status, ECHO_ST_BAD_HOST);
  if (sub_prot) {
    // protected slots leave the occupied-slot histogram: the first protector of each slot
    // subtracts its priority bin (priorities do not change before the eviction kernels)
    int32_t pr[LJ];
    uint32_t old[LJ], pbin[LJ];
#pragma unroll
    for (int i = 0; i < LJ; ++i) pr[i] = hit[i] ? P.priority[slot[i]] : 0;
#pragma unroll
    for (int i = 0; i < LJ; ++i)
      old[i] = hit[i] ? atomicOr(&PW.prot[slot[i] >> 5], 1u << (slot[i] & 31)) : ~0u;
#pragma unroll
    for (int i = 0; i < LJ; ++i)
      pbin[i] = (hit[i] && !((old[i] >> (slot[i] & 31)) & 1u)) ? prio_bin(pr[i], stamp_of(stamp)) : 0xFFFFFFFFu;
    hist_flush_bins<TF_T, LJ, true, 2 * TF_CAP>(pbin, cbuf, tmp, PW.fine, PW.coarse);
  } else {
#pragma unroll
    for (int i = 0; i < LJ; ++i)
      if (hit[i]) atomicOr(&PW.prot[slot[i] >> 5], 1u << (slot[i] & 31));
  }
  // misses found here take the staging rows after the split's, in column order
  uint32_t cm[LJ], cmo[LJ], n_cm, mc[LJ], mo[LJ], n_miss;
#pragma unroll
  for (int i = 0; i < LJ; ++i) cm[i] = (cand[i] && res[i] == INF) ? 1u : 0u;
  group_excl_scan<TF_T, LJ>(cm, cmo, gscan, &n_cm);
#pragma unroll
  for (int i = 0; i < LJ; ++i)
    if (cm[i]) {
      srow[i] = r * k + static_cast<int32_t>(sa + cmo[i]);
      PW.stage_h[srow[i]] = h[i];
    }
  if (t == 0) PW.stage_b[r] = n_cm;
#pragma unroll
  for (int i = 0; i < LJ; ++i) mc[i] = res[i] == INF ? 1u : 0u;
  group_excl_scan<TF_T, LJ>(mc, mo, gscan, &n_miss);
#pragma unroll
  for (int i = 0; i < LJ; ++i) {
    const int32_t j = t + TF_T * i;
    if (mc[i]) {
      PW.row_miss_h[static_cast<int64_t>(r) * k + mo[i]] = h[i];
      PW.row_miss_j[static_cast<int64_t>(r) * k + mo[i]] = j;
      PW.row_miss_s[static_cast<int64_t>(r) * k + mo[i]] = srow[i];
    }
    if (j < k) slot_out[j] = (res[i] >= 0 && res[i] != INF) ? res[i] : -1;
  }
  if (t == 0) PW.row_miss_cnt[r] = n_miss;
}

int launch_topk_split(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                      int32_t max_len, int32_t k, const uint32_t *hist0, void *split_ws,
                      const echo_pool *pool, const PoolFastWs *pw, const int64_t *key_begin,
                      const int32_t *req_to_host, Stamp stamp, const SideWork *side,
                      hipStream_t st) {
  if (n_rows == 0) return ECHO_OK;
  if ((max_len + TS_CH - 1) / TS_CH > 1024) return fail(ECHO_EUNSUPPORTED, "decode top-k: rows longer than 4M tokens");
  SplitWs W = make_split_ws(split_ws, n_rows, max_len, k);
  SideWork no_side{};
  const SideWork &sw = side && pool ? *side : no_side;
  const int64_t blocks = static_cast<int64_t>(W.nch) * n_rows + sw.n_stats;
  if (blocks > 0x7FFFFFFF) return fail(ECHO_EUNSUPPORTED, "decode top-k: grid too large");
  if (sw.n_gather) return fail(ECHO_EINVAL, "decode top-k: the split carries no gathers");
  SplitLookup L{};
  if (pool) {
    L.P = PoolArgs{pool->gpu_free, pool->gpu_priority, pool->gpu_to_host, pool->host_to_gpu,
                   pool->indices_buf, pool->status, pool->n_gpu, pool->n_host};
    L.W = *pw;
    L.key_begin = key_begin;
    L.req_to_host = req_to_host;
    L.stamp = stamp;
    topk_split_kernel<true><<<static_cast<unsigned>(blocks), TS_T, 0, st>>>(scores, ld, len, max_len, k, hist0, W, L, sw);
  } else {
    topk_split_kernel<false><<<static_cast<unsigned>(blocks), TS_T, 0, st>>>(scores, ld, len, max_len, k, hist0, W, L, sw);
  }
  return check_launch("topk_split");
}

int launch_topk_finish(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                       int32_t max_len, int32_t k, const uint32_t *hist0, void *split_ws,
                       int32_t *idx, const echo_pool *pool, const PoolFastWs *pw,
                       const int64_t *key_begin, const int32_t *req_to_host, Stamp stamp,
                       int32_t *topk_slot, bool early, uint16_t *stage, hipStream_t st) {
  if (n_rows == 0) return ECHO_OK;
  SplitWs W = make_split_ws(split_ws, n_rows, max_len, k);
  PoolArgs P{};
  PoolFastWs PW{};
  StageArgs SA{nullptr, nullptr};
  int extra = 0;
  if (pool) {
    P = PoolArgs{pool->gpu_free, pool->gpu_priority, pool->gpu_to_host, pool->host_to_gpu,
                 pool->indices_buf, pool->status, pool->n_gpu, pool->n_host};
    PW = *pw;
    if (early && stage) {
      SA = StageArgs{pool->host_kv, stage};
      extra = n_rows * ((k + 127) / 128);
    }
  }
  topk_finish_kernel<<<n_rows + extra, TF_T, 0, st>>>(scores, ld, len, max_len, k, hist0, W, idx, P, PW,
                                                      key_begin, req_to_host, stamp, topk_slot,
                                                      pool != nullptr, early && pool != nullptr, n_rows, SA);
  return check_launch("topk_finish");
}

}  // namespace echo
