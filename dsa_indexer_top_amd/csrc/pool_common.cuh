// Device helpers shared by the pool-step kernels and the fused top-k lookup.
#pragma once

#include "internal.hpp"

namespace echo {

constexpr int PF_T = 256;                     // threads of the slot / entry workgroups
constexpr int PF_CH = 4096;                   // slots per chunk
constexpr int PF_FINE = 32768;                // fine priority bins
constexpr int PF_COARSE = 1024;               // coarse bins (32 fine bins each)
constexpr int PF_HIST_WORDS = 32768;          // words of each histogram array (layout below)

// Histogram layout: bin b lives at word (b % 32) * 1024 + b / 32, so consecutive bins are 4 KB
// apart and land in different memory channels.  The bins that collect most updates are
// neighbours (priorities are step stamps), and device-scope atomics confined to one channel
// run several times slower than spread ones.  The coarse array uses the same map (1024 of its
// 32768 words are used).
ECHO_DEV uint32_t hist_at(uint32_t b) { return (b & 31u) * 1024u + (b >> 5); }
constexpr int STATS_HW = 4096;               // LDS histogram window (words) of a stats chunk
constexpr int STATS_LDS_WORDS = STATS_HW + 48;

// ---------------------------------------------------------------- priority code
ECHO_DEV uint32_t lc9(uint64_t x) {           // monotone code of x in [0, 2^33), 9 mantissa bits
  const uint64_t y = x + 1;
  const int e = 63 - __clzll(static_cast<unsigned long long>(y));
  const uint32_t m = static_cast<uint32_t>((y << 9) >> e) & 511u;
  return static_cast<uint32_t>(e) * 512u + m;
}

// Fine bin of a priority, in [0, 32768): ascending bin <=> ascending priority (non-strict).
// Ages (step - priority) of either sign get a log code each; the two extreme ages share the
// outermost bins, which keeps the code monotone.
ECHO_DEV uint32_t prio_bin(int32_t prio, int32_t step) {
  const int64_t age = static_cast<int64_t>(step) - static_cast<int64_t>(prio);
  const uint32_t c = age >= 0 ? 16384u + min(lc9(static_cast<uint64_t>(age)), 16383u)
                              : 16383u - min(lc9(static_cast<uint64_t>(-age - 1)), 16383u);
  return 32767u - c;
}

// LDS histogram add on 16-bit counters packed two per word, the wave's most common bin first.
ECHO_DEV void hist16_add_peeled(uint32_t *h, uint32_t bin, bool act) {
  const uint64_t m_act = __ballot(act);
  if (!m_act) return;
  const int leader = __ffsll(static_cast<unsigned long long>(m_act)) - 1;
  const uint32_t lead = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), leader));
  const uint64_t same = __ballot(act && bin == lead);
  if (lane_id() == leader)
    atomicAdd(&h[lead >> 1], static_cast<uint32_t>(__popcll(same)) << ((lead & 1u) * 16));
  if (act && bin != lead) atomicAdd(&h[bin >> 1], 1u << ((bin & 1u) * 16));
}

// Block-wide min of lo and max of hi (NT threads, tmp >= 2 * NT / 64 words).
template <int NT>
ECHO_DEV void block_min_max(uint32_t &lo, uint32_t &hi, uint32_t *tmp) {
  constexpr int NW = NT / 64;
  lo = wave_min(lo);
  hi = wave_max(hi);
  const int w = threadIdx.x >> 6;
  if (lane_id() == 0) { tmp[w] = lo; tmp[NW + w] = hi; }
  __syncthreads();
  lo = tmp[0];
  hi = tmp[NW];
#pragma unroll
  for (int i = 1; i < NW; ++i) { lo = min(lo, tmp[i]); hi = max(hi, tmp[NW + i]); }
  __syncthreads();
}

// Block-wide min of lo, max of hi and sum of cnt (NT threads, tmp >= 3 * NT / 64 words).
template <int NT>
ECHO_DEV void block_min_max_cnt(uint32_t &lo, uint32_t &hi, uint32_t &cnt, uint32_t *tmp) {
  constexpr int NW = NT / 64;
  lo = wave_min(lo);
  hi = wave_max(hi);
  cnt = wave_sum(cnt);
  const int w = threadIdx.x >> 6;
  if (lane_id() == 0) { tmp[w] = lo; tmp[NW + w] = hi; tmp[2 * NW + w] = cnt; }
  __syncthreads();
  lo = tmp[0];
  hi = tmp[NW];
  cnt = tmp[2 * NW];
#pragma unroll
  for (int i = 1; i < NW; ++i) { lo = min(lo, tmp[i]); hi = max(hi, tmp[NW + i]); cnt += tmp[2 * NW + i]; }
  __syncthreads();
}

// One bin per active lane added to (SUB: subtracted from) the global fine and coarse
// histograms directly, the wave's most common bin (the first active lane's) in one atomic.
template <bool SUB>
ECHO_DEV void hist_global_add_peeled(uint32_t *fine, uint32_t *coarse, uint32_t bin, bool act) {
  const uint64_t m_act = __ballot(act);
  if (!m_act) return;
  const int leader = __ffsll(static_cast<unsigned long long>(m_act)) - 1;
  const uint32_t lead = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), leader));
  const uint32_t n = static_cast<uint32_t>(__popcll(__ballot(act && bin == lead)));
  const bool own = act && bin != lead;
  const uint32_t b = lane_id() == leader ? lead : bin, v = lane_id() == leader ? n : 1u;
  if (lane_id() == leader || own) {
    if (SUB) { atomicSub(&fine[hist_at(b)], v); atomicSub(&coarse[hist_at(b >> 5)], v); }
    else { atomicAdd(&fine[hist_at(b)], v); atomicAdd(&coarse[hist_at(b >> 5)], v); }
  }
}

// Bins a workgroup adds with direct global atomics rather than through its LDS histogram: the
// LDS path clears, fills and scans a window of the bin range, a fixed cost of several
// barriers that few bins do not repay (measured on MI355X in the decode step's top-k finish).
constexpr uint32_t HIST_DIRECT_MAX = 512;

// Adds (SUB: subtracts) a workgroup's priority bins to the global fine/coarse histograms: the
// bins are counted in LDS first (h: HW words of two 16-bit counters, HW a multiple of 16;
// bins[i] == 0xFFFFFFFF for none) and only non-empty bins reach global memory; 16 consecutive
// lanes sum one coarse bin.  A bin range wider than the LDS window is done in several passes.
// A workgroup with at most HIST_DIRECT_MAX bins adds them directly instead.  NT threads; tmp
// >= 3 * NT / 64 words.
template <int NT, int NB, bool SUB, int HW>
ECHO_DEV void hist_flush_bins(const uint32_t (&bins)[NB], uint32_t *h, uint32_t *tmp, uint32_t *fine,
                              uint32_t *coarse) {
  static_assert(HW % 16 == 0, "whole coarse bins per pass");
  uint32_t lo = 0xFFFFFFFFu, hi = 0, cnt = 0;
#pragma unroll
  for (int i = 0; i < NB; ++i)
    if (bins[i] != 0xFFFFFFFFu) { lo = min(lo, bins[i]); hi = max(hi, bins[i]); ++cnt; }
  block_min_max_cnt<NT>(lo, hi, cnt, tmp);
  if (lo > hi) return;                                  // uniform: no bin in this workgroup
  if (cnt <= HIST_DIRECT_MAX) {                         // uniform
#pragma unroll
    for (int i = 0; i < NB; ++i) hist_global_add_peeled<SUB>(fine, coarse, bins[i], bins[i] != 0xFFFFFFFFu);
    return;
  }
  const int w_lo = static_cast<int>(lo >> 1) & ~15, w_hi = static_cast<int>(hi >> 1) | 15;
  for (int base = w_lo; base <= w_hi; base += HW) {
    const int top = min(w_hi, base + HW - 1);           // words [base, top] in this pass
    for (int w = static_cast<int>(threadIdx.x); w <= top - base; w += NT) h[w] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int w = static_cast<int>(bins[i] >> 1);
      const bool in = bins[i] != 0xFFFFFFFFu && w >= base && w <= top;
      hist16_add_peeled(h, bins[i] - 2u * static_cast<uint32_t>(base), in);
    }
    __syncthreads();
    for (int w0 = base; w0 <= top; w0 += NT) {
      const int w = w0 + static_cast<int>(threadIdx.x);
      const uint32_t v = w <= top ? h[w - base] : 0u;
      const uint32_t a = v & 0xFFFFu, b = v >> 16;
      if (a) { if (SUB) atomicSub(&fine[hist_at(2 * w)], a); else atomicAdd(&fine[hist_at(2 * w)], a); }
      if (b) { if (SUB) atomicSub(&fine[hist_at(2 * w + 1)], b); else atomicAdd(&fine[hist_at(2 * w + 1)], b); }
      const uint32_t sum = row16_incl_scan(a + b);     // lane 15 of the row: the coarse bin's total
      if ((threadIdx.x & 15) == 15 && sum) {
        if (SUB) atomicSub(&coarse[hist_at(w >> 4)], sum); else atomicAdd(&coarse[hist_at(w >> 4)], sum);
      }
    }
    __syncthreads();
  }
}

ECHO_DEV bool is_protected(const uint32_t *prot, int32_t slot) {
  return (prot[slot >> 5] >> (slot & 31)) & 1u;
}

// ---------------------------------------------------------------- lookup of one entry
// Returns the slot of a hit (after setting its protection bit), INF for a miss, or -1 for a
// bad index (status bit set).
ECHO_DEV int32_t lookup_entry(const PoolArgs &P, const PoolFastWs &W, int32_t h, int32_t slot) {
  if (h < 0 || h >= P.n_host) {
    atomicOr(P.status, ECHO_ST_BAD_HOST);
    return -1;
  }
  if (slot == INF) return INF;
  if (slot < 0 || slot >= P.n_gpu) {
    atomicOr(P.status, ECHO_ST_BAD_HOST);
    return -1;
  }
  atomicOr(&W.prot[slot >> 5], 1u << (slot & 31));
  return slot;
}


// ---------------------------------------------------------------- pool statistics of one chunk
// Slots [c*PF_CH, (c+1)*PF_CH) (PF_T threads, 16 slots each): the free ones are added to
// W.counters[0], the priority bins of the occupied ones (EXCL_PROT: only the unprotected ones)
// to W.fine / W.coarse through an LDS histogram.  lds: STATS_LDS_WORDS words.
template <bool EXCL_PROT>
ECHO_DEV void stats_chunk(const PoolArgs &P, const PoolFastWs &W, int32_t step_id, int32_t c,
                          uint32_t *lds) {
  uint32_t *h = lds, *tmp = lds + STATS_HW;
  const int t = threadIdx.x;
  constexpr uint32_t NONE = 0xFFFFFFFFu;
  uint32_t bin[16];
  uint32_t nf = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int32_t s0 = c * PF_CH + j * 4 * PF_T + t * 4;
    uint32_t fw, pb = 0;
    int4 pr;
    if (s0 + 3 < P.n_gpu) {
      fw = *reinterpret_cast<const uint32_t *>(P.free_ + s0);
      pr = *reinterpret_cast<const int4 *>(P.priority + s0);
    } else {
      fw = 0xFFFFFFFFu;
      pr = int4{0, 0, 0, 0};
      for (int e = 0; e < 4; ++e)
        if (s0 + e < P.n_gpu) {
          fw = (fw & ~(0xFFu << (8 * e))) | (static_cast<uint32_t>(P.free_[s0 + e]) << (8 * e));
          (&pr.x)[e] = P.priority[s0 + e];
        }
    }
    if (EXCL_PROT && s0 < P.n_gpu) pb = (W.prot[s0 >> 5] >> (s0 & 31)) & 0xFu;   // s0 % 4 == 0: one word
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t f = (fw >> (8 * e)) & 0xFFu;
      nf += f == 1;
      bin[4 * j + e] = NONE;
      if (f == 0 && !((pb >> e) & 1u)) bin[4 * j + e] = prio_bin((&pr.x)[e], step_id);
    }
  }
  nf = block_sum<PF_T>(nf, tmp);
  if (t == 0 && nf) atomicAdd(&W.counters[0], static_cast<int32_t>(nf));
  hist_flush_bins<PF_T, 16, false, STATS_HW>(bin, h, tmp, W.fine, W.coarse);
}

// ---------------------------------------------------------------- prefetch gather of one request
constexpr int PG_THREADS = 256;
constexpr int PG_BATCH = 128;
constexpr int PG_ROUND = 32;                                  // rows per round of host reads
constexpr int PG_PER = PG_ROUND * (ROW * 2 / 16) / PG_THREADS;  // 16-byte reads per thread = 9
static_assert(PG_PER * PG_THREADS == PG_ROUND * (ROW * 2 / 16), "whole rows per round");
constexpr int PG_LDS_WORDS = 2 * PG_BATCH + 48 + 2;

// Request r's candidates take the next free slots (in list order) and their rows are copied
// from host memory; a candidate that became resident meanwhile is skipped (its reserved slot
// stays free).  PG_THREADS threads; lds: PG_LDS_WORDS words.
ECHO_DEV void gather_request(const GatherArgs &G, int r, uint32_t *lds) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  constexpr int UNITS = ROW * 2 / 16;    // 72 x 16 B per row
  int32_t *s_host = reinterpret_cast<int32_t *>(lds), *s_slot = s_host + PG_BATCH;
  uint32_t *tmp = lds + 2 * PG_BATCH;
  int32_t *s_bn = reinterpret_cast<int32_t *>(tmp + 48);
  if (*(volatile const int32_t *)G.status) return;
  const int32_t cnt = min(G.cand_cnt[r], G.cap);
  if (cnt <= 0) return;
  if (threadIdx.x == 0) {
    const int32_t avail = G.free_count[0];
    const int32_t b = atomicAdd(&G.free_count[1], cnt);
    s_bn[0] = b;
    s_bn[1] = max(0, min(cnt, avail - b));
    if (s_bn[1] > 0) atomicAdd(G.n_prefetched, s_bn[1]);
  }
  __syncthreads();
  const int32_t n = s_bn[1], base = s_bn[0];
  const int64_t kb = G.key_begin[r];
  const v4i *src = reinterpret_cast<const v4i *>(G.host_kv);
  v4i *dst = reinterpret_cast<v4i *>(G.gpu_kv);
  uint32_t n_ok = 0;
  for (int32_t c0 = 0; c0 < n; c0 += PG_BATCH) {
    const int m = min(PG_BATCH, n - c0);
    for (int t = threadIdx.x; t < m; t += PG_THREADS) {
      const int32_t tok = G.cand[static_cast<int64_t>(r) * G.cap + c0 + t];
      const int32_t h = G.req_to_host[kb + tok];
      const int32_t slot = G.free_list[base + c0 + t];
      int32_t ok_h = -1;
      if (h >= 0 && h < G.n_host && slot >= 0 && slot < G.n_gpu && G.host_to_gpu[h] == INF) {
        G.free_[slot] = 0;
        G.to_host[slot] = h;
        G.host_to_gpu[h] = slot;
        G.priority[slot] = 0;
        ok_h = h;
        ++n_ok;
      }
      s_host[t] = ok_h;
      s_slot[t] = slot;
    }
    __syncthreads();
    // rows in rounds of PG_ROUND, every host read of a round in flight before its first store
    for (int r0 = 0; r0 < m; r0 += PG_ROUND) {
      v4i v[PG_PER];
      int64_t d_off[PG_PER];
#pragma unroll
      for (int i = 0; i < PG_PER; ++i) {
        const int u = threadIdx.x + i * PG_THREADS;
        const int t = r0 + u / UNITS, part = u % UNITS;
        d_off[i] = -1;
        if (t < m && s_host[t] >= 0) {
          v[i] = __builtin_nontemporal_load(src + static_cast<int64_t>(s_host[t]) * UNITS + part);
          d_off[i] = static_cast<int64_t>(s_slot[t]) * UNITS + part;
        }
      }
#pragma unroll
      for (int i = 0; i < PG_PER; ++i)
        if (d_off[i] >= 0) dst[d_off[i]] = v[i];
    }
    __syncthreads();
  }
  if (G.st_free) {          // the new slots are occupied with priority 0 (pool-step statistics)
    n_ok = block_sum<PG_THREADS>(n_ok, tmp);
    if (threadIdx.x == 0 && n_ok) {
      const uint32_t b = prio_bin(0, stamp_of(G.stamp));
      atomicSub(G.st_free, static_cast<int32_t>(n_ok));
      atomicAdd(&G.st_fine[hist_at(b)], n_ok);
      atomicAdd(&G.st_coarse[hist_at(b >> 5)], n_ok);
    }
  }
}

constexpr int SIDE_LDS_WORDS = STATS_LDS_WORDS > PG_LDS_WORDS ? STATS_LDS_WORDS : PG_LDS_WORDS;

// Runs block b's side work if b < n_stats + n_gather; returns whether it did.
ECHO_DEV bool side_work(const SideWork &S, int b, uint32_t *lds) {
  static_assert(PF_T == PG_THREADS, "side work shares one block size");
  if (b < S.n_stats) {
    stats_chunk<false>(S.P, S.W, stamp_of(S.stamp), b, lds);
    return true;
  }
  if (b < S.n_stats + S.n_gather) {
    gather_request(S.G, b - S.n_stats, lds);
    return true;
  }
  return false;
}


// ---------------------------------------------------------------- recall staging
// The host reads of a request's misses are spread over three launches so that the link works
// through all of them: the top-k finish launch reads the first STAGE_F16/16 of the misses the
// split found (rows [0, stage_cut_f)), evict-1 reads up to STAGE_E16/16 of all the request's
// misses (rows [stage_cut_f, stage_cut_e)), evict-2 the rest.  Measured on MI355X (decode
// step, 8 x 65536 tokens): 14/14 gives 106.9 us against 107.8 for 12/14, 108.7 for 16/16, 109.2
// for 10/13 and 109.5 for 12/16; at 64 x 131072 tokens the shares move the step by under 0.3%.
constexpr int STAGE_F16 = 14, STAGE_E16 = 14;
ECHO_DEV int32_t stage_cut_f(int32_t a) { return (a * STAGE_F16 + 15) / 16; }
ECHO_DEV int32_t stage_cut_e(int32_t a, int32_t total) {
  return max(stage_cut_f(a), min(total, (total * STAGE_E16 + 15) / 16));
}

// Copies staging rows r*k + i, i in [i0, i0 + ROWS) and in [lo, hi), from host memory:
// stage[r*k + i] = host_kv[stage_h[r*k + i]] (NT threads, ROWS * 72 / NT sixteen-byte loads
// each, all in flight before the first store).
template <int NT, int ROWS>
ECHO_DEV void stage_rows(const uint16_t *__restrict__ host_kv, uint16_t *__restrict__ stage,
                         const int32_t *__restrict__ stage_h, const int32_t *status, int32_t k,
                         int32_t n_host, int r, int32_t i0, int32_t lo, int32_t hi) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  constexpr int UNITS = ROW * 2 / 16;
  constexpr int PER = ROWS * UNITS / NT;
  static_assert(PER * NT == ROWS * UNITS, "whole rows per block");
  if (*(volatile const int32_t *)status) return;
  lo = max(lo, i0);
  hi = min(min(hi, i0 + ROWS), k);
  if (lo >= hi) return;
  const v4i *src = reinterpret_cast<const v4i *>(host_kv);
  v4i *dst = reinterpret_cast<v4i *>(stage);
  const int64_t e0 = static_cast<int64_t>(r) * k;
  v4i v[PER];
  int64_t d_off[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int u = threadIdx.x + m * NT;
    const int32_t i = i0 + u / UNITS;
    const int part = u % UNITS;
    d_off[m] = -1;
    if (i >= lo && i < hi) {
      const int32_t h = stage_h[e0 + i];
      if (h >= 0 && h < n_host) {
        v[m] = __builtin_nontemporal_load(src + static_cast<int64_t>(h) * UNITS + part);
        d_off[m] = (e0 + i) * UNITS + part;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < PER; ++m)
    if (d_off[m] >= 0) dst[d_off[m]] = v[m];
}

}  // namespace echo
