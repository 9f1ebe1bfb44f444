// Guaranteed residency of the selected tokens (ECHO review page §5.1 metadata; §5.2 free,
// allocate and the lookup half of recall) as a few multi-workgroup kernels with every count
// on the device.  Canonical rule (several results would be correct; this one is the
// documented one): protect the slots that hold a selected token; need = #miss - #free; evict
// the `need` unprotected occupied slots with the smallest (priority, slot); the i-th miss (in
// request, token order) takes the i-th free slot in ascending slot order.
//
//   lookup   per selected entry: host index -> slot; a hit sets the slot's bit in a
//            protection bitmap, a miss goes to an ordered per-request list.  (The decode step
//            fuses this into the top-k finish kernel.)
//   stats    per 4096-slot chunk: free count, and a 32768-bin histogram (plus a 1024-bin
//            coarse one) of the evictable (occupied, unprotected) slots' priorities under a
//            monotone "log-age" code relative to the step stamp (ages below 512 get a bin
//            each, older ones bins 1/512 of an octave wide).  Each workgroup counts its chunk in
//            LDS (16-bit counters) and adds only its non-empty bins to the global histograms:
//            priorities are step stamps, so whole chunks share a few bins and per-slot global
//            atomics would serialise on them.
//   evict-1  multi-workgroup: the misses are laid out in global order; every slot chunk
//            finds the threshold bin from the histograms, evicts its unprotected slots below
//            it (a set: order does not matter) and lists the threshold-bin slots in slot order.
//   evict-2  multi-workgroup: every chunk resolves the threshold-bin list exactly (radix
//            digits on the keys, ties to the lower slot) - the same result in every workgroup
//            - evicts its own share, and allocates its free slots to the misses from a prefix
//            over the chunks' free counts.  Entry workgroups stamp the hits' priorities and pad
//            the fixed-length lists.
// Eviction and allocation touch metadata only; rows are copied by the recall gather.
#include <algorithm>
#include <mutex>

#include "internal.hpp"
#include "pool_common.cuh"

namespace echo {

constexpr int PF_RES_T = 1024;                // threads of the resolving workgroups
constexpr int PF_CAP = 8192;                  // threshold-bin slots resolved in LDS

// ---------------------------------------------------------------- workspace
void pool_fast_ws_layout(int32_t n_rows, int32_t k, int32_t n_gpu, void *base, PoolFastWs *w,
                         size_t *bytes) {
  auto al = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  const int32_t n_chunks = std::max(1, (n_gpu + PF_CH - 1) / PF_CH);
  const int64_t n_ent = static_cast<int64_t>(n_rows) * k;
  size_t off = 0;
  auto take = [&](size_t b) { size_t o = off; off += al(b); return o; };
  // zeroed region first (one fill per step): counters, histograms, protection bits
  const size_t o_cnt = take(16 * 4), o_fine = take(PF_HIST_WORDS * 4), o_coarse = take(PF_HIST_WORDS * 4),
               o_prot = take(static_cast<size_t>((n_gpu + 31) / 32) * 4),
               o_sa = take(static_cast<size_t>(n_rows) * 4);
  const size_t zero_end = off;
  const size_t o_rmc = take(static_cast<size_t>(n_rows) * 4),
               o_rmh = take(static_cast<size_t>(n_ent) * 4), o_rmj = take(static_cast<size_t>(n_ent) * 4),
               o_rms = take(static_cast<size_t>(n_ent) * 4), o_sb = take(static_cast<size_t>(n_rows) * 4),
               o_sh = take(static_cast<size_t>(n_ent) * 4),
               o_cf = take(static_cast<size_t>(n_chunks) * 4), o_cc = take(static_cast<size_t>(n_chunks) * 4),
               o_cand = take(static_cast<size_t>(n_chunks) * PF_CH * 8),
               o_me = take(static_cast<size_t>(n_ent) * 4), o_ms = take(static_cast<size_t>(n_ent) * 4);
  *bytes = off;
  w->n_chunks = n_chunks;
  w->zero_words = static_cast<int64_t>(zero_end / 4);
  w->reserve = 0;
  if (base) {
    char *b = static_cast<char *>(base);
    w->counters = reinterpret_cast<int32_t *>(b + o_cnt);
    w->fine = reinterpret_cast<uint32_t *>(b + o_fine);
    w->coarse = reinterpret_cast<uint32_t *>(b + o_coarse);
    w->prot = reinterpret_cast<uint32_t *>(b + o_prot);
    w->stage_a = reinterpret_cast<uint32_t *>(b + o_sa);
    w->row_miss_cnt = reinterpret_cast<uint32_t *>(b + o_rmc);
    w->row_miss_h = reinterpret_cast<int32_t *>(b + o_rmh);
    w->row_miss_j = reinterpret_cast<int32_t *>(b + o_rmj);
    w->row_miss_s = reinterpret_cast<int32_t *>(b + o_rms);
    w->stage_b = reinterpret_cast<uint32_t *>(b + o_sb);
    w->stage_h = reinterpret_cast<int32_t *>(b + o_sh);
    w->chunk_free = reinterpret_cast<uint32_t *>(b + o_cf);
    w->chunk_cand = reinterpret_cast<uint32_t *>(b + o_cc);
    w->cand = reinterpret_cast<uint64_t *>(b + o_cand);
    w->miss_entry = reinterpret_cast<int32_t *>(b + o_me);
    w->miss_stage = reinterpret_cast<int32_t *>(b + o_ms);
    w->base = base;
  }
}

size_t pool_fast_ws_bytes(int32_t n_rows, int32_t k, int32_t n_gpu) {
  PoolFastWs w;
  size_t b;
  pool_fast_ws_layout(n_rows, k, n_gpu, nullptr, &w, &b);
  return b;
}

// ---------------------------------------------------------------- stats (after the lookup)
// EXCL_PROT: leave protected slots out (stats taken after the lookup).  Without it the
// histogram counts every occupied slot and the lookup subtracts the slots it protects.
template <bool EXCL_PROT>
__global__ __launch_bounds__(PF_T) void pool_stats_kernel(PoolArgs P, PoolFastWs W, Stamp stamp) {
  __shared__ uint32_t lds[STATS_LDS_WORDS];
  stats_chunk<EXCL_PROT>(P, W, stamp_of(stamp), blockIdx.x, lds);
}

// Standalone lookup (echo_pool_lookup_alloc): one 1024-thread workgroup per request, entries in
// order; misses go to the request's ordered list.
__global__ __launch_bounds__(PF_RES_T) void pool_lookup_rows_kernel(
    PoolArgs P, PoolFastWs W, const int32_t *__restrict__ idx, const int64_t *__restrict__ key_begin,
    const int32_t *__restrict__ req_to_host, int64_t n_k, int32_t k, int32_t *__restrict__ topk_slot) {
  __shared__ uint32_t tmp[48];
  const int r = blockIdx.x;
  uint32_t n_miss = 0;
  for (int32_t j0 = 0; j0 < k; j0 += PF_RES_T) {
    const int32_t j = j0 + threadIdx.x;
    const int32_t s = j < k ? idx[static_cast<int64_t>(r) * k + j] : -1;
    bool has = false;
    int32_t h = -1, slot = -1, res = -1;
    if (s >= 0) {
      const int64_t tok = key_begin[r] + s;
      if (tok < 0 || tok >= n_k) {
        atomicOr(P.status, ECHO_ST_BAD_HOST);
      } else {
        h = req_to_host[tok];
        has = true;
      }
    }
    if (has && h >= 0 && h < P.n_host) slot = P.host_to_gpu[h];
    if (has) res = lookup_entry(P, W, h, slot);
    const bool miss = res == INF;
    uint32_t tot;
    const uint32_t pos = n_miss + block_excl_scan<PF_RES_T>(miss ? 1u : 0u, tmp, &tot);
    if (miss) {
      W.row_miss_h[static_cast<int64_t>(r) * k + pos] = h;
      W.row_miss_j[static_cast<int64_t>(r) * k + pos] = j;
      W.row_miss_s[static_cast<int64_t>(r) * k + pos] = r * k + static_cast<int32_t>(pos);
    }
    if (j < k) topk_slot[static_cast<int64_t>(r) * k + j] = (res >= 0 && res != INF) ? res : -1;
    n_miss += tot;
  }
  if (threadIdx.x == 0) W.row_miss_cnt[r] = n_miss;
}

// ---------------------------------------------------------------- step state
// counters[] slots written by evict-1 (chunk 0) for evict-2
constexpr int CT_FB = 2, CT_BELOW = 3, CT_NMISS = 4, CT_NEED = 5, CT_ABORT = 6;

struct StepState {
  uint32_t n_miss, must, need, evictable, fb, below;
  bool abort;
};

// Totals, the abort decision and the threshold fine bin (the bin holding the need-th smallest
// evictable priority, with the count of evictable slots in lower bins).  PF_T threads; every
// independent global load is issued before the first wait.
ECHO_DEV StepState step_pick(const PoolArgs &P, const PoolFastWs &W, int32_t n_rows, uint32_t *tmp) {
  constexpr int PER = PF_COARSE / PF_T;
  static_assert(PER == 4, "four coarse bins per thread");
  const int t = threadIdx.x;
  uint32_t nm = 0;
  for (int r = t; r < n_rows; r += PF_T) nm += W.row_miss_cnt[r];
  const uint4 cv{W.coarse[hist_at(t * PER)], W.coarse[hist_at(t * PER + 1)], W.coarse[hist_at(t * PER + 2)],
                 W.coarse[hist_at(t * PER + 3)]};
  const int32_t status = *(volatile int32_t *)P.status;
  const uint32_t n_free = static_cast<uint32_t>(W.counters[0]);
  const uint32_t local = cv.x + cv.y + cv.z + cv.w;
  StepState s;
  const uint32_t before = block_excl_scan<PF_T>(local, tmp, &s.evictable);
  s.n_miss = block_sum<PF_T>(nm, tmp);
  // must: evictions the misses need; need: those plus the ones that leave W.reserve slots free
  // for the next step's prefetch, as far as evictable slots allow
  const uint32_t want = s.n_miss + W.reserve;
  s.must = s.n_miss > n_free ? s.n_miss - n_free : 0u;
  s.need = min(want > n_free ? want - n_free : 0u, s.evictable);
  s.abort = status != 0 || s.must > s.evictable;
  s.fb = 0xFFFFFFFFu;
  s.below = 0;
  if (s.abort || s.need == 0) return s;
  const uint32_t need = s.need;
  if (before < need && need <= before + local) {
    uint32_t cum = before;
    int cb = t * PER;
    const uint32_t c4[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (cum < need && need <= cum + c4[i]) { cb = t * PER + i; break; }
      cum += c4[i];
    }
    tmp[40] = static_cast<uint32_t>(cb);
    tmp[41] = cum;
  }
  __syncthreads();
  if (t < 64) {
    const uint32_t cb = tmp[40], cum = tmp[41];
    const uint32_t v = t < 32 ? W.fine[hist_at(cb * 32 + t)] : 0u;
    const uint32_t inc = wave_incl_scan(v);
    if (t < 32 && cum + inc - v < need && need <= cum + inc) {
      tmp[42] = cb * 32 + t;
      tmp[43] = cum + inc - v;
    }
  }
  __syncthreads();
  s.fb = tmp[42];
  s.below = tmp[43];
  __syncthreads();
  return s;
}

// The same state as published by evict-1.
ECHO_DEV StepState step_read(const PoolFastWs &W) {
  StepState s;
  s.fb = static_cast<uint32_t>(W.counters[CT_FB]);
  s.below = static_cast<uint32_t>(W.counters[CT_BELOW]);
  s.n_miss = static_cast<uint32_t>(W.counters[CT_NMISS]);
  s.need = static_cast<uint32_t>(W.counters[CT_NEED]);
  s.abort = W.counters[CT_ABORT] != 0;
  s.evictable = 0;
  return s;
}

ECHO_DEV void evict_slot(const PoolArgs &P, int32_t slot) {
  const int32_t h = P.to_host[slot];
  if (h >= 0 && h < P.n_host) P.host_to_gpu[h] = INF;
  P.to_host[slot] = INF;
  P.priority[slot] = -1;
  P.free_[slot] = 1;                       // the row stays: the host holds the backup
}

// ---------------------------------------------------------------- evict-1
// blocks [0, n_rows): lay the misses out in global order; blocks [n_rows, n_rows + n_chunks):
// slot chunks.
__global__ __launch_bounds__(PF_T) void pool_evict1_kernel(PoolArgs P, PoolFastWs W, int32_t n_rows,
                                                           int32_t k, Stamp stamp,
                                                           int32_t *__restrict__ miss_host,
                                                           StageArgs SA) {
  const int32_t step_id = stamp_of(stamp);
  __shared__ uint32_t tmp[48];
  __shared__ uint32_t gscan[4 * (PF_T / 64) + PF_T / 64 + 2];
  if (static_cast<int>(blockIdx.x) >= n_rows + W.n_chunks) {
    // recall staging, the middle share of every request's misses, 32 staging rows per block
    const int u = blockIdx.x - n_rows - W.n_chunks, per = (k + 31) / 32, r = u / per;
    const int32_t a = static_cast<int32_t>(W.stage_a[r]), tot = a + static_cast<int32_t>(W.stage_b[r]);
    const int32_t lo = stage_cut_f(a), hi = stage_cut_e(a, tot);
    stage_rows<PF_T, 32>(SA.host_kv, SA.stage, W.stage_h, P.status, k, P.n_host, r, lo + (u % per) * 32, lo, hi);
    return;
  }
  if (static_cast<int>(blockIdx.x) < n_rows) {
    const int r = blockIdx.x;
    uint32_t before = 0;
    for (int q = threadIdx.x; q < r; q += PF_T) before += W.row_miss_cnt[q];
    before = block_sum<PF_T>(before, tmp);
    const uint32_t cnt = W.row_miss_cnt[r];
    for (uint32_t i = threadIdx.x; i < cnt; i += PF_T) {
      miss_host[before + i] = W.row_miss_h[static_cast<int64_t>(r) * k + i];
      W.miss_entry[before + i] = r * k + W.row_miss_j[static_cast<int64_t>(r) * k + i];
      W.miss_stage[before + i] = W.row_miss_s[static_cast<int64_t>(r) * k + i];
    }
    return;
  }
  const int32_t c = blockIdx.x - n_rows;
  const int t = threadIdx.x;
  // the chunk's slots (16 per thread: slot c*PF_CH + 4*PF_T*j + 4*t + e), loaded before the
  // step state is known
  uint32_t fre[4], pw[4];
  int32_t pr[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int32_t s0 = c * PF_CH + j * 4 * PF_T + t * 4;
    pw[j] = s0 < P.n_gpu ? (W.prot[s0 >> 5] >> (s0 & 31)) & 0xFu : 0xFu;   // s0 % 4 == 0
    if (s0 + 3 < P.n_gpu) {
      fre[j] = *reinterpret_cast<const uint32_t *>(P.free_ + s0);
      const int4 v = *reinterpret_cast<const int4 *>(P.priority + s0);
      pr[j][0] = v.x; pr[j][1] = v.y; pr[j][2] = v.z; pr[j][3] = v.w;
    } else {
      fre[j] = 0xFFFFFFFFu;
      for (int e = 0; e < 4; ++e) {
        pr[j][e] = 0;
        if (s0 + e < P.n_gpu) {
          fre[j] = (fre[j] & ~(0xFFu << (8 * e))) | (static_cast<uint32_t>(P.free_[s0 + e]) << (8 * e));
          pr[j][e] = P.priority[s0 + e];
        }
      }
    }
  }
  const StepState st = step_pick(P, W, n_rows, tmp);
  if (c == 0 && t == 0) {                              // for evict-2
    W.counters[CT_FB] = static_cast<int32_t>(st.fb);
    W.counters[CT_BELOW] = static_cast<int32_t>(st.below);
    W.counters[CT_NMISS] = static_cast<int32_t>(st.n_miss);
    W.counters[CT_NEED] = static_cast<int32_t>(st.need);
    W.counters[CT_ABORT] = st.abort ? 1 : 0;
    if (st.abort && st.must > st.evictable && !(*(volatile int32_t *)P.status))
      atomicOr(P.status, ECHO_ST_EXHAUSTED);
  }
  if (st.abort) return;
  // classify: evict below the threshold bin (a set: order does not matter), list the
  // threshold bin in slot order
  uint32_t ev = 0, cand = 0, cc[4], nf = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cc[j] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t f = (fre[j] >> (8 * e)) & 0xFFu;
      if (f == 1) { ++nf; continue; }
      if (f != 0 || st.need == 0 || ((pw[j] >> e) & 1u)) continue;
      const uint32_t b = prio_bin(pr[j][e], step_id);
      if (b < st.fb) {
        ev |= 1u << (4 * j + e);
        ++nf;
      } else if (b == st.fb) {
        cand |= 1u << (4 * j + e);
        ++cc[j];
      }
    }
  }
  // evictions: every to_host load first, then the stores
  int32_t th[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    th[i] = ((ev >> i) & 1u) ? P.to_host[c * PF_CH + (i >> 2) * 4 * PF_T + t * 4 + (i & 3)] : -1;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if ((ev >> i) & 1u) {
      const int32_t slot = c * PF_CH + (i >> 2) * 4 * PF_T + t * 4 + (i & 3);
      if (th[i] >= 0 && th[i] < P.n_host) P.host_to_gpu[th[i]] = INF;
      P.to_host[slot] = INF;
      P.priority[slot] = -1;
      P.free_[slot] = 1;                     // the row stays: the host holds the backup
    }
  uint32_t co[4], tot;
  group_excl_scan<PF_T, 4>(cc, co, gscan, &tot);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t pos = co[j];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((cand >> (4 * j + e)) & 1u) {
        const int32_t slot = c * PF_CH + j * 4 * PF_T + t * 4 + e;
        W.cand[static_cast<int64_t>(c) * PF_CH + pos] =
            (static_cast<uint64_t>(i32_key(pr[j][e])) << 32) | static_cast<uint32_t>(slot);
        ++pos;
      }
  }
  nf = block_sum<PF_T>(nf, tmp);
  if (t == 0) {
    W.chunk_free[c] = nf;
    W.chunk_cand[c] = tot;
  }
}

// ---------------------------------------------------------------- evict-2 + allocation
// Resolve the threshold-bin list (keys ascending, ties by slot) to the k_rem slots that go.
// Every chunk workgroup computes the same answer; it evicts its own and counts every chunk's.
template <bool IN_LDS>
struct CandView {
  const uint64_t *lds;
  const uint64_t *g;
  const uint32_t *chunk_cand;
  const uint32_t *chunk_off;   // LDS: exclusive prefix of chunk_cand
  ECHO_DEV uint64_t at(uint32_t i, int32_t n_chunks) const {
    if (IN_LDS) return lds[i];
    // locate the chunk holding list position i (binary search over the prefix)
    int lo = 0, hi = n_chunks - 1;
    while (lo < hi) {
      const int md = (lo + hi + 1) >> 1;
      if (chunk_off[md] <= i) lo = md; else hi = md - 1;
    }
    return g[static_cast<int64_t>(lo) * PF_CH + (i - chunk_off[lo])];
  }
};

__global__ __launch_bounds__(PF_RES_T) void pool_evict2_kernel(
    PoolArgs P, PoolFastWs W, int32_t n_rows, int32_t k, Stamp stamp,
    int32_t *__restrict__ miss_host, int32_t *__restrict__ miss_slot, int32_t *__restrict__ topk_slot,
    int32_t *__restrict__ n_miss_out, const int32_t *__restrict__ idx, int32_t entry_blocks,
    StageArgs SA) {
  const int32_t step_id = stamp_of(stamp);
  __shared__ uint32_t tmp[48];
  __shared__ uint64_t cl[PF_CAP];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t coff[1024];
  __shared__ uint32_t cev[1024];
  const int t = threadIdx.x;
  const int32_t n_chunks = W.n_chunks;
  const int64_t n_ent = static_cast<int64_t>(n_rows) * k;
  if (static_cast<int>(blockIdx.x) >= n_chunks + entry_blocks) {
    // recall staging, the last share of every request's misses, 128 staging rows per block
    const int u = blockIdx.x - n_chunks - entry_blocks, per = (k + 127) / 128, r = u / per;
    const int32_t a = static_cast<int32_t>(W.stage_a[r]), tot = a + static_cast<int32_t>(W.stage_b[r]);
    const int32_t lo = stage_cut_e(a, tot);
    stage_rows<PF_RES_T, 128>(SA.host_kv, SA.stage, W.stage_h, P.status, k, P.n_host, r,
                              lo + (u % per) * 128, lo, tot);
    return;
  }
  if (static_cast<int>(blockIdx.x) >= n_chunks) {
    // ---- entry workgroups: stamp hits, pad the fixed-length lists
    const StepState st = step_read(W);
    const int64_t e = static_cast<int64_t>(blockIdx.x - n_chunks) * PF_RES_T + t;
    if (st.abort) return;
    if (e < n_ent && idx[e] >= 0) {
      const int32_t sl = topk_slot[e];
      if (sl >= 0 && sl < P.n_gpu && is_protected(W.prot, sl)) P.priority[sl] = step_id;
    }
    const int64_t lim = min(static_cast<int64_t>(P.n_gpu), n_ent);
    if (st.n_miss + e < lim) P.indices_buf[st.n_miss + e] = -1;
    if (st.n_miss + e < n_ent) {
      miss_host[st.n_miss + e] = -1;
      miss_slot[st.n_miss + e] = -1;
    }
    if (e == 0) *n_miss_out = static_cast<int32_t>(st.n_miss);
    return;
  }
  const int32_t c = blockIdx.x;
  const StepState st = step_read(W);
  if (c == 0 && t == 0) *n_miss_out = static_cast<int32_t>(st.n_miss);
  if (st.abort) return;
  // chunk prefixes of the threshold-bin list (n_chunks <= 1024 per resolving pass)
  for (int q = t; q < n_chunks; q += PF_RES_T) cev[q] = 0;
  uint32_t n_c = 0;
  if (st.need > 0) {
    // exclusive prefix of chunk_cand (n_chunks may exceed the block: loop)
    uint32_t run = 0;
    for (int base = 0; base < n_chunks; base += PF_RES_T) {
      const int q = base + t;
      const uint32_t v = q < n_chunks ? W.chunk_cand[q] : 0u;
      uint32_t tot;
      const uint32_t ex = block_excl_scan<PF_RES_T>(v, tmp, &tot);
      if (q < n_chunks) coff[q & 1023] = run + ex;   // n_chunks <= 1024 (checked on the host)
      run += tot;
    }
    n_c = run;
  }
  __syncthreads();
  if (st.need > 0) {
    uint32_t k_rem = st.need - st.below;          // slots of the threshold bin that go
    const bool in_lds = n_c <= PF_CAP;
    if (in_lds) {
      for (uint32_t i = t; i < n_c; i += PF_RES_T) {
        int lo = 0, hi = n_chunks - 1;
        while (lo < hi) { const int md = (lo + hi + 1) >> 1; if (coff[md] <= i) lo = md; else hi = md - 1; }
        cl[i] = W.cand[static_cast<int64_t>(lo) * PF_CH + (i - coff[lo])];
      }
      __syncthreads();
    }
    CandView<true> vl{cl, W.cand, W.chunk_cand, coff};
    CandView<false> vg{cl, W.cand, W.chunk_cand, coff};
    // radix digits over the 32-bit keys of the list
    uint32_t prefix = 0, mask = 0;
    for (int d = 0; d < 3; ++d) {
      const int sh = d == 0 ? 21 : (d == 1 ? 10 : 0);
      const uint32_t dm = d == 2 ? 0x3FFu : 0x7FFu;
      for (int b = t; b < 2048; b += PF_RES_T) hist[b] = 0;
      __syncthreads();
      for (uint32_t i0 = 0; i0 < n_c; i0 += PF_RES_T) {      // uniform trip count per wave
        const uint32_t i = i0 + t;
        const uint32_t key = i < n_c ? static_cast<uint32_t>((in_lds ? vl.at(i, n_chunks) : vg.at(i, n_chunks)) >> 32) : 0u;
        hist_add_peeled(hist, (key >> sh) & dm, i < n_c && (key & mask) == prefix);
      }
      __syncthreads();
      uint32_t lo_cnt = 0;
      const int per = 2048 / PF_RES_T;
      for (int i = 0; i < per; ++i) lo_cnt += hist[t * per + i];
      uint32_t total;
      const uint32_t before = block_excl_scan<PF_RES_T>(lo_cnt, tmp, &total);
      if (before < k_rem && k_rem <= before + lo_cnt) {
        uint32_t cum = before;
        for (int i = 0; i < per; ++i) {
          const uint32_t h = hist[t * per + i];
          if (cum < k_rem && k_rem <= cum + h) { tmp[40] = t * per + i; tmp[41] = cum; break; }
          cum += h;
        }
      }
      __syncthreads();
      const uint32_t b = tmp[40], bl = tmp[41];
      __syncthreads();
      k_rem -= bl;
      prefix |= b << sh;
      mask |= dm << sh;
    }
    const uint32_t kstar = prefix;
    // ordered pass over the list (slot order): keys < K* go, then the first k_rem ties
    uint32_t eq_seen = 0;
    for (uint32_t base = 0; base < n_c; base += PF_RES_T) {
      const uint32_t i = base + t;
      const bool in = i < n_c;
      const uint64_t v = in ? (in_lds ? vl.at(i, n_chunks) : vg.at(i, n_chunks)) : 0ull;
      const uint32_t key = static_cast<uint32_t>(v >> 32);
      const int32_t slot = static_cast<int32_t>(v & 0xFFFFFFFFu);
      uint32_t tot;
      const uint32_t r = eq_seen + block_excl_scan<PF_RES_T>(in && key == kstar, tmp, &tot);
      const bool go = in && (key < kstar || (key == kstar && r < k_rem));
      if (go) {
        const int32_t ch = slot / PF_CH;
        atomicAdd(&cev[ch], 1u);
        if (ch == c) evict_slot(P, slot);
      }
      eq_seen += tot;
    }
  }
  __syncthreads();
  // allocation: free slots of this chunk (after every eviction) in ascending order
  uint32_t base = 0;
  for (int q = t; q < c; q += PF_RES_T) base += W.chunk_free[q] + cev[q];
  base = block_sum<PF_RES_T>(base, tmp);
  if (base >= st.n_miss) return;
  const int32_t s0 = c * PF_CH + t * 4;
  uint32_t fw = 0xFFFFFFFFu;
  if (s0 + 3 < P.n_gpu) fw = *reinterpret_cast<const uint32_t *>(P.free_ + s0);
  else
    for (int e = 0; e < 4; ++e)
      if (s0 + e < P.n_gpu) fw = (fw & ~(0xFFu << (8 * e))) | (static_cast<uint32_t>(P.free_[s0 + e]) << (8 * e));
  uint32_t nf = 0;
  for (int e = 0; e < 4; ++e) nf += ((fw >> (8 * e)) & 0xFFu) == 1;
  uint32_t tot;
  uint32_t rank = base + block_excl_scan<PF_RES_T>(nf, tmp, &tot);
  for (int e = 0; e < 4; ++e) {
    if (((fw >> (8 * e)) & 0xFFu) != 1 || rank >= st.n_miss) continue;
    const int32_t slot = s0 + e;
    const int32_t hh = miss_host[rank];
    P.free_[slot] = 0;
    P.to_host[slot] = hh;
    P.host_to_gpu[hh] = slot;
    P.priority[slot] = step_id;
    P.indices_buf[rank] = slot;
    miss_slot[rank] = slot;
    topk_slot[W.miss_entry[rank]] = slot;
    ++rank;
  }
}

int launch_pool_stats(const echo_pool *pool, const PoolFastWs &W, Stamp stamp, bool excl_prot,
                      hipStream_t st) {
  PoolArgs P{pool->gpu_free, pool->gpu_priority, pool->gpu_to_host, pool->host_to_gpu,
             pool->indices_buf, pool->status, pool->n_gpu, pool->n_host};
  if (excl_prot) pool_stats_kernel<true><<<W.n_chunks, PF_T, 0, st>>>(P, W, stamp);
  else pool_stats_kernel<false><<<W.n_chunks, PF_T, 0, st>>>(P, W, stamp);
  return check_launch("pool_stats");
}

int launch_pool_lookup_rows(const echo_pool *pool, const PoolFastWs &W, const int32_t *idx,
                            const int64_t *key_begin, const int32_t *req_to_host, int64_t n_k,
                            int32_t n_rows, int32_t k, Stamp stamp, int32_t *topk_slot,
                            hipStream_t st) {
  PoolArgs P{pool->gpu_free, pool->gpu_priority, pool->gpu_to_host, pool->host_to_gpu,
             pool->indices_buf, pool->status, pool->n_gpu, pool->n_host};
  if (n_rows > 0)
    pool_lookup_rows_kernel<<<n_rows, PF_RES_T, 0, st>>>(P, W, idx, key_begin, req_to_host, n_k, k,
                                                         topk_slot);
  (void)stamp;                             // the lookup itself stamps nothing
  return check_launch("pool_lookup_rows");
}

int launch_pool_evict(const echo_pool *pool, const PoolFastWs &W, const int32_t *idx, int32_t n_rows,
                      int32_t k, Stamp stamp, int32_t *topk_slot, int32_t *miss_host,
                      int32_t *miss_slot, int32_t *n_miss, uint16_t *stage, hipStream_t st) {
  if (W.n_chunks > 1024) return fail(ECHO_EUNSUPPORTED, "pool: more than 4M slots");
  PoolArgs P{pool->gpu_free, pool->gpu_priority, pool->gpu_to_host, pool->host_to_gpu,
             pool->indices_buf, pool->status, pool->n_gpu, pool->n_host};
  // with a staging area, both launches also read shares of the misses from host memory
  StageArgs SA{pool->host_kv, stage};
  const int s1 = stage ? n_rows * ((k + 31) / 32) : 0;
  const int s2 = stage ? n_rows * ((k + 127) / 128) : 0;
  pool_evict1_kernel<<<n_rows + W.n_chunks + s1, PF_T, 0, st>>>(P, W, n_rows, k, stamp, miss_host, SA);
  const int64_t n_ent = static_cast<int64_t>(n_rows) * k;
  const int entry_blocks = static_cast<int>(std::max<int64_t>(1, (n_ent + PF_RES_T - 1) / PF_RES_T));
  pool_evict2_kernel<<<W.n_chunks + entry_blocks + s2, PF_RES_T, 0, st>>>(
      P, W, n_rows, k, stamp, miss_host, miss_slot, topk_slot, n_miss, idx, entry_blocks, SA);
  return check_launch("pool_evict");
}

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

int launch_pool_step(const echo_pool *pool, const int32_t *idx, const int64_t *key_begin,
                     const int32_t *req_to_host, int64_t n_k, int32_t n_rows, int32_t k,
                     Stamp stamp, int32_t *topk_slot, int32_t *miss_host, int32_t *miss_slot,
                     int32_t *n_miss, void *ws, size_t ws_bytes, hipStream_t st) {
  PoolFastWs W;
  size_t need;
  pool_fast_ws_layout(n_rows, k, pool->n_gpu, ws, &W, &need);
  if (ws_bytes < need) return fail(ECHO_EWORKSPACE, "echo_pool_lookup_alloc: workspace %zu < %zu", ws_bytes, need);
  int rc;
  if ((rc = launch_zero_i32(W.counters, W.zero_words, st))) return rc;
  if ((rc = launch_pool_lookup_rows(pool, W, idx, key_begin, req_to_host, n_k, n_rows, k, stamp,
                                    topk_slot, st)))
    return rc;
  if ((rc = launch_pool_stats(pool, W, stamp, true, st))) return rc;
  return launch_pool_evict(pool, W, idx, n_rows, k, stamp, topk_slot, miss_host, miss_slot, n_miss,
                           nullptr, st);
}

}  // namespace echo

using namespace echo;

static int check_pool(const echo_pool *pool, const char *fn) {
  if (!pool) return fail(ECHO_EINVAL, "%s: NULL pool", fn);
  if (pool->n_gpu < 1 || pool->n_host < 1) return fail(ECHO_EINVAL, "%s: pool sizes must be >= 1", fn);
  if (pool->n_gpu > (1 << 22)) return fail(ECHO_EUNSUPPORTED, "%s: more than 4M GPU slots", fn);
  if (!pool->gpu_free || !pool->gpu_priority || !pool->gpu_to_host || !pool->host_to_gpu ||
      !pool->indices_buf || !pool->status)
    return fail(ECHO_EINVAL, "%s: NULL pool member", fn);
  return ECHO_OK;
}

extern "C" size_t echo_pool_workspace_bytes(int32_t n_rows, int32_t k, int32_t n_gpu) {
  if (n_rows < 0 || k < 0 || n_gpu < 0) return 0;
  return pool_fast_ws_bytes(n_rows, k, n_gpu);
}

extern "C" int echo_pool_lookup_alloc(const echo_pool *pool, const int32_t *idx,
                                      const int64_t *key_begin, const int32_t *req_to_host,
                                      int64_t n_k, int32_t n_rows, int32_t k, int32_t step_id,
                                      int32_t *topk_slot, int32_t *miss_host, int32_t *miss_slot,
                                      int32_t *n_miss, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_pool(pool, "echo_pool_lookup_alloc");
  if (rc) return rc;
  if (n_rows < 0 || k < 1 || k > ECHO_MAX_TOPK || n_k < 0)
    return fail(ECHO_EINVAL, "echo_pool_lookup_alloc: bad n_rows/k/n_k");
  if (static_cast<int64_t>(n_rows) * k > (1LL << 30)) return fail(ECHO_EUNSUPPORTED, "echo_pool_lookup_alloc: too many entries");
  if (!idx || !key_begin || !req_to_host || !topk_slot || !miss_host || !miss_slot || !n_miss || !ws)
    return fail(ECHO_EINVAL, "echo_pool_lookup_alloc: NULL pointer");
  return launch_pool_step(pool, idx, key_begin, req_to_host, n_k, n_rows, k, Stamp{step_id, nullptr}, topk_slot,
                          miss_host, miss_slot, n_miss, ws, ws_bytes, S(stream));
}

// ---------------------------------------------------------------- no-allocation variant
// For callers that cannot allocate (code under graph capture, tight serving loops): the same
// pool step with its workspace in a fixed device array.  Each GPU holds its own copy of the array
// until the process ends; host code reaches it only through the address hipGetSymbolAddress
// gives on that device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[ECHO_STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptr[MAX_DEVICES];                      // per device, set on its first call
}  // namespace

// Device address of the calling device's scratch array (nullptr after setting the error text).
static void *scratch_of_current_device(const char *fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(ECHO_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= MAX_DEVICES) {
    fail(ECHO_EUNSUPPORTED, "%s: device %d outside [0, %d)", fn, dev, MAX_DEVICES);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      fail(ECHO_EHIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
      return nullptr;
    }
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

extern "C" int echo_pool_lookup_alloc_static(const echo_pool *pool, const int32_t *idx,
                                             const int64_t *key_begin, const int32_t *req_to_host,
                                             int64_t n_k, int32_t n_rows, int32_t k, int32_t step_id,
                                             int32_t *topk_slot, int32_t *miss_host,
                                             int32_t *miss_slot, int32_t *n_miss, void *stream) {
  static const char *fn = "echo_pool_lookup_alloc_static";
  int rc = check_pool(pool, fn);
  if (rc) return rc;
  if (n_rows < 0 || k < 1 || k > ECHO_MAX_TOPK || n_k < 0) return fail(ECHO_EINVAL, "%s: bad n_rows/k/n_k", fn);
  if (static_cast<int64_t>(n_rows) * k > (1LL << 30)) return fail(ECHO_EUNSUPPORTED, "%s: too many entries", fn);
  if (!idx || !key_begin || !req_to_host || !topk_slot || !miss_host || !miss_slot || !n_miss)
    return fail(ECHO_EINVAL, "%s: NULL pointer", fn);
  const size_t need = pool_fast_ws_bytes(n_rows, k, pool->n_gpu);
  if (need > ECHO_STATIC_SCRATCH_BYTES)
    return fail(ECHO_EUNSUPPORTED, "%s: %d rows x top-%d over %d GPU slots need %zu bytes of scratch, "
                "more than the fixed %zu (use echo_pool_lookup_alloc with a workspace)", fn, n_rows, k,
                pool->n_gpu, need, static_cast<size_t>(ECHO_STATIC_SCRATCH_BYTES));
  void *ws = scratch_of_current_device(fn);
  if (!ws) return ECHO_EHIP;
  // the step clears the part of the workspace that must start at zero with a kernel of its own
  return launch_pool_step(pool, idx, key_begin, req_to_host, n_k, n_rows, k, Stamp{step_id, nullptr},
                          topk_slot, miss_host, miss_slot, n_miss, ws, ECHO_STATIC_SCRATCH_BYTES,
                          S(stream));
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
