// Scoring and threshold prefetch in one kernel (ECHO review page §6.3: the indexer kernel in
// three stages, a loader, the score computation whose threshold test feeds a bounded queue, and
// a copy stage that moves queued rows from host memory while later keys are still being
// scored, so that the host link works during indexing).
//
// gfx950 form: a workgroup of four scoring waves and one gather wave.
//   loader + MFMA  The scoring waves stream the workgroup's token range in 128-token chunks as
//                  the plain scoring kernel does: the next chunk is fetched into registers
//                  while the current one is multiplied out from a swizzled LDS stage (the
//                  page's separate loader stage is this one-chunk-ahead register fetch).
//                  Tokens scoring above the request's threshold go, in token order, to the
//                  chunk's LDS queue.
//   gather wave    A software pipeline with one step per chunk period: look the queued tokens
//                  of the previous chunk up in req_to_host; a period later look their host
//                  indices up in HostTokenToGPU; a period later claim places for the
//                  non-resident ones from the request's counter; a period later read the
//                  claimed places' slots from the free-slot list; a period later set both maps
//                  and priority 0 and queue the rows.  While the scoring runs, every period it
//                  starts reading one queued row from mapped host memory and stores the row it
//                  started the period before; after the last chunk it finishes the pipeline and
//                  copies the rows still queued eight at a time.
// The gather wave meets the scoring waves only at the chunk barriers.  A gfx950 workgroup
// barrier waits for LDS traffic only, so its host reads stay in flight across barriers: the
// scoring waves wait for the host link only when a read is still outstanding a whole chunk
// period after it was issued.  After the last chunk the gather wave drains its pipeline alone;
// no wave ever waits for another outside the barriers.
//
// The cap.  Request r may prefetch c_r = min(cap, ceil(L_r / cap_div)) rows, the page's bound
// in proportion to the context, scaled down in proportion when the requests' caps add up to more
// than the free slots.  Request r owns c_r consecutive entries of the ascending free-slot list
// (after those of requests < r); its ranges claim places among them first come, first served,
// through one counter per request, as the page's prefetch counter does.  At most 128 rows per
// range (its candidates: the first 128 qualifying tokens).  When a request's candidates fit its
// cap, every one of them moves, so what moves depends on the inputs alone; which of the
// request's slots each one gets depends on timing.
//
// Launches: free slots per 4096-slot chunk (with the pool-step statistics in the decode step)
// -> ascending free-slot list, every request's places and their offset -> the fused kernel ->
// per-step totals.
#include "internal.hpp"
#include "pool_common.cuh"
#include "score_tile.cuh"

namespace echo {

constexpr int FZ_SW = 4;                                // scoring waves
constexpr int FZ_ST = 64 * FZ_SW;                       // scoring threads
constexpr int FZ_THREADS = FZ_ST + 64;                  // + the gather wave
constexpr int FZ_CHUNK = 128;                           // tokens per LDS stage
constexpr int FZ_LOADS = FZ_CHUNK * D / 16 / FZ_ST;     // 16-byte loads per scoring thread = 4
constexpr int FZ_MAXW = ECHO_FUSED_MAX_PER_RANGE;       // rows per range at most (128)
constexpr int FZ_UNITS = ROW * 2 / 16;                  // 16-byte units per latent row = 72
constexpr int FZ_DRAIN = 8;                             // rows per batch once the scoring is over
constexpr int FZ_DRAIN_UNITS = (FZ_DRAIN * FZ_UNITS + 63) / 64;   // 16-byte units per lane = 9
static_assert(FZ_CHUNK <= 128, "a chunk's queue is two entries per lane of the gather wave");
static_assert(FZ_UNITS <= 128, "a row is two 16-byte units per lane of the gather wave");

ECHO_DEV int fz_swz(int tok, int seg) { return tok * 128 + ((seg ^ ((tok >> 1) & 7)) << 4); }

// Request r's cap before scaling, c_r (above), at most n_gpu.
ECHO_DEV int32_t fz_request_cap(int32_t L, int32_t cap, int32_t cap_div, int32_t n_gpu) {
  if (L <= 0) return 0;
  int64_t c = (static_cast<int64_t>(L) + cap_div - 1) / cap_div;
  if (c > cap) c = cap;
  return static_cast<int32_t>(c < n_gpu ? c : n_gpu);
}

struct FusedArgs {
  const float *theta;          // [n_q] threshold (strict >; NaN: none)
  const int32_t *req_to_host;  // [n_k]
  const uint16_t *host_kv;     // [n_host][ROW] mapped host memory
  uint16_t *gpu_kv;            // [n_gpu][ROW]
  uint8_t *free_;
  int32_t *priority, *to_host, *host_to_gpu;
  const int32_t *status;
  int32_t n_gpu, n_host;
  const int32_t *free_list;    // ascending free slots
  const int32_t *counts;       // [0]: length of free_list
  const int32_t *slice_off;    // [n_q] first free_list entry of request r's places
  const int32_t *cap_eff;      // [n_q] request r's places (its cap, scaled to the free slots)
  int32_t *claimed;            // [n_q] places claimed so far (zeroed by the list launch)
  int32_t *demand;             // [n_q] qualifying tokens (zeroed by the list launch)
  int32_t *taken;              // [n_q] rows prefetched (zeroed by the list launch)
  int32_t range;
};

// Pipeline state of the gather wave.  Each lane carries entries e = lane and lane + 64 of a
// chunk's queue.
struct FzA { int32_t tok[2], h[2]; };      // token (-1: none), its host index (in flight)
struct FzB { int32_t h[2], g[2]; };        // host index (-1: none), its slot or INF (in flight)
struct FzC { int32_t h[2], rank[2], base, want; };   // claim: rank among the claimed (-1: none),
                                                     // the counter's old value (lane 0, in flight)
struct FzD { int32_t h[2], slot[2], pos[2], take; }; // slot of the claimed place (in flight), its
                                                     // position in the row queue
template <int P> struct FzParity { static constexpr int value = P; };

template <bool HAS_SCALE, bool HIST>
__global__ __launch_bounds__(FZ_THREADS) void score_fused_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ w, const uint8_t *__restrict__ k,
    const float *__restrict__ k_scale, const int64_t *__restrict__ key_begin,
    const int32_t *__restrict__ key_len, int32_t max_len, int32_t gx, float *__restrict__ scores,
    int64_t ld, FusedArgs F, uint32_t *__restrict__ hist0) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[2][FZ_CHUNK * D];
  __shared__ uint32_t hl[HIST ? 1024 : 1];          // 2048 bins, two 16-bit counters per word
  __shared__ uint8_t qtok[2][FZ_CHUNK];             // queue: token offsets in the chunk, 32 per wave
  __shared__ uint32_t qn[2][FZ_SW];                 // queue length per scoring wave
  __shared__ int32_t ring_h[FZ_MAXW], ring_s[FZ_MAXW];   // rows to copy: host index, slot

  const int b = blockIdx.x;
  const int r = b / gx, x = b % gx;
  const int32_t L = min(max(key_len[r], 0), max_len);
  const int32_t t_begin = x * F.range;
  if (t_begin >= L) return;
  const int32_t t_end = min(L, t_begin + F.range);
  const int n_ch = (t_end - t_begin + FZ_CHUNK - 1) / FZ_CHUNK;
  const int64_t kb = key_begin[r];
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int l = lane_id();

  if (wv < FZ_SW) {
    // ------------------------------------------------------------ scoring waves
    const int tid = threadIdx.x, j = l & 15, g = l >> 4;
    const uint8_t *__restrict__ kr = k + kb * D;
    float *__restrict__ srow = scores + static_cast<int64_t>(r) * ld;
    QOperand qo;
    load_q_operand(q, w, r, qo);
    const float theta = F.theta[r];
    int4 pre[FZ_LOADS];
    auto fetch = [&](int32_t c0) {
#pragma unroll
      for (int m = 0; m < FZ_LOADS; ++m) {
        const int e = tid + m * FZ_ST;
        const int32_t t = c0 + (e >> 3);
        if (t < t_end)
          pre[m] = *reinterpret_cast<const int4 *>(kr + static_cast<int64_t>(t) * D + ((e & 7) << 4));
        else
          pre[m] = int4{0, 0, 0, 0};
      }
    };
    if constexpr (HIST)
      for (int i = tid; i < 1024; i += FZ_ST) hl[i] = 0;   // ordered by the first barrier
    fetch(t_begin);
    for (int c = 0; c < n_ch; ++c) {
      const int32_t c0 = t_begin + c * FZ_CHUNK;
      uint8_t *sb = stage[c & 1];
#pragma unroll
      for (int m = 0; m < FZ_LOADS; ++m) {
        const int e = tid + m * FZ_ST;
        *reinterpret_cast<int4 *>(sb + fz_swz(e >> 3, e & 7)) = pre[m];
      }
      __syncthreads();
      if (c + 1 < n_ch) fetch(c0 + FZ_CHUNK);
      float part[2];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const int tt = wv * 32 + tile * 16 + j;
        const int4 b0 = *reinterpret_cast<const int4 *>(sb + fz_swz(tt, 2 * g));
        const int4 b1 = *reinterpret_cast<const int4 *>(sb + fz_swz(tt, 2 * g + 1));
        part[tile] = reduce_groups(score_tile_partial(qo, v8i{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w}));
      }
      // lanes 0..31 write tokens c0 + 32 wv + lane, in lane order
      const int32_t t_out = c0 + wv * 32 + g * 16 + j;
      const bool writer = g < 2 && t_out < t_end;
      float s_out = (g == 0) ? part[0] : part[1];
      if (writer) {
        if constexpr (HAS_SCALE) s_out *= k_scale[kb + t_out];
        srow[t_out] = s_out;
      }
      const bool over = writer && s_out > theta;
      const uint64_t m_over = __ballot(over);
      if (over)
        qtok[c & 1][wv * 32 + __popcll(m_over & ((1ull << l) - 1ull))] = static_cast<uint8_t>(t_out - c0);
      if (l == 0) qn[c & 1][wv] = static_cast<uint32_t>(__popcll(m_over));
      if constexpr (HIST) hist16_add_peeled(hl, (~f32_key(s_out)) >> 21, writer);
    }
    __syncthreads();                                    // final barrier, met by the gather wave
    if constexpr (HIST) {
      uint32_t *gh = hist0 + static_cast<int64_t>(r) * 2048;
      for (int i = tid; i < 1024; i += FZ_ST) {
        const uint32_t v = hl[i];
        if (v & 0xFFFFu) atomicAdd(&gh[2 * i], v & 0xFFFFu);
        if (v >> 16) atomicAdd(&gh[2 * i + 1], v >> 16);
      }
    }
    return;
  }

  // -------------------------------------------------------------- gather wave
  typedef int v4i __attribute__((ext_vector_type(4)));
  int32_t places = F.cap_eff[r];
  if (*(volatile const int32_t *)F.status) places = 0;            // a failed step moves nothing
  const int64_t off = F.slice_off[r];
  const v4i *__restrict__ src = reinterpret_cast<const v4i *>(F.host_kv);
  v4i *__restrict__ dst = reinterpret_cast<v4i *>(F.gpu_kv);

  FzA A[2];
  FzB Bs[2];
  FzC Cs[2];
  FzD Ds[2];
  v4i cp[2][2];
  int32_t cslot[2] = {-1, -1};
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      A[p].tok[m] = A[p].h[m] = -1;
      Bs[p].h[m] = -1;
      Bs[p].g[m] = 0;
      Cs[p].h[m] = Cs[p].rank[m] = -1;
      Ds[p].h[m] = Ds[p].slot[m] = Ds[p].pos[m] = -1;
      cp[p][m] = v4i{0, 0, 0, 0};
    }
    Cs[p].base = Cs[p].want = Ds[p].take = 0;
  }
  // wanted: places this range has asked for (at most FZ_MAXW, the row queue); queued: rows in
  // the queue; ready: rows whose slot and maps are set; rd: rows whose copy has started
  int32_t wanted = 0, queued = 0, ready = 0, rd = 0, demand = 0;
  const uint64_t below = (1ull << l) - 1ull;

  // One chunk period w, with the pipeline buffers of parity P.
  auto period = [&](auto P, int32_t w) {
    constexpr int p = decltype(P)::value;
    // maps: chunk w - 5's claimed places have their slots (read the period before)
    if (w >= 5 && w - 5 < n_ch) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int32_t h = Ds[p ^ 1].h[m];
        if (h >= 0) {
          const int32_t sl = Ds[p ^ 1].slot[m];
          F.free_[sl] = 0;
          F.to_host[sl] = h;
          F.host_to_gpu[h] = sl;
          F.priority[sl] = 0;
          ring_h[Ds[p ^ 1].pos[m]] = h;
          ring_s[Ds[p ^ 1].pos[m]] = sl;
        }
      }
      ready += Ds[p ^ 1].take;
      __builtin_amdgcn_wave_barrier();     // the queued rows, written by several lanes, are read below
    }
    // slots: chunk w - 4's claim came back; its first `take` places get slots from the list
    if (w >= 4 && w - 4 < n_ch) {
      const int32_t base = __builtin_amdgcn_readlane(Cs[p ^ 1].base, 0);
      const int32_t left = places - base;
      const int32_t take = Cs[p ^ 1].want < left ? Cs[p ^ 1].want : (left > 0 ? left : 0);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int32_t rk = Cs[p ^ 1].rank[m];
        Ds[p].h[m] = -1;
        if (rk >= 0 && rk < take) {
          Ds[p].h[m] = Cs[p ^ 1].h[m];
          Ds[p].pos[m] = queued + rk;
          Ds[p].slot[m] = F.free_list[off + base + rk];
        }
      }
      Ds[p].take = take;
      queued += take;
    }
    // claim: chunk w - 3's non-resident tokens (lookups issued in the two periods before)
    if (w >= 3 && w - 3 < n_ch) {
      bool qual[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) qual[m] = Bs[p ^ 1].h[m] >= 0 && Bs[p ^ 1].g[m] == INF;
      const uint64_t b0 = __ballot(qual[0]), b1 = __ballot(qual[1]);
      const int32_t n0 = static_cast<int32_t>(__popcll(b0)), nq = n0 + static_cast<int32_t>(__popcll(b1));
      const int32_t rk[2] = {static_cast<int32_t>(__popcll(b0 & below)),
                             n0 + static_cast<int32_t>(__popcll(b1 & below))};
      const int32_t room = FZ_MAXW - wanted;
      const int32_t want = places > 0 ? (nq < room ? nq : room) : 0;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        Cs[p].h[m] = Bs[p ^ 1].h[m];
        Cs[p].rank[m] = qual[m] && rk[m] < want ? rk[m] : -1;
      }
      Cs[p].want = want;
      Cs[p].base = 0;
      if (want > 0 && l == 0) Cs[p].base = atomicAdd(&F.claimed[r], want);
      wanted += want;
      demand += nq;
    }
    // copy: while the scoring runs, start reading the next queued row
    cslot[p] = -1;
    if (w <= n_ch && rd < ready) {
      const int32_t h = ring_h[rd];
      cslot[p] = ring_s[rd];
      ++rd;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int u = l + 64 * m;
        if (u < FZ_UNITS) cp[p][m] = __builtin_nontemporal_load(src + static_cast<int64_t>(h) * FZ_UNITS + u);
      }
    }
    // residency: chunk w - 2's host indices (issued the period before) -> HostTokenToGPU
    if (w >= 2 && w - 2 < n_ch) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int32_t h = A[p ^ 1].h[m];
        const bool ok = A[p ^ 1].tok[m] >= 0 && h >= 0 && h < F.n_host;
        Bs[p].h[m] = ok ? h : -1;
        Bs[p].g[m] = ok ? F.host_to_gpu[h] : 0;
      }
    }
    // host index: chunk w - 1's queue -> req_to_host
    if (w >= 1 && w - 1 < n_ch) {
      const int qb = (w - 1) & 1;
      const int32_t p1 = static_cast<int32_t>(qn[qb][0]), p2 = p1 + static_cast<int32_t>(qn[qb][1]);
      const int32_t p3 = p2 + static_cast<int32_t>(qn[qb][2]), n = p3 + static_cast<int32_t>(qn[qb][3]);
      const int32_t c0 = t_begin + (w - 1) * FZ_CHUNK;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int32_t e = l + 64 * m;
        A[p].tok[m] = -1;
        A[p].h[m] = -1;
        if (e < n) {
          const int seg = e < p1 ? 0 : e < p2 ? 1 : e < p3 ? 2 : 3;
          const int32_t base = seg == 0 ? 0 : seg == 1 ? p1 : seg == 2 ? p2 : p3;
          const int32_t tok = c0 + qtok[qb][seg * 32 + (e - base)];
          A[p].tok[m] = tok;
          A[p].h[m] = F.req_to_host[kb + tok];
        }
      }
    }
    // copy: store the row started the period before
    if (cslot[p ^ 1] >= 0) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int u = l + 64 * m;
        if (u < FZ_UNITS) dst[static_cast<int64_t>(cslot[p ^ 1]) * FZ_UNITS + u] = cp[p ^ 1][m];
      }
      cslot[p ^ 1] = -1;
    }
  };
  // Periods 0 .. n_ch - 1 follow the chunk barriers, period n_ch the final one; periods
  // n_ch + 1 .. n_ch + 4 finish the pipeline without barriers (and start no more single rows).
  for (int32_t w = 0;; w += 2) {
    if (w <= n_ch) __syncthreads();
    period(FzParity<0>{}, w);
    if (w >= n_ch + 4) break;
    if (w + 1 <= n_ch) __syncthreads();
    period(FzParity<1>{}, w + 1);
    if (w + 1 >= n_ch + 4) break;
  }
  // The scoring is over: the rows still queued go FZ_DRAIN at a time, all reads in flight
  // before the first store.
  for (int32_t b0 = rd; b0 < ready; b0 += FZ_DRAIN) {
    const int32_t nb = ready - b0 < FZ_DRAIN ? ready - b0 : FZ_DRAIN;
    v4i v[FZ_DRAIN_UNITS];
#pragma unroll
    for (int m = 0; m < FZ_DRAIN_UNITS; ++m) {
      const int u = l + 64 * m, row = u / FZ_UNITS;
      if (row < nb)
        v[m] = __builtin_nontemporal_load(src + static_cast<int64_t>(ring_h[b0 + row]) * FZ_UNITS + u % FZ_UNITS);
    }
#pragma unroll
    for (int m = 0; m < FZ_DRAIN_UNITS; ++m) {
      const int u = l + 64 * m, row = u / FZ_UNITS;
      if (row < nb) dst[static_cast<int64_t>(ring_s[b0 + row]) * FZ_UNITS + u % FZ_UNITS] = v[m];
    }
  }
  if (l == 0) {
    if (demand) atomicAdd(&F.demand[r], demand);
    if (ready) atomicAdd(&F.taken[r], ready);
  }
}

// ---------------------------------------------------------------- free-slot list
// Block c: free slots of slots [4096 c, 4096 c + 4096); with STATS the same block first adds the
// chunk to the pool-step statistics (free count, priority histograms of the occupied slots).
template <bool STATS>
__global__ __launch_bounds__(PF_T) void fz_count_kernel(PoolArgs P, PoolFastWs W, Stamp stamp,
                                                        int32_t *__restrict__ chunk_free) {
  __shared__ uint32_t lds[STATS ? STATS_LDS_WORDS : 48];
  const int c = blockIdx.x;
  if constexpr (STATS) {
    stats_chunk<false>(P, W, stamp_of(stamp), c, lds);
    __syncthreads();
  }
  uint32_t n = 0;
  const int32_t s0 = c * PF_CH + static_cast<int32_t>(threadIdx.x) * 16;
  for (int e = 0; e < 16; ++e) n += (s0 + e < P.n_gpu && P.free_[s0 + e] == 1) ? 1u : 0u;
  n = block_sum<PF_T>(n, lds);
  if (threadIdx.x == 0) chunk_free[c] = static_cast<int32_t>(n);
}

// Blocks c < n_fc: chunk c's free slots, ascending, after those of the chunks before it.  Block
// n_fc: the list length; every request's places c_r, scaled by (free slots) / (sum of c_r) when
// the caps add up to more than the free slots; their offsets in the list; the per-request
// counters cleared.
__global__ __launch_bounds__(PF_T) void fz_list_kernel(
    const uint8_t *__restrict__ free_, int32_t n_gpu, int32_t n_fc,
    const int32_t *__restrict__ chunk_free, int32_t *__restrict__ free_list, int32_t *counts,
    const int32_t *__restrict__ key_len, int32_t n_q, int32_t max_len, int32_t cap,
    int32_t cap_div, int32_t *slice_off, int32_t *cap_eff, int32_t *claimed, int32_t *demand,
    int32_t *taken) {
  __shared__ uint32_t tmp[48];
  const int c = blockIdx.x, t = threadIdx.x;
  if (c < n_fc) {
    uint32_t before = 0;
    for (int i = t; i < c; i += PF_T) before += static_cast<uint32_t>(chunk_free[i]);
    before = block_sum<PF_T>(before, tmp);
    const int32_t s0 = c * PF_CH + t * 16;
    uint32_t m = 0;
    for (int e = 0; e < 16; ++e)
      if (s0 + e < n_gpu && free_[s0 + e] == 1) m |= 1u << e;
    uint32_t tot;
    uint32_t pos = before + block_excl_scan<PF_T>(static_cast<uint32_t>(__popc(m)), tmp, &tot);
    while (m) {
      free_list[pos++] = s0 + __ffs(m) - 1;
      m &= m - 1;
    }
    return;
  }
  uint32_t nf = 0;
  for (int i = t; i < n_fc; i += PF_T) nf += static_cast<uint32_t>(chunk_free[i]);
  nf = block_sum<PF_T>(nf, tmp);
  if (t == 0) counts[0] = static_cast<int32_t>(nf);
  auto cap_of = [&](int32_t r) {
    return fz_request_cap(min(max(key_len[r], 0), max_len), cap, cap_div, n_gpu);   // <= 2^22
  };
  int64_t total = 0;                                  // sum of the c_r
  for (int32_t r0 = 0; r0 < n_q; r0 += PF_T) {
    const int32_t r = r0 + t;
    total += block_sum<PF_T>(r < n_q ? static_cast<uint32_t>(cap_of(r)) : 0u, tmp);   // <= 2^30
  }
  int64_t base = 0;
  for (int32_t r0 = 0; r0 < n_q; r0 += PF_T) {
    const int32_t r = r0 + t;
    uint32_t a = 0;
    if (r < n_q) {
      int64_t cr = cap_of(r);
      if (total > nf) cr = cr * static_cast<int64_t>(nf) / total;
      a = static_cast<uint32_t>(cr);
      cap_eff[r] = static_cast<int32_t>(cr);
      claimed[r] = 0;
      demand[r] = 0;
      taken[r] = 0;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<PF_T>(a, tmp, &tot);
    if (r < n_q) slice_off[r] = static_cast<int32_t>(base + ex);   // base + ex + cap_eff <= nf
    base += tot;
  }
}

// Per-step totals; with the pool-step statistics, the prefetched slots move from free to
// occupied with priority 0.
__global__ __launch_bounds__(256) void fz_fold_kernel(const int32_t *__restrict__ demand,
                                                      const int32_t *__restrict__ taken, int32_t n_q,
                                                      int32_t *demand_out, int32_t *taken_out,
                                                      PoolFastWs W, bool stats, Stamp stamp) {
  __shared__ uint32_t tmp[48];
  uint32_t d = 0, n = 0;
  for (int i = threadIdx.x; i < n_q; i += 256) {
    d += static_cast<uint32_t>(demand[i]);
    n += static_cast<uint32_t>(taken[i]);
  }
  d = block_sum<256>(d, tmp);
  n = block_sum<256>(n, tmp);
  if (threadIdx.x == 0) {
    if (demand_out) *demand_out = static_cast<int32_t>(d);
    if (taken_out) *taken_out = static_cast<int32_t>(n);
    if (stats && n) {
      const uint32_t bin = prio_bin(0, stamp_of(stamp));
      atomicSub(W.counters, static_cast<int32_t>(n));
      atomicAdd(&W.fine[hist_at(bin)], n);
      atomicAdd(&W.coarse[hist_at(bin >> 5)], n);
    }
  }
}

static int32_t fz_n_chunks(int32_t n_gpu) { return n_gpu < 1 ? 1 : (n_gpu + PF_CH - 1) / PF_CH; }

size_t fused_ws_layout(int32_t n_q, int32_t n_gpu, void *base, FusedWs *w) {
  auto al = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  const size_t nq = n_q > 0 ? static_cast<size_t>(n_q) : 0, ng = n_gpu > 0 ? static_cast<size_t>(n_gpu) : 0;
  size_t off = 0;
  auto take = [&](size_t b) { size_t o = off; off += al(b); return o; };
  const size_t o_cf = take(static_cast<size_t>(fz_n_chunks(n_gpu)) * 4), o_fl = take(ng * 4);
  const size_t o_so = take(nq * 4), o_c = take(2 * 4), o_d = take(nq * 4), o_t = take(nq * 4);
  const size_t o_ce = take(nq * 4), o_cl = take(nq * 4);
  if (w && base) {
    char *b = static_cast<char *>(base);
    w->chunk_free = reinterpret_cast<int32_t *>(b + o_cf);
    w->free_list = reinterpret_cast<int32_t *>(b + o_fl);
    w->slice_off = reinterpret_cast<int32_t *>(b + o_so);
    w->counts = reinterpret_cast<int32_t *>(b + o_c);
    w->demand = reinterpret_cast<int32_t *>(b + o_d);
    w->taken = reinterpret_cast<int32_t *>(b + o_t);
    w->cap_eff = reinterpret_cast<int32_t *>(b + o_ce);
    w->claimed = reinterpret_cast<int32_t *>(b + o_cl);
  }
  return off;
}

int32_t fused_range(int64_t total_tokens, int32_t max_len, int32_t pf_range) {
  if (pf_range > 0) return pf_range;
  const int64_t target = total_tokens / (256 * 4);          // several workgroups per CU
  int32_t t = FZ_CHUNK;
  while (t < target && t < ECHO_FUSED_MAX_RANGE) t <<= 1;
  if (t > max_len) t = ((max_len + FZ_CHUNK - 1) / FZ_CHUNK) * FZ_CHUNK;
  return t < FZ_CHUNK ? FZ_CHUNK : t;
}

int launch_fused_prefetch(const uint8_t *q, const float *w, const uint8_t *k, const float *k_scale,
                          const int64_t *key_begin, const int32_t *key_len, int32_t n_q,
                          int32_t max_len, float *scores, int64_t ld, const float *theta,
                          const int32_t *req_to_host, const echo_pool *pool, int32_t cap,
                          int32_t cap_div, int32_t range, const FusedWs &Z, uint32_t *hist0,
                          const PoolFastWs *stats, Stamp stamp, int32_t *demand_out,
                          int32_t *taken_out, hipStream_t st) {
  if (range % FZ_CHUNK != 0 || range < FZ_CHUNK || range > ECHO_FUSED_MAX_RANGE)
    return fail(ECHO_EUNSUPPORTED, "fused prefetch: range %d is not a multiple of %d in [%d, %d]",
                range, FZ_CHUNK, FZ_CHUNK, ECHO_FUSED_MAX_RANGE);
  const int32_t n_fc = fz_n_chunks(pool->n_gpu);
  PoolArgs P{pool->gpu_free, pool->gpu_priority, pool->gpu_to_host, pool->host_to_gpu,
             pool->indices_buf, pool->status, pool->n_gpu, pool->n_host};
  if (stats) fz_count_kernel<true><<<n_fc, PF_T, 0, st>>>(P, *stats, stamp, Z.chunk_free);
  else fz_count_kernel<false><<<n_fc, PF_T, 0, st>>>(P, PoolFastWs{}, stamp, Z.chunk_free);
  int rc = check_launch("fused_count");
  if (rc) return rc;
  fz_list_kernel<<<n_fc + 1, PF_T, 0, st>>>(pool->gpu_free, pool->n_gpu, n_fc, Z.chunk_free, Z.free_list,
                                            Z.counts, key_len, n_q, max_len, cap, cap_div,
                                            Z.slice_off, Z.cap_eff, Z.claimed, Z.demand, Z.taken);
  if ((rc = check_launch("fused_list"))) return rc;
  const int32_t gx = max_len > 0 ? (max_len + range - 1) / range : 0;
  const int64_t blocks = static_cast<int64_t>(gx) * n_q;
  if (blocks > 0x7FFFFFFF) return fail(ECHO_EUNSUPPORTED, "fused prefetch: grid too large");
  if (blocks > 0) {
    FusedArgs F{theta, req_to_host, pool->host_kv, pool->gpu_kv, pool->gpu_free, pool->gpu_priority,
                pool->gpu_to_host, pool->host_to_gpu, pool->status, pool->n_gpu, pool->n_host,
                Z.free_list, Z.counts, Z.slice_off, Z.cap_eff, Z.claimed, Z.demand, Z.taken, range};
#define ECHO_FZ(SC, HI)                                                                          \
  score_fused_kernel<SC, HI><<<static_cast<unsigned>(blocks), FZ_THREADS, 0, st>>>(              \
      q, w, k, k_scale, key_begin, key_len, max_len, gx, scores, ld, F, hist0)
    if (k_scale && hist0) ECHO_FZ(true, true);
    else if (k_scale) ECHO_FZ(true, false);
    else if (hist0) ECHO_FZ(false, true);
    else ECHO_FZ(false, false);
#undef ECHO_FZ
    if ((rc = check_launch("score_fused"))) return rc;
  }
  fz_fold_kernel<<<1, 256, 0, st>>>(Z.demand, Z.taken, n_q, demand_out, taken_out,
                                    stats ? *stats : PoolFastWs{}, stats != nullptr, stamp);
  return check_launch("fused_fold");
}

}  // namespace echo

using namespace echo;

extern "C" size_t echo_fused_workspace_bytes(int32_t n_q, int32_t n_gpu) {
  if (n_q < 0 || n_gpu < 0) return 0;
  return fused_ws_layout(n_q, n_gpu, nullptr, nullptr);
}

extern "C" int echo_index_scores_fused(const uint8_t *q, const float *w, const uint8_t *k,
                                       const float *k_scale, const int64_t *key_begin,
                                       const int32_t *key_len, int32_t n_q, int32_t max_key_len,
                                       float *scores, int64_t ld, const float *theta,
                                       const int32_t *req_to_host, const echo_pool *pool,
                                       int32_t cap, int32_t cap_div, int32_t range,
                                       int32_t *n_prefetched, int32_t *demand, void *ws,
                                       size_t ws_bytes, void *stream) {
  if (n_q < 0 || max_key_len < 0) return fail(ECHO_EINVAL, "echo_index_scores_fused: negative n_q or max_key_len");
  if (n_q > 65535) return fail(ECHO_EUNSUPPORTED, "echo_index_scores_fused: n_q %d > 65535", n_q);
  if (max_key_len > (1 << 22)) return fail(ECHO_EUNSUPPORTED, "echo_index_scores_fused: max_key_len above 4M");
  if (ld < max_key_len) return fail(ECHO_EINVAL, "echo_index_scores_fused: ld < max_key_len");
  if (cap < 0 || cap_div < 1) return fail(ECHO_EINVAL, "echo_index_scores_fused: cap < 0 or cap_div < 1");
  if (!pool || !pool->gpu_kv || !pool->host_kv || !pool->status || !pool->gpu_free ||
      !pool->gpu_priority || !pool->gpu_to_host || !pool->host_to_gpu)
    return fail(ECHO_EINVAL, "echo_index_scores_fused: NULL pool member");
  if (pool->n_gpu < 1 || pool->n_host < 1) return fail(ECHO_EINVAL, "echo_index_scores_fused: empty pool");
  if (pool->n_gpu > (1 << 22)) return fail(ECHO_EUNSUPPORTED, "echo_index_scores_fused: more than 4M GPU slots");
  if (!ws) return fail(ECHO_EINVAL, "echo_index_scores_fused: NULL workspace");
  if (n_q > 0 && (!q || !w || !key_begin || !key_len || !scores || !theta || !req_to_host ||
                  (max_key_len > 0 && !k)))
    return fail(ECHO_EINVAL, "echo_index_scores_fused: NULL pointer");
  const size_t need = fused_ws_layout(n_q, pool->n_gpu, nullptr, nullptr);
  if (ws_bytes < need) return fail(ECHO_EWORKSPACE, "echo_index_scores_fused: workspace %zu < %zu", ws_bytes, need);
  if (range != 0 && (range % FZ_CHUNK != 0 || range < FZ_CHUNK || range > ECHO_FUSED_MAX_RANGE))
    return fail(ECHO_EUNSUPPORTED, "echo_index_scores_fused: range %d is not 0 or a multiple of %d in [%d, %d]",
                range, FZ_CHUNK, FZ_CHUNK, ECHO_FUSED_MAX_RANGE);
  FusedWs Z{};
  fused_ws_layout(n_q, pool->n_gpu, ws, &Z);
  const int32_t rg = fused_range(static_cast<int64_t>(n_q) * max_key_len, max_key_len, range);
  return launch_fused_prefetch(q, w, k, k_scale, key_begin, key_len, n_q, max_key_len, scores, ld,
                               theta, req_to_host, pool, cap, cap_div, rg, Z, nullptr, nullptr,
                               Stamp{0, nullptr}, demand, n_prefetched, S(stream));
}
