// Guaranteed residency (ECHO review page §5.1 metadata, §5.2 free / allocate / recall lookup)
// for pools of up to 262144 slots, as ONE kernel of one 1024-thread workgroup.
//
// Same result as the multi-kernel path in pool.hip (the canonical rule: protect hits, evict
// the need = #miss - #free unprotected slots with the smallest (priority, slot), the i-th miss
// takes the i-th free slot in ascending order), with no kernel boundaries.  Inside a pass no
// load waits on another: thread t owns groups of 4 consecutive elements 4096 apart, issues
// all of a batch's 16-byte loads at once, and a group-ordered block scan restores index order
// wherever order matters (the miss list, ties at the eviction threshold, the allocation).
//
// Eviction select (keys = order keys of the priorities of occupied, unprotected slots):
//   pass A   counts (free, evictable) and the key range; digits start at the highest bit
//            where the evictable keys differ, so step-stamp priorities need few digits;
//   pass B   11-bit histogram of the first digit -> threshold bin b0;
//   pass C   evict every key below b0 (a set: order is irrelevant) and list the b0 keys with
//            their slots in slot order in LDS;
//   LDS      the remaining digits on that list -> threshold key K*; evict the keys below K*
//            and, of the K* ties, the lowest slots.
// A first digit whose threshold bin overflows the LDS list falls back to digit passes over
// memory (same result).
#include "internal.hpp"

namespace echo {

constexpr int PS_THREADS = 1024;
constexpr int PS_NW = PS_THREADS / 64;
constexpr int PS_GROUP = 4 * PS_THREADS;          // 4096 elements per group row
constexpr int PS_EJ = 4;                          // entry groups per thread per block
constexpr int PS_EBLOCK = PS_EJ * PS_GROUP;       // 16384 entries
constexpr int PS_SJ = 8;                          // slot groups per thread per batch
constexpr int PS_SBATCH = PS_SJ * PS_GROUP;       // 32768 slots
constexpr int PS_CAP = 8192;                      // threshold-bin list in LDS
constexpr int PS_SCAN = PS_SJ * PS_NW + PS_NW + 2;
constexpr int32_t PS_MAX_GPU = 262144;

ECHO_DEV uint32_t block_min_u32(uint32_t v, uint32_t *tmp) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(v, off, 64)));
  if (lane_id() == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = tmp[0];
  for (int i = 1; i < PS_NW; ++i) r = min(r, tmp[i]);
  __syncthreads();
  return r;
}

ECHO_DEV uint32_t block_max_u32(uint32_t v, uint32_t *tmp) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(v, off, 64)));
  if (lane_id() == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = tmp[0];
  for (int i = 1; i < PS_NW; ++i) r = max(r, tmp[i]);
  __syncthreads();
  return r;
}

// bin holding the k_rem-th smallest key in `hist` (2048 bins) and the count below it
ECHO_DEV void ps_pick(const uint32_t *hist, uint32_t k_rem, uint32_t *tmp, uint32_t &bin,
                      uint32_t &below) {
  const int t = threadIdx.x;
  const uint32_t a = hist[2 * t], b = hist[2 * t + 1];
  uint32_t total;
  const uint32_t before = block_excl_scan<PS_THREADS>(a + b, tmp, &total);
  if (before < k_rem && k_rem <= before + a) {
    tmp[40] = 2 * t;
    tmp[41] = before;
  } else if (before + a < k_rem && k_rem <= before + a + b) {
    tmp[40] = 2 * t + 1;
    tmp[41] = before + a;
  }
  __syncthreads();
  bin = tmp[40];
  below = tmp[41];
  __syncthreads();
}

// One batch of slots in the group layout: free state (1 free, 0 evictable, else neither) and
// order keys of the priorities.  Slot of (group j, element e) = base + j*4096 + 4t + e.
struct SlotBatch {
  uint32_t key[PS_SJ][4];
  uint32_t fre[PS_SJ];    // 4 free bytes
  ECHO_DEV void load(const PoolArgs &P, int32_t base, bool keys) {
#pragma unroll
    for (int j = 0; j < PS_SJ; ++j) {
      const int32_t s0 = base + j * PS_GROUP + threadIdx.x * 4;
      if (s0 + 3 < P.n_gpu) {
        fre[j] = *reinterpret_cast<const uint32_t *>(P.free_ + s0);
        if (keys) {
          const int4 v = *reinterpret_cast<const int4 *>(P.priority + s0);
          key[j][0] = i32_key(v.x);
          key[j][1] = i32_key(v.y);
          key[j][2] = i32_key(v.z);
          key[j][3] = i32_key(v.w);
        }
      } else {
        fre[j] = 0xFFFFFFFFu;               // 0xFF: no slot
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (s0 + e < P.n_gpu) {
            fre[j] = (fre[j] & ~(0xFFu << (8 * e))) | (static_cast<uint32_t>(P.free_[s0 + e]) << (8 * e));
            if (keys) key[j][e] = i32_key(P.priority[s0 + e]);
          }
        }
      }
    }
  }
  ECHO_DEV uint32_t state(int j, int e) const { return (fre[j] >> (8 * e)) & 0xFFu; }
};

ECHO_DEV void evict_slot(const PoolArgs &P, int32_t slot) {
  const int32_t h = P.to_host[slot];
  if (h >= 0 && h < P.n_host) P.host_to_gpu[h] = INF;
  P.to_host[slot] = INF;
  P.priority[slot] = -1;
  P.free_[slot] = 1;                       // the row stays: the host holds the backup
}

__global__ __launch_bounds__(PS_THREADS) void pool_step_small_kernel(
    PoolArgs P, int32_t *__restrict__ miss_entry, const int32_t *__restrict__ idx,
    const int64_t *__restrict__ key_begin, const int32_t *__restrict__ req_to_host, int64_t n_k,
    int32_t n_rows, int32_t k, int32_t step_id, int32_t *__restrict__ topk_slot,
    int32_t *__restrict__ miss_host, int32_t *__restrict__ miss_slot, int32_t *__restrict__ n_miss_out) {
  __shared__ uint32_t tmp[48];
  __shared__ uint32_t gscan[PS_SCAN];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t ckey[PS_CAP];
  __shared__ int32_t cslot[PS_CAP];
  __shared__ int s_bad;
  const int t = threadIdx.x;
  const int64_t n_ent = static_cast<int64_t>(n_rows) * k;
  if (t == 0) s_bad = 0;
  __syncthreads();
  if (*(volatile int32_t *)P.status) return;

  // ---------------------------------------------------------------- 1. lookup + ordered misses
  uint32_t n_miss = 0;
  for (int64_t blk = 0; blk < n_ent; blk += PS_EBLOCK) {
    int32_t s[PS_EJ][4], h[PS_EJ][4], sl[PS_EJ][4];
#pragma unroll
    for (int j = 0; j < PS_EJ; ++j) {
      const int64_t e0 = blk + j * PS_GROUP + t * 4;
      if (e0 + 3 < n_ent) {
        const int4 v = *reinterpret_cast<const int4 *>(idx + e0);
        s[j][0] = v.x; s[j][1] = v.y; s[j][2] = v.z; s[j][3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[j][e] = (e0 + e < n_ent) ? idx[e0 + e] : -1;
      }
    }
    uint32_t has = 0;                                // bit 4j+e: entry has a token in range
#pragma unroll
    for (int j = 0; j < PS_EJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[j][e] = -1;
        if (s[j][e] >= 0) {
          const int64_t ent = blk + j * PS_GROUP + t * 4 + e;
          const int64_t tok = key_begin[ent / k] + s[j][e];
          if (tok < 0 || tok >= n_k) {
            s_bad = 1;
          } else {
            h[j][e] = req_to_host[tok];
            has |= 1u << (4 * j + e);
          }
        }
      }
#pragma unroll
    for (int j = 0; j < PS_EJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sl[j][e] = -1;
        if (!((has >> (4 * j + e)) & 1)) continue;
        if (h[j][e] < 0 || h[j][e] >= P.n_host) { s_bad = 1; h[j][e] = -1; continue; }
        sl[j][e] = P.host_to_gpu[h[j][e]];
      }
    uint32_t cnt[PS_EJ], off[PS_EJ], tot;
#pragma unroll
    for (int j = 0; j < PS_EJ; ++j) {
      cnt[j] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (h[j][e] < 0) continue;
        if (sl[j][e] == INF) { ++cnt[j]; continue; }
        if (sl[j][e] < 0 || sl[j][e] >= P.n_gpu) { s_bad = 1; h[j][e] = -1; sl[j][e] = -1; continue; }
        P.free_[sl[j][e]] = 2;                       // protected for this call
        h[j][e] = -1;                                // a hit
      }
    }
    // (a PS_EJ-group scan through the PS_SJ-sized helper: pad the unused groups with zero)
    uint32_t c8[PS_SJ], o8[PS_SJ];
#pragma unroll
    for (int j = 0; j < PS_SJ; ++j) c8[j] = j < PS_EJ ? cnt[j] : 0u;
    group_excl_scan<PS_THREADS, PS_SJ>(c8, o8, gscan, &tot);
#pragma unroll
    for (int j = 0; j < PS_EJ; ++j) off[j] = o8[j];
#pragma unroll
    for (int j = 0; j < PS_EJ; ++j) {
      uint32_t pos = n_miss + off[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t ent = blk + j * PS_GROUP + t * 4 + e;
        if (ent >= n_ent) continue;
        if (h[j][e] >= 0) {
          miss_host[pos] = h[j][e];
          miss_entry[pos] = static_cast<int32_t>(ent);
          ++pos;
          topk_slot[ent] = -1;
        } else {
          topk_slot[ent] = (s[j][e] >= 0 && sl[j][e] >= 0 && sl[j][e] < P.n_gpu) ? sl[j][e] : -1;
        }
      }
    }
    n_miss += tot;
  }
  __syncthreads();
  bool abort = s_bad != 0;
  if (abort && t == 0) atomicOr(P.status, ECHO_ST_BAD_HOST);

  SlotBatch sb;
  // ---------------------------------------------------------------- 2. pass A: counts, key range
  uint32_t nf = 0, ne = 0, kmin = ~0u, kmax = 0u;
  if (!abort) {
    for (int32_t base = 0; base < P.n_gpu; base += PS_SBATCH) {
      sb.load(P, base, true);
#pragma unroll
      for (int j = 0; j < PS_SJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t st = sb.state(j, e);
          nf += st == 1;
          if (st == 0) { ++ne; kmin = min(kmin, sb.key[j][e]); kmax = max(kmax, sb.key[j][e]); }
        }
    }
  }
  nf = block_sum<PS_THREADS>(nf, tmp);
  ne = block_sum<PS_THREADS>(ne, tmp);
  kmin = block_min_u32(kmin, tmp);
  kmax = block_max_u32(kmax, tmp);
  const uint32_t need = n_miss > nf ? n_miss - nf : 0u;
  if (!abort && need > ne) {
    abort = true;
    if (t == 0) atomicOr(P.status, ECHO_ST_EXHAUSTED);
  }

  // ---------------------------------------------------------------- 3. eviction
  if (!abort && need > 0) {
    if (need == ne) {                                 // every evictable slot goes
      for (int32_t base = 0; base < P.n_gpu; base += PS_SBATCH) {
        sb.load(P, base, false);
#pragma unroll
        for (int j = 0; j < PS_SJ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (sb.state(j, e) == 0) evict_slot(P, base + j * PS_GROUP + t * 4 + e);
      }
    } else {
      const uint32_t diff = kmin ^ kmax;              // != 0: need < ne means keys differ or ties
      uint32_t prefix = kmin, mask = 0xFFFFFFFFu, k_rem = need;
      int top = -1;
      if (diff) {
        top = 31 - __clz(diff);
        mask = top == 31 ? 0u : ~((2u << top) - 1u);
        prefix = kmin & mask;
      }
      bool listed = false;                            // the remaining ties/candidates are in LDS
      uint32_t n_c = 0;
      if (top >= 0) {
        // pass B: first digit histogram
        const int lo = top >= 10 ? top - 10 : 0;
        const uint32_t dm = (2u << (top - lo)) - 1u;
        for (int b = t; b < 2048; b += PS_THREADS) hist[b] = 0;
        __syncthreads();
        for (int32_t base = 0; base < P.n_gpu; base += PS_SBATCH) {
          sb.load(P, base, true);
#pragma unroll
          for (int j = 0; j < PS_SJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              hist_add_peeled(hist, (sb.key[j][e] >> lo) & dm, sb.state(j, e) == 0);
        }
        __syncthreads();
        uint32_t b0, below;
        ps_pick(hist, k_rem, tmp, b0, below);
        const uint32_t c0 = hist[b0];
        __syncthreads();
        k_rem -= below;
        const uint32_t pre0 = prefix | (b0 << lo), mask0 = mask | (dm << lo);
        if (c0 <= PS_CAP) {
          // pass C: evict below b0, list the b0 bin in slot order
          for (int32_t base = 0; base < P.n_gpu; base += PS_SBATCH) {
            sb.load(P, base, true);
            uint32_t cc[PS_SJ], co[PS_SJ], tot;
#pragma unroll
            for (int j = 0; j < PS_SJ; ++j) {
              cc[j] = 0;
#pragma unroll
              for (int e = 0; e < 4; ++e) cc[j] += sb.state(j, e) == 0 && (sb.key[j][e] & mask0) == pre0;
            }
            group_excl_scan<PS_THREADS, PS_SJ>(cc, co, gscan, &tot);
#pragma unroll
            for (int j = 0; j < PS_SJ; ++j) {
              uint32_t pos = n_c + co[j];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (sb.state(j, e) != 0) continue;
                const int32_t slot = base + j * PS_GROUP + t * 4 + e;
                const uint32_t kk = sb.key[j][e];
                if ((kk & mask0) == pre0) {
                  if (pos < PS_CAP) { ckey[pos] = kk; cslot[pos] = slot; }
                  ++pos;
                } else if (kk < pre0) {
                  evict_slot(P, slot);
                }
              }
            }
            n_c += tot;
          }
          listed = true;
        }
        prefix = pre0;
        mask = mask0;
        top = lo - 1;
        __syncthreads();
        if (listed) {
          // remaining digits on the LDS list
          while (top >= 0) {
            const int lo2 = top >= 10 ? top - 10 : 0;
            const uint32_t dm2 = (2u << (top - lo2)) - 1u;
            for (int b = t; b < 2048; b += PS_THREADS) hist[b] = 0;
            __syncthreads();
            for (uint32_t c = t; c < n_c; c += PS_THREADS)
              if ((ckey[c] & mask) == prefix) atomicAdd(&hist[(ckey[c] >> lo2) & dm2], 1u);
            __syncthreads();
            uint32_t b, bl;
            ps_pick(hist, k_rem, tmp, b, bl);
            k_rem -= bl;
            prefix |= b << lo2;
            mask |= dm2 << lo2;
            top = lo2 - 1;
          }
        } else {
          // overflow: remaining digits by passes over memory
          while (top >= 0) {
            const int lo2 = top >= 10 ? top - 10 : 0;
            const uint32_t dm2 = (2u << (top - lo2)) - 1u;
            for (int b = t; b < 2048; b += PS_THREADS) hist[b] = 0;
            __syncthreads();
            for (int32_t base = 0; base < P.n_gpu; base += PS_SBATCH) {
              sb.load(P, base, true);
#pragma unroll
              for (int j = 0; j < PS_SJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  hist_add_peeled(hist, (sb.key[j][e] >> lo2) & dm2,
                                  sb.state(j, e) == 0 && (sb.key[j][e] & mask) == prefix);
            }
            __syncthreads();
            uint32_t b, bl;
            ps_pick(hist, k_rem, tmp, b, bl);
            k_rem -= bl;
            prefix |= b << lo2;
            mask |= dm2 << lo2;
            top = lo2 - 1;
          }
        }
      }
      const uint32_t kstar = prefix;                  // full key of the threshold
      if (listed) {
        // the list is in slot order: keys < K* go, then the first k_rem ties
        uint32_t eq_seen = 0;
        for (uint32_t cb = 0; cb < n_c; cb += PS_THREADS) {
          const uint32_t c = cb + t;
          const bool in = c < n_c;
          const uint32_t kk = in ? ckey[c] : ~0u;
          uint32_t tot;
          const uint32_t r = eq_seen + block_excl_scan<PS_THREADS>(in && kk == kstar, tmp, &tot);
          if (in && (kk < kstar || (kk == kstar && r < k_rem))) evict_slot(P, cslot[c]);
          eq_seen += tot;
        }
      } else {
        // no list (single distinct key, or overflow): ordered pass over memory
        uint32_t eq_seen = 0;
        for (int32_t base = 0; base < P.n_gpu; base += PS_SBATCH) {
          sb.load(P, base, true);
          uint32_t qc[PS_SJ], qo[PS_SJ], tot;
#pragma unroll
          for (int j = 0; j < PS_SJ; ++j) {
            qc[j] = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) qc[j] += sb.state(j, e) == 0 && sb.key[j][e] == kstar;
          }
          group_excl_scan<PS_THREADS, PS_SJ>(qc, qo, gscan, &tot);
#pragma unroll
          for (int j = 0; j < PS_SJ; ++j) {
            uint32_t r = eq_seen + qo[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (sb.state(j, e) != 0) continue;
              const uint32_t kk = sb.key[j][e];
              bool take = kk < kstar;
              if (kk == kstar) { take = r < k_rem; ++r; }
              if (take) evict_slot(P, base + j * PS_GROUP + t * 4 + e);
            }
          }
          eq_seen += tot;
        }
      }
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- 4. ordered allocation
  if (!abort && n_miss > 0) {
    uint32_t seen = 0;
    for (int32_t base = 0; base < P.n_gpu && seen < n_miss; base += PS_SBATCH) {
      sb.load(P, base, false);
      uint32_t fc[PS_SJ], fo[PS_SJ], tot;
#pragma unroll
      for (int j = 0; j < PS_SJ; ++j) {
        fc[j] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) fc[j] += sb.state(j, e) == 1;
      }
      group_excl_scan<PS_THREADS, PS_SJ>(fc, fo, gscan, &tot);
#pragma unroll
      for (int j = 0; j < PS_SJ; ++j) {
        uint32_t rank = seen + fo[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (sb.state(j, e) != 1 || rank >= n_miss) continue;
          const int32_t slot = base + j * PS_GROUP + t * 4 + e;
          const int32_t hh = miss_host[rank];
          P.free_[slot] = 0;
          P.to_host[slot] = hh;
          P.host_to_gpu[hh] = slot;
          P.priority[slot] = step_id;
          P.indices_buf[rank] = slot;
          miss_slot[rank] = slot;
          topk_slot[miss_entry[rank]] = slot;
          ++rank;
        }
      }
      seen += tot;
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- 5. finalize
  for (int64_t blk = 0; blk < n_ent; blk += PS_EBLOCK) {
    int32_t sl[PS_EJ][4];
    uint32_t st[PS_EJ][4];
#pragma unroll
    for (int j = 0; j < PS_EJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t ent = blk + j * PS_GROUP + t * 4 + e;
        sl[j][e] = ent < n_ent ? topk_slot[ent] : -1;
      }
#pragma unroll
    for (int j = 0; j < PS_EJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        st[j][e] = (sl[j][e] >= 0 && sl[j][e] < P.n_gpu) ? P.free_[sl[j][e]] : 0u;
#pragma unroll
    for (int j = 0; j < PS_EJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (st[j][e] == 2) {                      // a hit: clear protection, stamp
          P.free_[sl[j][e]] = 0;
          if (!abort) P.priority[sl[j][e]] = step_id;
        }
  }
  if (!abort) {
    for (uint32_t i = t; i < n_miss; i += PS_THREADS)
      if (P.host_to_gpu[miss_host[i]] != miss_slot[i]) atomicOr(P.status, ECHO_ST_DUP_HOST);
    const int64_t lim = min(static_cast<int64_t>(P.n_gpu), n_ent);
    for (int64_t j = n_miss + t; j < lim; j += PS_THREADS) P.indices_buf[j] = -1;
    for (int64_t j = n_miss + t; j < n_ent; j += PS_THREADS) {
      miss_host[j] = -1;
      miss_slot[j] = -1;
    }
  }
  if (t == 0) *n_miss_out = static_cast<int32_t>(n_miss);
}

bool pool_small_fits(int32_t n_gpu) { return n_gpu <= PS_MAX_GPU; }

int launch_pool_small(const echo_pool *pool, int32_t *miss_entry_ws, const int32_t *idx,
                      const int64_t *key_begin, const int32_t *req_to_host, int64_t n_k,
                      int32_t n_rows, int32_t k, int32_t step_id, int32_t *topk_slot,
                      int32_t *miss_host, int32_t *miss_slot, int32_t *n_miss, hipStream_t st) {
  if (pool->n_gpu > PS_MAX_GPU) return fail(ECHO_EUNSUPPORTED, "pool_small: n_gpu %d too large", pool->n_gpu);
  PoolArgs P{pool->gpu_free, pool->gpu_priority, pool->gpu_to_host, pool->host_to_gpu,
             pool->indices_buf, pool->status, pool->n_gpu, pool->n_host};
  pool_step_small_kernel<<<1, PS_THREADS, 0, st>>>(P, miss_entry_ws, idx, key_begin, req_to_host,
                                                   n_k, n_rows, k, step_id, topk_slot, miss_host,
                                                   miss_slot, n_miss);
  return check_launch("pool_step_small");
}

}  // namespace echo
