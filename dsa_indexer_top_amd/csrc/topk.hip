// Exact top-k of the indexer scores (ECHO review page §2: the top-k tokens feed sparse
// attention, so every score must be known first).  Ties at the k-th score go to the lower
// token index; -0.0 equals +0.0; the output lists the selected indices in ascending order,
// -1 padded to k.
//
// One 1024-thread workgroup per row, no host sync, so it can sit inside the step's graph.
// Selecting the k largest scores = selecting the k smallest keys ~order_key(score):
//   1. digit-0 histogram of bits 31..21 (2048 bins) — precomputed by the scoring kernel, or
//      built here in LDS;
//   2. the bin b0 that holds the k-th key: every key in a lower bin is selected for sure;
//   3. one ordered pass over the row (block scans keep index order) writes the sure indices
//      and the b0 candidates (key, index) into LDS;
//   4. digits 20..10 and 9..0 resolved on the candidates only -> threshold key K* and the
//      number of K*-ties to take (the lowest indices among them);
//   5. the two ascending lists (sure, selected candidates) are merged by binary search.
// If b0 holds more candidates than fit in LDS, digits 1-2 and the ordered output are done
// with further passes over the row instead (same result, slower).
#include <algorithm>

#include "internal.hpp"

namespace echo {

constexpr int TK_THREADS = 1024;
constexpr int TK_PER = 4;                           // consecutive elements per thread per pass step
constexpr int TK_STEP = TK_THREADS * TK_PER;        // 4096
constexpr int TK_CAP = 8192;                        // candidates kept in LDS
constexpr int TK_BINS = 2048;

__global__ void zero_u32_kernel(uint32_t *p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

__global__ void zero_u32x2_kernel(uint32_t *p, int64_t n, uint32_t *q, int64_t m) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n + m; i += stride) {
    if (i < n) p[i] = 0u;
    else q[i - n] = 0u;
  }
}

int launch_zero2_i32(int32_t *p, int64_t n, int32_t *q, int64_t m, hipStream_t st) {
  if (n + m <= 0) return ECHO_OK;
  zero_u32x2_kernel<<<static_cast<unsigned>(std::min<int64_t>((n + m + 255) / 256, 4096)), 256, 0, st>>>(
      reinterpret_cast<uint32_t *>(p), n, reinterpret_cast<uint32_t *>(q), m);
  return check_launch("zero2");
}

int launch_zero_i32(int32_t *p, int64_t n, hipStream_t st) {
  if (n <= 0) return ECHO_OK;
  zero_u32_kernel<<<static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 4096)), 256, 0, st>>>(
      reinterpret_cast<uint32_t *>(p), n);
  return check_launch("zero");
}

// Block-wide: the bin holding the k_rem-th smallest key of `hist` (nb bins) and the count of
// keys in lower bins.  1024 threads, nb in {1024, 2048}.
ECHO_DEV void tk_pick(const uint32_t *hist, int nb, uint32_t k_rem, uint32_t *tmp, uint32_t &bin,
                      uint32_t &below) {
  const int per = nb / TK_THREADS;
  const int t = threadIdx.x;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[t * per + i];
  uint32_t total;
  const uint32_t before = block_excl_scan<TK_THREADS>(local, tmp, &total);
  if (before < k_rem && k_rem <= before + local) {
    uint32_t cum = before;
    for (int i = 0; i < per; ++i) {
      const uint32_t c = hist[t * per + i];
      if (cum < k_rem && k_rem <= cum + c) {
        tmp[40] = static_cast<uint32_t>(t * per + i);
        tmp[41] = cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  bin = tmp[40];
  below = tmp[41];
  __syncthreads();
}

struct RowView {
  const float *s;
  int32_t n;
  bool vec;   // 16-byte aligned row: float4 loads
  // keys of elements i0 .. i0+3 (i0 multiple of 4); bit e of `valid` marks element i0+e present
  ECHO_DEV void load4(int32_t i0, uint32_t key[4], int &valid) const {
    valid = 0;
    if (vec && i0 + 3 < n) {
      const float4 v = *reinterpret_cast<const float4 *>(s + i0);
      key[0] = ~f32_key(v.x);
      key[1] = ~f32_key(v.y);
      key[2] = ~f32_key(v.z);
      key[3] = ~f32_key(v.w);
      valid = 0xF;
      return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e < n) {
        key[e] = ~f32_key(s[i0 + e]);
        valid |= 1 << e;
      } else {
        key[e] = 0xFFFFFFFFu;
      }
    }
  }
};

constexpr int TK_J = 8;                             // groups of 4 per thread per batch
constexpr int TK_BATCH = TK_J * TK_STEP;            // 32768 elements per batch
constexpr int TK_SCAN_LDS = TK_J * (TK_THREADS / 64) + TK_THREADS / 64 + 2;

// All loads of a batch are issued before any use: one memory round trip per batch.
ECHO_DEV void load_batch(const RowView &rv, int32_t base, uint32_t (&key)[TK_J][4],
                         int (&valid)[TK_J]) {
#pragma unroll
  for (int j = 0; j < TK_J; ++j) rv.load4(base + j * TK_STEP + threadIdx.x * TK_PER, key[j], valid[j]);
}

template <bool HAVE_HIST>
__global__ __launch_bounds__(TK_THREADS) void topk_row_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ len, int32_t max_len,
    int32_t k, const uint32_t *__restrict__ g_hist, int32_t *__restrict__ idx) {
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t cand_key[TK_CAP];
  __shared__ int32_t cand_idx[TK_CAP];
  __shared__ int32_t sure[ECHO_MAX_TOPK];
  __shared__ int32_t sel[ECHO_MAX_TOPK];
  __shared__ uint32_t tmp[48];
  __shared__ uint32_t gscan[TK_SCAN_LDS];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int32_t n = min(max(len[r], 0), max_len);
  const int32_t m = min(k, n);
  int32_t *out = idx + static_cast<int64_t>(r) * k;
  for (int j = m + t; j < k; j += TK_THREADS) out[j] = -1;
  if (m == n) {                                   // every token is selected
    for (int j = t; j < n; j += TK_THREADS) out[j] = j;
    return;
  }
  const float *row = scores + static_cast<int64_t>(r) * ld;
  RowView rv{row, n, ((reinterpret_cast<uintptr_t>(row) & 15) == 0)};
  uint32_t key[TK_J][4];
  int valid[TK_J];

  // 1. digit-0 histogram
  if (HAVE_HIST) {
    for (int b = t; b < TK_BINS; b += TK_THREADS) hist[b] = g_hist[static_cast<int64_t>(r) * TK_BINS + b];
  } else {
    for (int b = t; b < TK_BINS; b += TK_THREADS) hist[b] = 0;
    __syncthreads();
    for (int32_t base = 0; base < n; base += TK_BATCH) {
      load_batch(rv, base, key, valid);
#pragma unroll
      for (int j = 0; j < TK_J; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) hist_add_peeled(hist, key[j][e] >> 21, (valid[j] >> e) & 1);
    }
  }
  __syncthreads();
  // 2. threshold bin of digit 0
  uint32_t b0, below0;
  tk_pick(hist, TK_BINS, static_cast<uint32_t>(m), tmp, b0, below0);
  uint32_t k_rem = static_cast<uint32_t>(m) - below0;
  const uint32_t c0 = hist[b0];
  __syncthreads();
  uint32_t prefix = b0 << 21, mask = 0xFFE00000u;

  if (c0 <= TK_CAP) {
    // 3. ordered split: sure (bin < b0) and candidates (bin == b0); per batch both counts are
    //    below 2^16 (sure < k <= 4096, candidates <= TK_CAP), so they share one scan word
    uint32_t n_sure = 0, n_cand = 0;
    for (int32_t base = 0; base < n; base += TK_BATCH) {
      load_batch(rv, base, key, valid);
      uint32_t cnt[TK_J], off[TK_J], tot;
#pragma unroll
      for (int j = 0; j < TK_J; ++j) {
        uint32_t cs = 0, cc = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((valid[j] >> e) & 1) {
            const uint32_t b = key[j][e] >> 21;
            cs += (b < b0);
            cc += (b == b0);
          }
        cnt[j] = cs | (cc << 16);
      }
      group_excl_scan<TK_THREADS, TK_J>(cnt, off, gscan, &tot);
#pragma unroll
      for (int j = 0; j < TK_J; ++j) {
        uint32_t ps = n_sure + (off[j] & 0xFFFF), pc = n_cand + (off[j] >> 16);
        const int32_t i0 = base + j * TK_STEP + t * TK_PER;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((valid[j] >> e) & 1) {
            const uint32_t b = key[j][e] >> 21;
            if (b < b0) {
              if (ps < ECHO_MAX_TOPK) sure[ps] = i0 + e;
              ++ps;
            } else if (b == b0) {
              if (pc < TK_CAP) { cand_key[pc] = key[j][e]; cand_idx[pc] = i0 + e; }
              ++pc;
            }
          }
      }
      n_sure += tot & 0xFFFF;
      n_cand += tot >> 16;
    }
    __syncthreads();
    // 4. digits 1 and 2 on the candidates
    for (int d = 1; d <= 2; ++d) {
      const int sh = d == 1 ? 10 : 0;
      const uint32_t dm = d == 1 ? 0x7FFu : 0x3FFu;
      for (int b = t; b < TK_BINS; b += TK_THREADS) hist[b] = 0;
      __syncthreads();
      for (uint32_t c = t; c < n_cand; c += TK_THREADS) {
        const uint32_t kk = cand_key[c];
        if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> sh) & dm], 1u);
      }
      __syncthreads();
      uint32_t b, below;
      tk_pick(hist, d == 1 ? 2048 : 1024, k_rem, tmp, b, below);
      k_rem -= below;
      prefix |= b << sh;
      mask |= dm << sh;
    }
    // 5. candidates in index order: key < K*, then the first k_rem keys == K*
    uint32_t n_sel = 0, eq_seen = 0;
    for (uint32_t base = 0; base < n_cand; base += TK_STEP) {
      const uint32_t ci = base + t * TK_PER;
      uint32_t eq = 0;
      for (int e = 0; e < TK_PER; ++e) {
        const uint32_t c = ci + e;
        if (c < n_cand) eq += cand_key[c] == prefix;
      }
      uint32_t tot;
      const uint32_t off = block_excl_scan<TK_THREADS>(eq, tmp, &tot);
      uint32_t er = eq_seen + off;
      uint32_t take = 0;
      for (int e = 0; e < TK_PER; ++e) {
        const uint32_t c = ci + e;
        if (c < n_cand) {
          if (cand_key[c] < prefix) ++take;
          else if (cand_key[c] == prefix) { if (er < k_rem) ++take; ++er; }
        }
      }
      uint32_t tot2;
      uint32_t pos = n_sel + block_excl_scan<TK_THREADS>(take, tmp, &tot2);
      er = eq_seen + off;
      for (int e = 0; e < TK_PER; ++e) {
        const uint32_t c = ci + e;
        if (c < n_cand) {
          bool tk = cand_key[c] < prefix;
          if (cand_key[c] == prefix) { tk = er < k_rem; ++er; }
          if (tk) {
            if (pos < ECHO_MAX_TOPK) sel[pos] = cand_idx[c];
            ++pos;
          }
        }
      }
      n_sel += tot2;
      eq_seen += tot;
    }
    __syncthreads();
    // 6. merge two ascending lists of distinct indices
    n_sure = min(n_sure, static_cast<uint32_t>(ECHO_MAX_TOPK));
    n_sel = min(n_sel, static_cast<uint32_t>(ECHO_MAX_TOPK));
    for (uint32_t a = t; a < n_sure; a += TK_THREADS) {
      const int32_t v = sure[a];
      uint32_t lo = 0, hi = n_sel;
      while (lo < hi) { const uint32_t md = (lo + hi) >> 1; if (sel[md] < v) lo = md + 1; else hi = md; }
      const uint32_t pos = a + lo;
      if (pos < static_cast<uint32_t>(k)) out[pos] = v;
    }
    for (uint32_t b = t; b < n_sel; b += TK_THREADS) {
      const int32_t v = sel[b];
      uint32_t lo = 0, hi = n_sure;
      while (lo < hi) { const uint32_t md = (lo + hi) >> 1; if (sure[md] < v) lo = md + 1; else hi = md; }
      const uint32_t pos = b + lo;
      if (pos < static_cast<uint32_t>(k)) out[pos] = v;
    }
    return;
  }

  // ---- overflow: digits 1 and 2 by passes over the row, then an ordered output pass
  for (int d = 1; d <= 2; ++d) {
    const int sh = d == 1 ? 10 : 0;
    const uint32_t dm = d == 1 ? 0x7FFu : 0x3FFu;
    for (int b = t; b < TK_BINS; b += TK_THREADS) hist[b] = 0;
    __syncthreads();
    for (int32_t base = 0; base < n; base += TK_BATCH) {
      load_batch(rv, base, key, valid);
#pragma unroll
      for (int j = 0; j < TK_J; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hist_add_peeled(hist, (key[j][e] >> sh) & dm,
                          ((valid[j] >> e) & 1) && (key[j][e] & mask) == prefix);
    }
    __syncthreads();
    uint32_t b, below;
    tk_pick(hist, d == 1 ? 2048 : 1024, k_rem, tmp, b, below);
    k_rem -= below;
    prefix |= b << sh;
    mask |= dm << sh;
  }
  uint32_t n_out = 0, eq_seen = 0;
  for (int32_t base = 0; base < n; base += TK_BATCH) {
    load_batch(rv, base, key, valid);
    uint32_t eqc[TK_J], eqo[TK_J], tot;
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      eqc[j] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) eqc[j] += ((valid[j] >> e) & 1) && key[j][e] == prefix;
    }
    group_excl_scan<TK_THREADS, TK_J>(eqc, eqo, gscan, &tot);
    uint32_t takec[TK_J], poso[TK_J], tot2;
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      uint32_t er = eq_seen + eqo[j];
      takec[j] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((valid[j] >> e) & 1) {
          if (key[j][e] < prefix) ++takec[j];
          else if (key[j][e] == prefix) { if (er < k_rem) ++takec[j]; ++er; }
        }
    }
    group_excl_scan<TK_THREADS, TK_J>(takec, poso, gscan, &tot2);
#pragma unroll
    for (int j = 0; j < TK_J; ++j) {
      uint32_t er = eq_seen + eqo[j], pos = n_out + poso[j];
      const int32_t i0 = base + j * TK_STEP + t * TK_PER;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((valid[j] >> e) & 1) {
          bool tk = key[j][e] < prefix;
          if (key[j][e] == prefix) { tk = er < k_rem; ++er; }
          if (tk) {
            if (pos < static_cast<uint32_t>(k)) out[pos] = i0 + e;
            ++pos;
          }
        }
    }
    n_out += tot2;
    eq_seen += tot;
  }
}

size_t topk_ws_bytes(int32_t, int32_t) { return 256; }

int launch_topk_rows(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                     int32_t max_len, int32_t k, const uint32_t *hist0, int32_t *idx,
                     hipStream_t st) {
  if (n_rows == 0) return ECHO_OK;
  if (hist0)
    topk_row_kernel<true><<<n_rows, TK_THREADS, 0, st>>>(scores, ld, len, max_len, k, hist0, idx);
  else
    topk_row_kernel<false><<<n_rows, TK_THREADS, 0, st>>>(scores, ld, len, max_len, k, nullptr, idx);
  return check_launch("topk");
}

int launch_topk(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                int32_t max_len, int32_t k, int32_t *idx, void *, size_t, hipStream_t st) {
  return launch_topk_rows(scores, ld, len, n_rows, max_len, k, nullptr, idx, st);
}

}  // namespace echo

using namespace echo;

extern "C" size_t echo_topk_workspace_bytes(int32_t n_rows, int32_t max_len) {
  if (n_rows < 0 || max_len < 0) return 0;
  return topk_ws_bytes(n_rows, max_len);
}

extern "C" int echo_topk(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                         int32_t max_len, int32_t k, int32_t *idx, void *ws, size_t ws_bytes,
                         void *stream) {
  if (n_rows < 0 || max_len < 0) return fail(ECHO_EINVAL, "echo_topk: negative n_rows or max_len");
  if (k < 1 || k > ECHO_MAX_TOPK) return fail(ECHO_EUNSUPPORTED, "echo_topk: k %d outside [1, %d]", k, ECHO_MAX_TOPK);
  if (ld < max_len) return fail(ECHO_EINVAL, "echo_topk: ld < max_len");
  if (n_rows > 0 && (!scores || !len || !idx)) return fail(ECHO_EINVAL, "echo_topk: NULL pointer");
  (void)ws;
  (void)ws_bytes;
  return launch_topk_rows(scores, ld, len, n_rows, max_len, k, nullptr, idx, S(stream));
}
