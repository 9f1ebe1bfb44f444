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
#include <type_traits>

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
template <int NT = TK_THREADS>
ECHO_DEV void tk_pick(const uint32_t *hist, int nb, uint32_t k_rem, uint32_t *tmp, uint32_t &bin,
                      uint32_t &below) {
  const int per = nb / NT;
  const int t = threadIdx.x;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[t * per + i];
  uint32_t total;
  const uint32_t before = block_excl_scan<NT>(local, tmp, &total);
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

// ---- rows of at most TK_BATCH (32768) scores: the row is read once, into registers
//
// The first digit is a linear bin of the score value between the row's minimum and maximum
// rather than the top 11 bits of its order key: scores of one row sit in a few exponents, so the
// top bits put most of them into a few dozen bins (contended LDS atomics, thousands of
// candidates in the threshold bin), while value bins spread them (about 15 candidates per row
// on the 32768^2 prefill).  The bin is a monotone function of the score (subtraction and
// multiplication by a positive constant round monotonically), so every element of a lower bin
// is selected for sure.  After the pick a thread keeps only two bit masks of its 32 elements
// (lower bins, threshold bin); the threshold bin's keys are copied to LDS and resolved exactly
// by one wave when at most 64 (pairwise ranks, no barrier), else by three radix passes; the few
// of them a thread owns are read again for the output, and the ties at the exact threshold key
// go to the lowest indices through an ordered block scan (only when not all of them are
// taken).  Measured on MI355X over the 32768 causal rows of the prefill: 1.21 ms against 2.56 ms
// for topk_row_kernel, which reads each row twice.

// values of elements i0 .. i0+3 of a row (-0 folded to +0); returns the presence bits
ECHO_DEV uint32_t row_value(const float *s, bool vec, int32_t n, int32_t i0, float (&x)[4]) {
  if (vec && i0 + 3 < n) {
    const float4 v = *reinterpret_cast<const float4 *>(s + i0);
    x[0] = v.x + 0.0f; x[1] = v.y + 0.0f; x[2] = v.z + 0.0f; x[3] = v.w + 0.0f;
    return 0xFu;
  }
  uint32_t valid = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = 0.f;
    if (i0 + e < n) {
      x[e] = s[i0 + e] + 0.0f;
      valid |= 1u << e;
    }
  }
  return valid;
}

// bin of a value: 0 for the row's largest scores, TK_BINS - 1 for its smallest
ECHO_DEV uint32_t value_bin(float x, float lo, float scale) {
  if (!(scale > 0.f)) return TK_BINS - 1;          // one bin (non-finite or empty span)
  const float f = (x - lo) * scale;
  const int b = f >= 2047.0f ? 2047 : static_cast<int>(f);
  return static_cast<uint32_t>(TK_BINS - 1 - max(b, 0));
}

constexpr int TK_RC = 4096;                         // threshold-bin elements resolved in LDS

// Order key of element i of a row (-0 folded to +0; ascending key = descending score).
ECHO_DEV uint32_t row_key(const float *row, int32_t i) { return ~f32_key(row[i]); }

// NT threads with J groups of four elements each: rows of at most 4 * NT * J scores; a launch
// takes the rows longer than N_LO that fit (the launches of a call split the rows between
// them; a compile-time N_LO lets the compiler drop the range checks of the groups every such
// row fills).  Every instance holds its values in at most 64 VGPRs, so 32 waves share a CU: two
// rows of 1024 threads, four of 512.  NT = 512, J = 4 takes rows of up to 8192 scores; NT =
// 1024 with J = 4 rows of up to 16384, in 63 VGPRs; J = 8 the longer ones, held to 64 VGPRs
// with some 46 spilled, which still pays: measured on MI355X over the 32768 causal prefill
// rows, 1.21 ms against 1.53 ms with the J = 8 rows one per CU (and 2.10 ms with every row one
// per CU).
template <int NT, int J, int WAVES_PER_SIMD, int N_LO>
__global__ __launch_bounds__(NT, WAVES_PER_SIMD) void topk_row_reg_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ len, int32_t max_len,
    int32_t k, int32_t *__restrict__ idx) {
  constexpr int STEP = NT * TK_PER;                // elements per group of the whole workgroup
  typedef typename std::conditional<(J * 4 <= 32), uint32_t, uint64_t>::type Mask;
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t tmp[48];
  __shared__ uint32_t gscan[TK_SCAN_LDS];
  __shared__ float red[2 * (NT / 64)];
  __shared__ uint32_t cand_key[TK_RC];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int w = t >> 6, l = lane_id();
  const int32_t n = min(max(len[r], 0), min(max_len, TK_BATCH));
  if (n <= N_LO || n > J * STEP) return;           // another launch's row
  const int32_t m = min(k, n);
  int32_t *out = idx + static_cast<int64_t>(r) * k;
  for (int j = m + t; j < k; j += NT) out[j] = -1;
  if (m == n) {                                   // every token is selected
    for (int j = t; j < n; j += NT) out[j] = j;
    return;
  }
  const float *row = scores + static_cast<int64_t>(r) * ld;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  // element (j, e) of this thread is row index j * STEP + t * TK_PER + e, bit 4j + e
  Mask lt_m = 0, b0_m = 0;                         // bins below b0; bin b0
  float lo, scale;
  uint32_t b0, k_rem, c0;
  {
    float x[J][4];
    Mask vm = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) vm |= static_cast<Mask>(row_value(row, vec, n, j * STEP + t * TK_PER, x[j])) << (4 * j);
    // row minimum and maximum
    lo = INFINITY;
    float hi = -INFINITY;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((vm >> (4 * j + e)) & 1) { lo = fminf(lo, x[j][e]); hi = fmaxf(hi, x[j][e]); }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, o));
      hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    if (l == 0) { red[w] = lo; red[NT / 64 + w] = hi; }
    for (int b = t; b < TK_BINS; b += NT) hist[b] = 0;
    if (t == 0) tmp[44] = 0;
    __syncthreads();
    lo = red[0];
    hi = red[NT / 64];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) { lo = fminf(lo, red[i]); hi = fmaxf(hi, red[NT / 64 + i]); }
    // a non-finite span (or one value) puts everything into one bin: still exact, only slower
    const float span = hi - lo;
    scale = (span > 0.f && span < INFINITY) ? 2047.0f / span : 0.f;
    // 1. value-bin histogram (the bins are spread, so plain LDS atomics).  The empty asm steps
    // here and before the masks keep the compiler from holding each value's bin across the
    // phases, which at J = 8 would double the registers the values take.
#pragma unroll
    for (int j = 0; j < J; ++j) asm volatile("" : "+v"(x[j][0]), "+v"(x[j][1]), "+v"(x[j][2]), "+v"(x[j][3]));
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((vm >> (4 * j + e)) & 1) atomicAdd(&hist[value_bin(x[j][e], lo, scale)], 1u);
    __syncthreads();
    uint32_t below0;
    tk_pick<NT>(hist, TK_BINS, static_cast<uint32_t>(m), tmp, b0, below0);
    k_rem = static_cast<uint32_t>(m) - below0;
    c0 = hist[b0];
#pragma unroll
    for (int j = 0; j < J; ++j) asm volatile("" : "+v"(x[j][0]), "+v"(x[j][1]), "+v"(x[j][2]), "+v"(x[j][3]));
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((vm >> (4 * j + e)) & 1) {
          const uint32_t bj = value_bin(x[j][e], lo, scale);
          if (bj < b0) lt_m |= Mask(1) << (4 * j + e);
          else if (bj == b0) b0_m |= Mask(1) << (4 * j + e);
        }
    // the threshold bin's keys go to LDS (in no particular order) when they fit
    if (c0 != k_rem && c0 <= TK_RC) {
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool act = (b0_m >> (4 * j + e)) & 1;
          const uint64_t ma = __ballot(act);
          if (ma) {
            const int lead = __ffsll(static_cast<unsigned long long>(ma)) - 1;
            uint32_t base = 0;
            if (l == lead) base = atomicAdd(&tmp[44], static_cast<uint32_t>(__popcll(ma)));
            base = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(base), lead));
            if (act) cand_key[base + static_cast<uint32_t>(__popcll(ma & ((1ull << l) - 1ull)))] = ~f32_key(x[j][e]);
          }
        }
    }
  }
  const bool all_b0 = c0 == k_rem;                 // the whole threshold bin is selected
  const bool in_lds = !all_b0 && c0 <= TK_RC;

  // 2. the threshold key among the bin's elements.  At most 64 of them (the usual case): one
  //    wave ranks them by comparing every pair, with no barrier in between.  Otherwise three
  //    radix passes over their order keys, from LDS when they fit, else read again from the
  //    row (cached).
  uint32_t prefix = 0, mask = 0, n_eq = 0;
  if (in_lds && c0 <= 64) {
    __syncthreads();                               // the bin's keys are in LDS
    if (w == 0) {
      const uint32_t key = l < static_cast<int>(c0) ? cand_key[l] : ~0u;
      uint32_t less = 0, eq = 0;
      for (uint32_t i = 0; i < c0; ++i) {
        const uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key), static_cast<int>(i)));
        less += o < key;
        eq += o == key;
      }
      // the threshold key: k_rem - 1 keys of the bin are below it, or tied with it
      const bool thr = l < static_cast<int>(c0) && less < k_rem && k_rem <= less + eq;
      const uint64_t mt = __ballot(thr);
      const int lead = __ffsll(static_cast<unsigned long long>(mt)) - 1;
      if (l == lead) {
        tmp[45] = key;
        tmp[46] = k_rem - less;                    // ties to take at the threshold key
        tmp[47] = eq;
      }
    }
    __syncthreads();
    prefix = tmp[45];
    k_rem = tmp[46];
    n_eq = tmp[47];
  } else if (!all_b0) {
    for (int d = 0; d < 3; ++d) {
      const int sh = d == 0 ? 21 : d == 1 ? 10 : 0;
      const uint32_t dm = d == 2 ? 0x3FFu : 0x7FFu;
      __syncthreads();
      for (int b = t; b < TK_BINS; b += NT) hist[b] = 0;
      __syncthreads();
      if (in_lds) {
        for (uint32_t base = 0; base < c0; base += NT) {
          const uint32_t c = base + t;
          const uint32_t kk = c < c0 ? cand_key[c] : 0u;
          hist_add_peeled(hist, (kk >> sh) & dm, c < c0 && (kk & mask) == prefix);
        }
      } else {
        for (int j = 0; j < J; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool in = (b0_m >> (4 * j + e)) & 1;
            const uint32_t kk = in ? row_key(row, j * STEP + t * TK_PER + e) : 0u;
            hist_add_peeled(hist, (kk >> sh) & dm, in && (kk & mask) == prefix);
          }
      }
      __syncthreads();
      uint32_t b, below;
      tk_pick<NT>(hist, d == 2 ? 1024 : 2048, k_rem, tmp, b, below);
      k_rem -= below;
      prefix |= b << sh;
      mask |= dm << sh;
      if (d == 2) n_eq = hist[b];                  // keys equal to the threshold key
    }
  }

  // 3. output in index order: bins below b0, then in b0 the keys below the threshold key and
  //    the first k_rem keys equal to it (ranked in index order only when not all are taken)
  Mask take_m = lt_m, eq_m = 0;
  if (all_b0) {
    take_m |= b0_m;
  } else {
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((b0_m >> (4 * j + e)) & 1) {
          const uint32_t kk = row_key(row, j * STEP + t * TK_PER + e);
          if (kk < prefix) take_m |= Mask(1) << (4 * j + e);
          else if (kk == prefix) eq_m |= Mask(1) << (4 * j + e);
        }
  }
  const bool rank_ties = !all_b0 && n_eq != k_rem;
  if (!rank_ties) {
    take_m |= eq_m;
  } else {
    uint32_t eqc[J], eqo[J], tot;
#pragma unroll
    for (int j = 0; j < J; ++j) eqc[j] = __popc(static_cast<uint32_t>((eq_m >> (4 * j)) & 0xFu));
    group_excl_scan<NT, J>(eqc, eqo, gscan, &tot);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      uint32_t er = eqo[j];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((eq_m >> (4 * j + e)) & 1) {
          if (er < k_rem) take_m |= Mask(1) << (4 * j + e);
          ++er;
        }
    }
  }
  uint32_t takec[J], poso[J], tot2;
#pragma unroll
  for (int j = 0; j < J; ++j) takec[j] = __popc(static_cast<uint32_t>((take_m >> (4 * j)) & 0xFu));
  group_excl_scan<NT, J>(takec, poso, gscan, &tot2);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    uint32_t pos = poso[j];
    const int32_t i0 = j * STEP + t * TK_PER;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((take_m >> (4 * j + e)) & 1) {
        if (pos < static_cast<uint32_t>(k)) out[pos] = i0 + e;
        ++pos;
      }
  }
}

size_t topk_ws_bytes(int32_t, int32_t) { return 256; }

int launch_topk_rows(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                     int32_t max_len, int32_t k, const uint32_t *hist0, int32_t *idx,
                     hipStream_t st) {
  if (n_rows == 0) return ECHO_OK;
  if (hist0)
    topk_row_kernel<true><<<n_rows, TK_THREADS, 0, st>>>(scores, ld, len, max_len, k, hist0, idx);
  else if (max_len <= TK_BATCH) {
    topk_row_reg_kernel<512, 4, 8, -1><<<n_rows, 512, 0, st>>>(scores, ld, len, max_len, k, idx);
    if (max_len > 8192)
      topk_row_reg_kernel<1024, 4, 8, 8192><<<n_rows, 1024, 0, st>>>(scores, ld, len, max_len, k, idx);
    if (max_len > 16384)
      topk_row_reg_kernel<1024, 8, 8, 16384><<<n_rows, 1024, 0, st>>>(scores, ld, len, max_len, k, idx);
  }
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
