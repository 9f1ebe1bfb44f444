// Segmented exact radix select: in every segment, the m elements with the smallest 32-bit
// keys, ties broken by the lower element index.  Used for the exact top-k of the indexer
// scores (ECHO review page §2; key = bitwise-inverted order key of the score) and for the
// lowest-priority eviction of the pool (§5.2 free; key = order key of the priority).
//
// The 32-bit key is resolved in three digits (bits 31..21, 20..10, 9..0).  Each digit is a
// multi-workgroup pass: workgroups cover 4096-element chunks of a segment, build a private
// LDS histogram of the elements that still match the prefix chosen so far, and add it into a
// per-segment global histogram.  There is no separate "pick" kernel: every workgroup of the
// next pass re-derives the chosen bins from the global histograms (a 2048-bin scan, cheap).
// After the three digits the threshold key K* and the number of K*-ties to take are known;
// a count pass and an apply pass then emit the selected elements in ascending index order
// with a prefix over chunk counts.  Everything is deterministic and needs no host sync.
#pragma once

#include "common.hpp"

namespace echo {

constexpr int SEL_THREADS = 256;
constexpr int SEL_PER_THREAD = 16;
constexpr int SEL_CHUNK = SEL_THREADS * SEL_PER_THREAD;   // 4096 elements per workgroup
constexpr int SEL_BINS = 2048;
constexpr int SEL_COPIES = 4;                              // LDS histogram replicas (contention)

ECHO_DEV int digit_shift(int d) { return d == 0 ? 21 : (d == 1 ? 10 : 0); }
ECHO_DEV uint32_t digit_mask(int d) { return d == 2 ? 0x3FFu : 0x7FFu; }
ECHO_DEV int digit_bins(int d) { return d == 2 ? 1024 : 2048; }

// Global workspace of one select: hist[3][n_seg][2048] then lt/eq counts [n_seg][n_chunks].
struct SelWs {
  uint32_t *hist;
  uint32_t *chunk_lt;
  uint32_t *chunk_eq;
  int32_t n_chunks;   // chunks per segment (grid.x)
  ECHO_DEV uint32_t *h(int d, int seg) const { return hist + (static_cast<int64_t>(d) * gridDim.y + seg) * SEL_BINS; }
};

inline size_t sel_ws_bytes(int32_t n_seg, int32_t n_chunks) {
  size_t b = static_cast<size_t>(3) * n_seg * SEL_BINS * 4 + static_cast<size_t>(2) * n_seg * n_chunks * 4;
  return (b + 255) & ~static_cast<size_t>(255);
}

struct Pick {
  uint32_t prefix;   // key bits chosen so far
  uint32_t mask;     // which bits are chosen
  uint32_t k_rem;    // how many of the elements matching the prefix are still to be taken
  int all;           // m >= number of valid elements: take everything
  int none;          // m == 0
};

// State after `ndig` digits, computed identically by every workgroup of a segment.
// lds: >= 2*SEL_THREADS/64 + 8 words of scratch.  Block-wide; every thread must call.
ECHO_DEV Pick sel_pick(const SelWs &ws, int seg, int ndig, uint32_t m, uint32_t *lds) {
  Pick p{0u, 0u, m, 0, 0};
  const int t = threadIdx.x;
  for (int d = 0; d < ndig; ++d) {
    const uint32_t *hist = ws.h(d, seg);
    const int nb = digit_bins(d);
    const int per = nb / SEL_THREADS;   // 8 or 4 bins per thread
    uint32_t local = 0;
    for (int i = 0; i < per; ++i) local += hist[t * per + i];
    uint32_t total;
    uint32_t before = block_excl_scan<SEL_THREADS>(local, lds, &total);
    if (d == 0) {
      if (m == 0) { p.none = 1; return p; }
      if (m >= total) { p.all = 1; return p; }
    }
    if (before < p.k_rem && p.k_rem <= before + local) {
      uint32_t cum = before;
      for (int i = 0; i < per; ++i) {
        const uint32_t c = hist[t * per + i];
        if (cum < p.k_rem && p.k_rem <= cum + c) {
          lds[32] = static_cast<uint32_t>(t * per + i);
          lds[33] = cum;
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    const uint32_t b = lds[32], cum_b = lds[33];
    __syncthreads();
    p.k_rem -= cum_b;
    p.prefix |= b << digit_shift(d);
    p.mask |= digit_mask(d) << digit_shift(d);
  }
  return p;
}

// One digit of histogram over this workgroup's chunk.  Src provides:
//   int32_t n(seg); bool get(seg, i, uint32_t &key)   (false = element not eligible)
template <class Src>
ECHO_DEV void sel_hist_chunk(const Src &src, const SelWs &ws, int seg, int chunk, int d,
                             const Pick &p, uint32_t *hist_lds /* SEL_COPIES*SEL_BINS */) {
  const int t = threadIdx.x;
  for (int i = t; i < SEL_COPIES * SEL_BINS; i += SEL_THREADS) hist_lds[i] = 0;
  __syncthreads();
  const int32_t n = src.n(seg);
  const int32_t base = chunk * SEL_CHUNK;
  const int sh = digit_shift(d);
  const uint32_t dm = digit_mask(d);
  uint32_t *mine = hist_lds + (t & (SEL_COPIES - 1)) * SEL_BINS;
#pragma unroll 4
  for (int e = 0; e < SEL_PER_THREAD; ++e) {
    const int32_t i = base + e * SEL_THREADS + t;
    uint32_t key;
    if (i < n && src.get(seg, i, key) && (key & p.mask) == p.prefix)
      atomicAdd(&mine[(key >> sh) & dm], 1u);
  }
  __syncthreads();
  uint32_t *gh = ws.h(d, seg);
  for (int b = t; b < digit_bins(d); b += SEL_THREADS) {
    uint32_t c = 0;
#pragma unroll
    for (int cp = 0; cp < SEL_COPIES; ++cp) c += hist_lds[cp * SEL_BINS + b];
    if (c) atomicAdd(&gh[b], c);
  }
}

// Zero histogram `d` of a segment (done by chunk 0 of the previous pass).
ECHO_DEV void sel_zero_hist(const SelWs &ws, int seg, int d) {
  uint32_t *gh = ws.h(d, seg);
  for (int b = threadIdx.x; b < SEL_BINS; b += SEL_THREADS) gh[b] = 0;
}

// Per-element classification against the final pick: 0 = not selected/ineligible,
// 1 = key < K* (always selected), 2 = key == K* (selected by rank among ties).
template <class Src>
ECHO_DEV int sel_class(const Src &src, int seg, int32_t i, const Pick &p) {
  uint32_t key;
  if (!src.get(seg, i, key)) return 0;
  if (p.all) return 1;
  if (key < p.prefix) return 1;
  if (key == p.prefix) return 2;
  return 0;
}

}  // namespace echo
