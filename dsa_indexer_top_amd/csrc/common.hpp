// Shared device/host helpers of the HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/echo.h"

#define ECHO_DEV __device__ __forceinline__

namespace echo {

constexpr int H = ECHO_H_INDEX;
constexpr int D = ECHO_D_INDEX;
constexpr int ROW = ECHO_ROW_ELEMS;
constexpr int32_t INF = ECHO_INF;

// ---------------------------------------------------------------- host-side error plumbing
void set_error(const char *fmt, ...);
int fail(int code, const char *fmt, ...);
int check_launch(const char *what);

inline hipStream_t S(void *s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------- ordering keys
// Order-preserving map of a float to uint32: a < b  <=>  key(a) < key(b); -0.0 is folded onto
// +0.0 first so the two compare equal (ties then go to the lower index).
ECHO_DEV uint32_t f32_key(float x) {
  uint32_t b = __float_as_uint(x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
// int32 priority -> uint32 with the same order
ECHO_DEV uint32_t i32_key(int32_t x) { return static_cast<uint32_t>(x) ^ 0x80000000u; }

// ---------------------------------------------------------------- wave / block scans
ECHO_DEV int lane_id() { return __lane_id(); }

// One DPP move: lane i receives the CTRL-selected lane's v; lanes outside ROW_MASK, and lanes
// whose source is outside its row, receive `old`.  Every lane of the wave must be active.
template <int CTRL, int ROW_MASK>
ECHO_DEV uint32_t dpp_mov(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v),
                                                           CTRL, ROW_MASK, 0xF, false));
}
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;
constexpr int DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

// Inclusive scan of OP over the 64 lanes: Hillis-Steele inside each 16-lane row with row
// shifts, then each row's total carried into the following rows with the row broadcasts.
template <typename OP>
ECHO_DEV uint32_t wave_incl_scan_op(uint32_t v, uint32_t identity, OP op) {
  v = op(v, dpp_mov<DPP_ROW_SHR1, 0xF>(identity, v));
  v = op(v, dpp_mov<DPP_ROW_SHR2, 0xF>(identity, v));
  v = op(v, dpp_mov<DPP_ROW_SHR4, 0xF>(identity, v));
  v = op(v, dpp_mov<DPP_ROW_SHR8, 0xF>(identity, v));
  v = op(v, dpp_mov<DPP_ROW_BCAST15, 0xA>(identity, v));
  v = op(v, dpp_mov<DPP_ROW_BCAST31, 0xC>(identity, v));
  return v;
}

struct OpAdd { ECHO_DEV uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMin { ECHO_DEV uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };
struct OpMax { ECHO_DEV uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };

// inclusive prefix sum over the 64 lanes of a wave
ECHO_DEV uint32_t wave_incl_scan(uint32_t v) { return wave_incl_scan_op(v, 0u, OpAdd{}); }

// inclusive prefix sum inside each 16-lane row (lane 15 of a row holds the row's total)
ECHO_DEV uint32_t row16_incl_scan(uint32_t v) {
  v += dpp_mov<DPP_ROW_SHR1, 0xF>(0u, v);
  v += dpp_mov<DPP_ROW_SHR2, 0xF>(0u, v);
  v += dpp_mov<DPP_ROW_SHR4, 0xF>(0u, v);
  v += dpp_mov<DPP_ROW_SHR8, 0xF>(0u, v);
  return v;
}

ECHO_DEV uint32_t wave_sum(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_incl_scan(v)), 63));
}
ECHO_DEV uint32_t wave_min(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_incl_scan_op(v, ~0u, OpMin{})), 63));
}
ECHO_DEV uint32_t wave_max(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_incl_scan_op(v, 0u, OpMax{})), 63));
}

// Exclusive block-wide prefix sum for a block of NT threads (NT multiple of 64, <= 1024).
// `tmp` is LDS scratch of at least NT/64 + 1 words.  Returns the exclusive prefix; *total
// receives the block sum.  Contains __syncthreads(): every thread must call it.
template <int NT>
ECHO_DEV uint32_t block_excl_scan(uint32_t v, uint32_t *tmp, uint32_t *total) {
  constexpr int NW = NT / 64;
  const int w = threadIdx.x >> 6, l = lane_id();
  uint32_t inc = wave_incl_scan(v);
  if (l == 63) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    uint32_t s = (l < NW) ? tmp[l] : 0u;
    uint32_t si = wave_incl_scan(s);
    if (l < NW) tmp[l] = si - s;
    if (l == NW - 1) tmp[NW] = si;
  }
  __syncthreads();
  uint32_t res = tmp[w] + inc - v;
  *total = tmp[NW];
  __syncthreads();
  return res;
}

// Exclusive prefix, in (group j, thread t) order, of per-thread per-group counts: an item of
// (j, t) comes after every item of groups < j and after group j's items of threads < t.  This
// is index order when thread t owns the elements [4t + G*j, 4t + G*j + 4) (G = 4*NT), the
// layout that keeps every 16-byte load of a wave contiguous.  lds: >= J*NT/64 + NT/64 + 2
// words.  Block-wide; *total = sum of all counts.
template <int NT, int J>
ECHO_DEV void group_excl_scan(const uint32_t (&cnt)[J], uint32_t (&base)[J], uint32_t *lds,
                              uint32_t *total) {
  constexpr int NW = NT / 64;
  constexpr int NTOT = J * NW;
  static_assert(NTOT <= NT, "too many groups for one block scan");
  const int w = threadIdx.x >> 6, l = lane_id();
  uint32_t incl[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    incl[j] = wave_incl_scan(cnt[j]);
    if (l == 63) lds[j * NW + w] = incl[j];
  }
  __syncthreads();
  const uint32_t v = threadIdx.x < NTOT ? lds[threadIdx.x] : 0u;
  __syncthreads();
  uint32_t tot;
  const uint32_t ex = block_excl_scan<NT>(v, lds + NTOT, &tot);
  if (threadIdx.x < NTOT) lds[threadIdx.x] = ex;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < J; ++j) base[j] = lds[j * NW + w] + incl[j] - cnt[j];
  *total = tot;
  __syncthreads();
}

// Bin of the m-th smallest key in a 2048-bin histogram, the count below it and the bin's own
// count.  NT threads.
template <int NT>
ECHO_DEV void pick2048(const uint32_t *hist, uint32_t m, uint32_t *tmp, uint32_t &bin, uint32_t &below,
                       uint32_t &count) {
  constexpr int PER = 2048 / NT;
  const int t = threadIdx.x;
  uint32_t v[PER], local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) { v[i] = hist[t * PER + i]; local += v[i]; }
  uint32_t total;
  const uint32_t before = block_excl_scan<NT>(local, tmp, &total);
  if (before < m && m <= before + local) {
    uint32_t cum = before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (cum < m && m <= cum + v[i]) { tmp[40] = t * PER + i; tmp[41] = cum; tmp[42] = v[i]; break; }
      cum += v[i];
    }
  }
  __syncthreads();
  bin = tmp[40];
  below = tmp[41];
  count = tmp[42];
  __syncthreads();
}

// LDS histogram add with the wave's most common bin peeled off first: the keys being
// counted (top bits of scores, step-stamp priorities) concentrate in few bins, and
// same-address LDS atomics within one instruction serialise.
ECHO_DEV void hist_add_peeled(uint32_t *hist, uint32_t bin, bool act) {
  const uint64_t m_act = __ballot(act);
  if (!m_act) return;
  const int leader = __ffsll(static_cast<unsigned long long>(m_act)) - 1;
  const uint32_t lead_bin = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), leader));
  const uint64_t same = __ballot(act && bin == lead_bin);
  if (lane_id() == leader) atomicAdd(&hist[lead_bin], static_cast<uint32_t>(__popcll(same)));
  if (act && bin != lead_bin) atomicAdd(&hist[bin], 1u);
}

template <int NT>
ECHO_DEV uint32_t block_sum(uint32_t v, uint32_t *tmp) {
  uint32_t total;
  block_excl_scan<NT>(v, tmp, &total);
  return total;
}

}  // namespace echo
