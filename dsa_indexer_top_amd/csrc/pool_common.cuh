// Device helpers shared by the pool-step kernels and the fused top-k lookup.
#pragma once

#include "internal.hpp"

namespace echo {

// ---------------------------------------------------------------- priority code
ECHO_DEV uint32_t lc9(uint64_t x) {           // monotone code of x in [0, 2^33), 9 mantissa bits
  const uint64_t y = x + 1;
  const int e = 63 - __clzll(static_cast<unsigned long long>(y));
  const uint32_t m = static_cast<uint32_t>((y << 9) >> e) & 511u;
  return static_cast<uint32_t>(e) * 512u + m;
}

// Fine bin of a priority: ascending bin <=> ascending priority (non-strict).
ECHO_DEV uint32_t prio_bin(int32_t prio, int32_t step) {
  const int64_t age = static_cast<int64_t>(step) - static_cast<int64_t>(prio);
  const uint32_t c = age >= 0 ? 32768u + lc9(static_cast<uint64_t>(age))
                              : 32767u - lc9(static_cast<uint64_t>(-age - 1));
  return 65535u - c;
}

ECHO_DEV bool is_protected(const uint32_t *prot, int32_t slot) {
  return (prot[slot >> 5] >> (slot & 31)) & 1u;
}

// ---------------------------------------------------------------- lookup of one entry
// Returns the slot of a hit (after protecting it), INF for a miss (h_out = host index), or -1
// for no entry / a bad index (status bit set).
ECHO_DEV int32_t lookup_entry(const PoolArgs &P, const PoolFastWs &W, int32_t h, int32_t slot,
                              int32_t step_id) {
  if (h < 0 || h >= P.n_host) {
    atomicOr(P.status, ECHO_ST_BAD_HOST);
    return -1;
  }
  if (slot == INF) return INF;
  if (slot < 0 || slot >= P.n_gpu) {
    atomicOr(P.status, ECHO_ST_BAD_HOST);
    return -1;
  }
  const uint32_t bit = 1u << (slot & 31);
  const uint32_t old = atomicOr(&W.prot[slot >> 5], bit);
  if (!(old & bit)) {                          // first protector: no longer evictable
    const uint32_t b = prio_bin(P.priority[slot], step_id);
    atomicSub(&W.fine[b], 1u);
    atomicSub(&W.coarse[b >> 5], 1u);
  }
  return slot;
}

}  // namespace echo
