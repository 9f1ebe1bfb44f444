// Recall of missed latent rows from the pinned host backup (ECHO review page §5.2: the copy is
// done by a GPU kernel reading host memory directly, which keeps the step inside the graph
// and uses the host link better than host-issued copies; §2: the host holds a full backup, so
// the copy is bitwise and one-way).
//
// Gather kernel: the rows of 1152 bytes (72 x 16 B) of up to 32 misses per workgroup
// iteration are read with 16-byte loads straight from mapped pinned host memory, nine loads
// in flight per thread before any store, then written to their GPU slots.  The miss count is
// read on the device, so the launch has a fixed grid sized for the maximum.  It also checks
// that HostTokenToGPU points back at each miss's slot (duplicate host indices otherwise).
//
// Staged form (the decode step): workgroups riding along in the eviction launches read each
// request's missed rows from host memory into a device staging area as soon as the lookup has
// listed them, so the host link works while eviction and allocation run; the scatter kernel
// here then copies the staged rows into their slots at device bandwidth.
//
// Memcpy mode (the host-driven baseline): the host waits for the stream, reads the miss list
// and enqueues one hipMemcpyAsync per row.
#include <algorithm>
#include <new>
#include <vector>

#include "internal.hpp"

namespace echo {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int RC_THREADS = 256;
constexpr int RC_ROWS = 32;                       // rows per workgroup iteration
constexpr int RC_UNITS_PER_ROW = ROW * 2 / 16;    // 72 x 16 B
constexpr int RC_PER_THREAD = RC_ROWS * RC_UNITS_PER_ROW / RC_THREADS;   // 9

__global__ __launch_bounds__(RC_THREADS) void recall_gather_kernel(
    const uint16_t *__restrict__ host_kv, uint16_t *__restrict__ gpu_kv,
    const int32_t *__restrict__ miss_host, const int32_t *__restrict__ miss_slot,
    const int32_t *__restrict__ n_miss_p, int32_t max_miss, int32_t *__restrict__ status,
    const int32_t *__restrict__ host_to_gpu, int32_t n_host, int32_t n_gpu) {
  if (*(volatile const int32_t *)status) return;
  const int32_t n = min(*n_miss_p, max_miss);
  const v4i *src = reinterpret_cast<const v4i *>(host_kv);
  v4i *dst = reinterpret_cast<v4i *>(gpu_kv);
  for (int32_t r0 = blockIdx.x * RC_ROWS; r0 < n; r0 += gridDim.x * RC_ROWS) {
    v4i v[RC_PER_THREAD];
    int64_t d_off[RC_PER_THREAD];
#pragma unroll
    for (int m = 0; m < RC_PER_THREAD; ++m) {
      const int u = threadIdx.x + m * RC_THREADS;
      const int32_t row = r0 + u / RC_UNITS_PER_ROW;
      const int part = u % RC_UNITS_PER_ROW;
      d_off[m] = -1;
      if (row < n) {
        const int32_t h = miss_host[row], s = miss_slot[row];
        if (h >= 0 && h < n_host && s >= 0 && s < n_gpu) {
          v[m] = __builtin_nontemporal_load(src + static_cast<int64_t>(h) * RC_UNITS_PER_ROW + part);
          d_off[m] = static_cast<int64_t>(s) * RC_UNITS_PER_ROW + part;
          // two misses sharing a host index leave the map pointing at only one of their slots
          if (part == 0 && host_to_gpu[h] != s) atomicOr(status, ECHO_ST_DUP_HOST);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < RC_PER_THREAD; ++m)
      if (d_off[m] >= 0) dst[d_off[m]] = v[m];
  }
}

int launch_recall_gather(const echo_pool *pool, const int32_t *miss_host, const int32_t *miss_slot,
                         const int32_t *n_miss, int32_t max_miss, hipStream_t st) {
  if (max_miss <= 0) return ECHO_OK;
  const int blocks = std::min(2048, (max_miss + RC_ROWS - 1) / RC_ROWS);
  recall_gather_kernel<<<blocks, RC_THREADS, 0, st>>>(pool->host_kv, pool->gpu_kv, miss_host, miss_slot,
                                                      n_miss, max_miss, pool->status, pool->host_to_gpu,
                                                      pool->n_host, pool->n_gpu);
  return check_launch("recall_gather");
}

// Scatter: 64 threads move 8 staged rows; the count and the block's list entries are read
// together, then the staged rows and the duplicate check, then the stores.
constexpr int SC_THREADS = 64;
constexpr int SC_ROWS = 8;
constexpr int SC_PER = SC_ROWS * RC_UNITS_PER_ROW / SC_THREADS;   // 9

__global__ __launch_bounds__(SC_THREADS) void recall_scatter_kernel(
    const uint16_t *__restrict__ stage, uint16_t *__restrict__ gpu_kv,
    const int32_t *__restrict__ miss_host, const int32_t *__restrict__ miss_slot,
    const int32_t *__restrict__ miss_stage, const int32_t *__restrict__ n_miss_p, int32_t max_miss,
    int32_t *__restrict__ status, const int32_t *__restrict__ host_to_gpu, int32_t n_host,
    int32_t n_gpu) {
  const int32_t r0 = blockIdx.x * SC_ROWS;
  const int32_t st = *(volatile const int32_t *)status;
  const int32_t n = min(*n_miss_p, max_miss);
  int32_t h[SC_PER], s[SC_PER], g[SC_PER];
#pragma unroll
  for (int m = 0; m < SC_PER; ++m) {
    const int32_t row = r0 + (threadIdx.x + m * SC_THREADS) / RC_UNITS_PER_ROW;
    const bool in = row < max_miss;
    h[m] = in ? miss_host[row] : -1;
    s[m] = in ? miss_slot[row] : -1;
    g[m] = in ? miss_stage[row] : -1;
  }
  if (st != 0 || r0 >= n) return;
  const v4i *src = reinterpret_cast<const v4i *>(stage);
  v4i *dst = reinterpret_cast<v4i *>(gpu_kv);
  v4i v[SC_PER];
  int64_t d_off[SC_PER];
  bool dup = false;
#pragma unroll
  for (int m = 0; m < SC_PER; ++m) {
    const int u = threadIdx.x + m * SC_THREADS;
    const int32_t row = r0 + u / RC_UNITS_PER_ROW;
    const int part = u % RC_UNITS_PER_ROW;
    d_off[m] = -1;
    if (row < n && h[m] >= 0 && h[m] < n_host && s[m] >= 0 && s[m] < n_gpu && g[m] >= 0) {
      v[m] = src[static_cast<int64_t>(g[m]) * RC_UNITS_PER_ROW + part];
      d_off[m] = static_cast<int64_t>(s[m]) * RC_UNITS_PER_ROW + part;
      // two misses sharing a host index leave the map pointing at only one of their slots
      if (part == 0 && host_to_gpu[h[m]] != s[m]) dup = true;
    }
  }
  if (dup) atomicOr(status, ECHO_ST_DUP_HOST);
#pragma unroll
  for (int m = 0; m < SC_PER; ++m)
    if (d_off[m] >= 0) dst[d_off[m]] = v[m];
}

int launch_recall_scatter(const echo_pool *pool, const PoolFastWs &W, const int32_t *miss_host,
                          const int32_t *miss_slot, const int32_t *n_miss, int32_t max_miss,
                          const uint16_t *stage, hipStream_t st) {
  if (max_miss <= 0) return ECHO_OK;
  const int blocks = (max_miss + SC_ROWS - 1) / SC_ROWS;
  recall_scatter_kernel<<<blocks, SC_THREADS, 0, st>>>(stage, pool->gpu_kv, miss_host, miss_slot, W.miss_stage,
                                                       n_miss, max_miss, pool->status, pool->host_to_gpu,
                                                       pool->n_host, pool->n_gpu);
  return check_launch("recall_scatter");
}

static int recall_memcpy(const echo_pool *pool, const int32_t *miss_host, const int32_t *miss_slot,
                         const int32_t *n_miss, int32_t max_miss, hipStream_t st) {
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(ECHO_EHIP, "echo_recall(memcpy): sync: %s", hipGetErrorString(e));
  int32_t n = 0, status = 0;
  if ((e = hipMemcpy(&n, n_miss, 4, hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(&status, pool->status, 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return fail(ECHO_EHIP, "echo_recall(memcpy): read count: %s", hipGetErrorString(e));
  if (status) return ECHO_OK;
  n = n < max_miss ? n : max_miss;
  if (n <= 0) return ECHO_OK;
  std::vector<int32_t> h, s;
  try {
    h.resize(n);
    s.resize(n);
  } catch (const std::bad_alloc &) {
    return fail(ECHO_EHIP, "echo_recall(memcpy): out of host memory for %d list entries", n);
  }
  if ((e = hipMemcpy(h.data(), miss_host, 4 * static_cast<size_t>(n), hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(s.data(), miss_slot, 4 * static_cast<size_t>(n), hipMemcpyDeviceToHost)) != hipSuccess)
    return fail(ECHO_EHIP, "echo_recall(memcpy): read lists: %s", hipGetErrorString(e));
  const size_t rb = ROW * 2;
  for (int32_t i = 0; i < n; ++i) {
    if (h[i] < 0 || h[i] >= pool->n_host || s[i] < 0 || s[i] >= pool->n_gpu) continue;
    e = hipMemcpyAsync(pool->gpu_kv + static_cast<size_t>(s[i]) * ROW,
                       pool->host_kv + static_cast<size_t>(h[i]) * ROW, rb, hipMemcpyDefault, st);
    if (e != hipSuccess) return fail(ECHO_EHIP, "echo_recall(memcpy): %s", hipGetErrorString(e));
  }
  return ECHO_OK;
}

}  // namespace echo

using namespace echo;

extern "C" int echo_recall(const echo_pool *pool, const int32_t *miss_host,
                           const int32_t *miss_slot, const int32_t *n_miss, int32_t max_miss,
                           int32_t mode, void *stream) {
  if (!pool || !pool->gpu_kv || !pool->host_kv || !pool->status || !pool->host_to_gpu)
    return fail(ECHO_EINVAL, "echo_recall: NULL pool member");
  if (pool->n_gpu < 1 || pool->n_host < 1) return fail(ECHO_EINVAL, "echo_recall: empty pool");
  if (max_miss < 0) return fail(ECHO_EINVAL, "echo_recall: max_miss < 0");
  if (max_miss > 0 && (!miss_host || !miss_slot || !n_miss)) return fail(ECHO_EINVAL, "echo_recall: NULL list");
  if (mode == ECHO_RECALL_GATHER) return launch_recall_gather(pool, miss_host, miss_slot, n_miss, max_miss, S(stream));
  if (mode == ECHO_RECALL_MEMCPY) return recall_memcpy(pool, miss_host, miss_slot, n_miss, max_miss, S(stream));
  return fail(ECHO_EINVAL, "echo_recall: unknown mode %d", mode);
}
