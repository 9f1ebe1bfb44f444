// What carries a decode step over to the next one (ECHO review page):
//   * §2 and §5.2: a newly generated token's latent row is backed up to host memory when it is
//     generated (which is why eviction never moves data), and allocate serves newly generated
//     KV as well as recalled tokens.  echo_decode_append does this for one new token per
//     request.
//   * §6.1: the k-th largest score of a layer is predicted for the next step by an exponential
//     moving average of the actual k-th scores; tokens scoring above the prediction are
//     prefetched while the indexer runs.  launch_kth_ema ends a decode step with that update.
//
// Append: one launch writes each request's token into the K cache (key, key scale, host
// index, length) and its latent row through the host link into its host row, and lists its
// position as a one-column selection; the pool step's lookup / evict / allocate (k = 1) gives
// every new token a slot; a last launch copies the rows from the tokens' own device copies into
// those slots (the host copy was only just written, so reading it back would cost a host-link
// round trip).
#include "internal.hpp"

namespace echo {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int AP_THREADS = 128;
constexpr int AP_ROW_UNITS = ROW * 2 / 16;     // 72 x 16 B per latent row
constexpr int AP_KEY_UNITS = D / 16;           // 8 x 16 B per indexer key
static_assert(AP_ROW_UNITS + AP_KEY_UNITS + 1 <= AP_THREADS, "one thread per 16-byte unit");

static size_t al(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

struct AppendWs {
  int32_t *pos;        // [n_rows] the new token's index in its request, -1 if not appended
  int32_t *miss_host;  // [n_rows]
  int32_t *miss_slot;  // [n_rows]
  int32_t *n_miss;     // [1]
  void *pool;
  size_t pool_bytes;
};

static size_t append_ws_layout(int32_t n_rows, int32_t n_gpu, void *base, AppendWs *w) {
  size_t off = 0;
  auto take = [&](size_t b) { size_t o = off; off += al(b); return o; };
  const size_t nr = static_cast<size_t>(n_rows);
  const size_t o_pos = take(nr * 4), o_mh = take(nr * 4), o_ms = take(nr * 4), o_n = take(4);
  const size_t pbytes = pool_fast_ws_bytes(n_rows, 1, n_gpu);
  const size_t o_pool = take(pbytes);
  if (w && base) {
    char *b = static_cast<char *>(base);
    w->pos = reinterpret_cast<int32_t *>(b + o_pos);
    w->miss_host = reinterpret_cast<int32_t *>(b + o_mh);
    w->miss_slot = reinterpret_cast<int32_t *>(b + o_ms);
    w->n_miss = reinterpret_cast<int32_t *>(b + o_n);
    w->pool = b + o_pool;
    w->pool_bytes = pbytes;
  }
  return off;
}

// One workgroup per request: threads 0..71 copy the latent row to the host backup, 72..79 the
// key, 80 the bookkeeping; the length is bumped after every thread has read it.
__global__ __launch_bounds__(AP_THREADS) void append_kernel(echo_append_args a, int32_t *pos,
                                                            int32_t *status, int32_t n_host) {
  const int r = blockIdx.x, t = threadIdx.x;
  const int32_t p = a.key_len[r];
  const int64_t row = a.key_begin[r] + p;
  const bool room = p >= 0 && p < a.capacity && row >= 0 && row < a.n_k;
  if (!room) {                                   // uniform over the workgroup
    if (t == 0) {
      pos[r] = -1;
      atomicOr(status, ECHO_ST_CACHE_FULL);
    }
    return;
  }
  const int32_t h = a.new_host[r];
  if (t < AP_ROW_UNITS) {
    if (h >= 0 && h < n_host) {                  // else the lookup reports the bad host index
      const v4i v = reinterpret_cast<const v4i *>(a.new_kv)[static_cast<int64_t>(r) * AP_ROW_UNITS + t];
      reinterpret_cast<v4i *>(a.host_kv_w)[static_cast<int64_t>(h) * AP_ROW_UNITS + t] = v;
    }
  } else if (t < AP_ROW_UNITS + AP_KEY_UNITS) {
    const int u = t - AP_ROW_UNITS;
    reinterpret_cast<v4i *>(a.k)[row * AP_KEY_UNITS + u] =
        reinterpret_cast<const v4i *>(a.new_k)[static_cast<int64_t>(r) * AP_KEY_UNITS + u];
  } else if (t == AP_ROW_UNITS + AP_KEY_UNITS) {
    a.req_to_host[row] = h;
    if (a.k_scale && a.new_scale) a.k_scale[row] = a.new_scale[r];
    pos[r] = p;
  }
  __syncthreads();
  if (t == 0) a.key_len[r] = p + 1;
}

// The new tokens' rows into their slots, from the tokens' own copies.
__global__ __launch_bounds__(AP_THREADS) void append_fill_kernel(
    const uint16_t *__restrict__ new_kv, const int32_t *__restrict__ slot, uint16_t *__restrict__ gpu_kv,
    const int32_t *__restrict__ status, int32_t n_gpu) {
  if (*(volatile const int32_t *)status) return;
  const int r = blockIdx.x, t = threadIdx.x;
  const int32_t s = slot[r];
  if (s < 0 || s >= n_gpu || t >= AP_ROW_UNITS) return;
  reinterpret_cast<v4i *>(gpu_kv)[static_cast<int64_t>(s) * AP_ROW_UNITS + t] =
      reinterpret_cast<const v4i *>(new_kv)[static_cast<int64_t>(r) * AP_ROW_UNITS + t];
}

// ---------------------------------------------------------------- k-th score and its EMA
constexpr int KE_THREADS = 256;

// One workgroup per request: kth = the smallest score among the selected tokens (NaN when
// none); theta = kth when theta is NaN (no estimate yet), else alpha * theta + (1 - alpha) *
// kth, rounded once (fmaf); a request with no selection keeps theta.
__global__ __launch_bounds__(KE_THREADS) void kth_ema_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ idx, int32_t k,
    float alpha, float *__restrict__ theta, float *__restrict__ kth) {
  __shared__ float red[KE_THREADS / 64];
  const int r = blockIdx.x, t = threadIdx.x;
  const float *__restrict__ srow = scores + static_cast<int64_t>(r) * ld;
  const int32_t *__restrict__ irow = idx + static_cast<int64_t>(r) * k;
  float m = __builtin_inff();
  bool any = false;
  for (int32_t j = t; j < k; j += KE_THREADS) {
    const int32_t s = irow[j];
    if (s >= 0 && s < ld) {
      m = fminf(m, srow[s]);
      any = true;
    }
  }
  // no selection anywhere in the request -> NaN; -0 and +0 compare equal, either may remain
  unsigned long long ok = __ballot(any);
  for (int o = 32; o >= 1; o >>= 1) m = fminf(m, __shfl_xor(m, o, 64));
  if ((t & 63) == 0) red[t >> 6] = ok ? m : __builtin_nanf("");
  __syncthreads();
  if (t == 0) {
    float v = __builtin_nanf("");
    bool have = false;
    for (int i = 0; i < KE_THREADS / 64; ++i)
      if (!__builtin_isnan(red[i])) {
        v = have ? fminf(v, red[i]) : red[i];
        have = true;
      }
    if (kth) kth[r] = v;
    if (theta && have) {
      const float old = theta[r];
      theta[r] = __builtin_isnan(old) ? v : fmaf(alpha, old, (1.0f - alpha) * v);
    }
  }
}

int launch_kth_ema(const float *scores, int64_t ld, const int32_t *idx, int32_t n_rows, int32_t k,
                   float alpha, float *theta, float *kth, hipStream_t st) {
  if (n_rows == 0 || (!theta && !kth)) return ECHO_OK;
  kth_ema_kernel<<<n_rows, KE_THREADS, 0, st>>>(scores, ld, idx, k, alpha, theta, kth);
  return check_launch("kth_ema");
}

static int append_impl(const echo_append_args *a, const echo_pool *pool, int32_t *new_slot,
                       void *ws, size_t ws_bytes, hipStream_t st) {
  if (!a || !pool || !new_slot) return fail(ECHO_EINVAL, "echo_decode_append: NULL argument");
  if (a->n_rows < 1 || a->n_rows > 65535) return fail(ECHO_EUNSUPPORTED, "echo_decode_append: n_rows %d outside [1, 65535]", a->n_rows);
  if (a->capacity < 1 || a->n_k < 1) return fail(ECHO_EINVAL, "echo_decode_append: capacity and n_k must be >= 1");
  if (!a->new_k || !a->new_kv || !a->new_host || !a->k || !a->key_begin || !a->key_len ||
      !a->req_to_host || !a->host_kv_w)
    return fail(ECHO_EINVAL, "echo_decode_append: NULL input");
  if ((a->k_scale == nullptr) != (a->new_scale == nullptr))
    return fail(ECHO_EINVAL, "echo_decode_append: k_scale and new_scale must both be given or both be NULL");
  if (pool->n_gpu < 1 || pool->n_host < 1 || !pool->gpu_free || !pool->gpu_priority ||
      !pool->gpu_to_host || !pool->host_to_gpu || !pool->indices_buf || !pool->gpu_kv || !pool->status)
    return fail(ECHO_EINVAL, "echo_decode_append: incomplete pool");
  if (pool->n_gpu > (1 << 22)) return fail(ECHO_EUNSUPPORTED, "echo_decode_append: more than 4M GPU slots");
  AppendWs W{};
  const size_t need = append_ws_layout(a->n_rows, pool->n_gpu, ws, &W);
  if (!ws || ws_bytes < need) return fail(ECHO_EWORKSPACE, "echo_decode_append: workspace %zu < %zu", ws_bytes, need);
  append_kernel<<<a->n_rows, AP_THREADS, 0, st>>>(*a, W.pos, pool->status, pool->n_host);
  int rc = check_launch("append");
  if (rc) return rc;
  if ((rc = launch_pool_step(pool, W.pos, a->key_begin, a->req_to_host, a->n_k, a->n_rows, 1,
                             Stamp{a->step_id, a->step_dev}, new_slot, W.miss_host, W.miss_slot, W.n_miss, W.pool,
                             W.pool_bytes, st)))
    return rc;
  append_fill_kernel<<<a->n_rows, AP_THREADS, 0, st>>>(a->new_kv, new_slot, pool->gpu_kv,
                                                       pool->status, pool->n_gpu);
  return check_launch("append_fill");
}

__global__ void step_advance_kernel(int32_t *step) { *step += 1; }

}  // namespace echo

using namespace echo;

extern "C" int echo_step_advance(int32_t *step_dev, void *stream) {
  if (!step_dev) return fail(ECHO_EINVAL, "echo_step_advance: NULL");
  step_advance_kernel<<<1, 1, 0, S(stream)>>>(step_dev);
  return check_launch("step_advance");
}

extern "C" size_t echo_append_workspace_bytes(int32_t n_rows, int32_t n_gpu) {
  if (n_rows < 0 || n_gpu < 0) return 0;
  return append_ws_layout(n_rows, n_gpu, nullptr, nullptr);
}

extern "C" int echo_decode_append(const echo_append_args *a, const echo_pool *pool,
                                  int32_t *new_slot, void *ws, size_t ws_bytes, void *stream) {
  return append_impl(a, pool, new_slot, ws, ws_bytes, S(stream));
}
