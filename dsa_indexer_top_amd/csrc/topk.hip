// Exact top-k of the indexer scores (ECHO review page §2: the top-k tokens feed sparse
// attention, so every score must be known first).  Ties at the k-th score go to the lower
// token index; -0.0 equals +0.0; the output lists the selected indices in ascending order,
// -1 padded to k.
//
// Selecting the k largest scores is selecting the k smallest keys ~order_key(score), done by
// the segmented radix select of select.cuh (one segment per row, 4096-score chunks per
// workgroup): three histogram passes, one count pass, one apply pass.
#include <algorithm>

#include "internal.hpp"
#include "select.cuh"

namespace echo {

struct TopkSrc {
  const float *scores;
  int64_t ld;
  const int32_t *len;
  int32_t max_len;
  int32_t k;
  ECHO_DEV int32_t n(int seg) const { return min(max(len[seg], 0), max_len); }
  ECHO_DEV bool get(int seg, int32_t i, uint32_t &key) const {
    key = ~f32_key(scores[static_cast<int64_t>(seg) * ld + i]);
    return true;
  }
  ECHO_DEV uint32_t m(int seg) const { return static_cast<uint32_t>(min(k, n(seg))); }
};

__global__ void zero_u32_kernel(uint32_t *p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

int launch_zero_i32(int32_t *p, int64_t n, hipStream_t st) {
  if (n <= 0) return ECHO_OK;
  zero_u32_kernel<<<static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 4096)), 256, 0, st>>>(
      reinterpret_cast<uint32_t *>(p), n);
  return check_launch("zero");
}

template <int DIG>
__global__ __launch_bounds__(SEL_THREADS) void topk_hist_kernel(TopkSrc src, SelWs ws) {
  __shared__ uint32_t hl[SEL_COPIES * SEL_BINS];
  __shared__ uint32_t tmp[48];
  const int seg = blockIdx.y, chunk = blockIdx.x;
  if (chunk == 0 && DIG < 2) sel_zero_hist(ws, seg, DIG + 1);
  const uint32_t m = src.m(seg);
  Pick p{0u, 0u, m, 0, 0};
  if (DIG > 0) p = sel_pick(ws, seg, DIG, m, tmp);
  const int32_t n = src.n(seg);
  if (m == 0 || m >= static_cast<uint32_t>(n) || p.none || p.all) return;
  if (chunk * SEL_CHUNK >= n) return;
  sel_hist_chunk(src, ws, seg, chunk, DIG, p, hl);
}

// Count of keys below K* (or eligible, when everything is taken) and equal to K*, per chunk.
template <class Src>
ECHO_DEV void sel_count_chunk(const Src &src, const SelWs &ws, int seg, int chunk, const Pick &p,
                              uint32_t *tmp) {
  const int32_t n = src.n(seg);
  const int32_t base = chunk * SEL_CHUNK;
  uint32_t lt = 0, eq = 0;
  for (int e = 0; e < SEL_PER_THREAD; ++e) {
    const int32_t i = base + e * SEL_THREADS + threadIdx.x;
    if (i < n) {
      const int c = sel_class(src, seg, i, p);
      lt += (c == 1);
      eq += (c == 2);
    }
  }
  lt = block_sum<SEL_THREADS>(lt, tmp);
  eq = block_sum<SEL_THREADS>(eq, tmp);
  if (threadIdx.x == 0) {
    ws.chunk_lt[static_cast<int64_t>(seg) * ws.n_chunks + chunk] = lt;
    ws.chunk_eq[static_cast<int64_t>(seg) * ws.n_chunks + chunk] = eq;
  }
}

__global__ __launch_bounds__(SEL_THREADS) void topk_count_kernel(TopkSrc src, SelWs ws) {
  __shared__ uint32_t tmp[48];
  const int seg = blockIdx.y, chunk = blockIdx.x;
  const Pick p = sel_pick(ws, seg, 3, src.m(seg), tmp);
  if (p.none || chunk * SEL_CHUNK >= src.n(seg)) return;
  sel_count_chunk(src, ws, seg, chunk, p, tmp);
}

// Exclusive sums over the chunks before `chunk`: (lt_before, eq_before).
ECHO_DEV void sel_chunk_prefix(const SelWs &ws, int seg, int chunk, uint32_t *tmp,
                               uint32_t &lt_before, uint32_t &eq_before) {
  uint32_t lt = 0, eq = 0;
  for (int c = threadIdx.x; c < chunk; c += SEL_THREADS) {
    lt += ws.chunk_lt[static_cast<int64_t>(seg) * ws.n_chunks + c];
    eq += ws.chunk_eq[static_cast<int64_t>(seg) * ws.n_chunks + c];
  }
  lt_before = block_sum<SEL_THREADS>(lt, tmp);
  eq_before = block_sum<SEL_THREADS>(eq, tmp);
}

__global__ __launch_bounds__(SEL_THREADS) void topk_apply_kernel(TopkSrc src, SelWs ws,
                                                                 int32_t *__restrict__ idx) {
  __shared__ uint32_t tmp[48];
  __shared__ uint8_t cls_lds[SEL_THREADS * (SEL_PER_THREAD + 1)];
  const int seg = blockIdx.y, chunk = blockIdx.x;
  const int32_t n = src.n(seg);
  const uint32_t m = src.m(seg);
  int32_t *out = idx + static_cast<int64_t>(seg) * src.k;
  if (chunk == 0)
    for (int j = static_cast<int>(m) + threadIdx.x; j < src.k; j += SEL_THREADS) out[j] = -1;
  const Pick p = sel_pick(ws, seg, 3, m, tmp);
  if (p.none || chunk * SEL_CHUNK >= n) return;
  uint32_t lt_before, eq_before;
  sel_chunk_prefix(ws, seg, chunk, tmp, lt_before, eq_before);
  const int32_t base = chunk * SEL_CHUNK;
  // classify coalesced, then let each thread walk 16 consecutive elements in index order
  for (int e = 0; e < SEL_PER_THREAD; ++e) {
    const int li = e * SEL_THREADS + threadIdx.x;
    const int32_t i = base + li;
    const int c = (i < n) ? sel_class(src, seg, i, p) : 0;
    cls_lds[(li >> 4) * (SEL_PER_THREAD + 1) + (li & 15)] = static_cast<uint8_t>(c);
  }
  __syncthreads();
  const uint8_t *mine = cls_lds + threadIdx.x * (SEL_PER_THREAD + 1);
  uint32_t n_eq = 0;
  for (int e = 0; e < SEL_PER_THREAD; ++e) n_eq += (mine[e] == 2);
  uint32_t tot;
  const uint32_t eq_rank0 = eq_before + block_excl_scan<SEL_THREADS>(n_eq, tmp, &tot);
  uint32_t n_sel = 0;
  {
    uint32_t r = eq_rank0;
    for (int e = 0; e < SEL_PER_THREAD; ++e) {
      const int c = mine[e];
      if (c == 1) ++n_sel;
      else if (c == 2) { if (r < p.k_rem) ++n_sel; ++r; }
    }
  }
  const uint32_t sel_before = lt_before + min(eq_before, p.k_rem);
  uint32_t pos = sel_before + block_excl_scan<SEL_THREADS>(n_sel, tmp, &tot);
  uint32_t r = eq_rank0;
  const int32_t i0 = base + threadIdx.x * SEL_PER_THREAD;
  for (int e = 0; e < SEL_PER_THREAD; ++e) {
    const int c = mine[e];
    bool take = (c == 1);
    if (c == 2) { take = r < p.k_rem; ++r; }
    if (take) {
      if (pos < static_cast<uint32_t>(src.k)) out[pos] = i0 + e;
      ++pos;
    }
  }
}

size_t topk_ws_bytes(int32_t n_rows, int32_t max_len) {
  return sel_ws_bytes(n_rows, std::max(1, (max_len + SEL_CHUNK - 1) / SEL_CHUNK));
}

int launch_topk(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                int32_t max_len, int32_t k, int32_t *idx, void *ws, size_t ws_bytes,
                hipStream_t st) {
  if (n_rows == 0) return ECHO_OK;
  const int32_t n_chunks = std::max(1, (max_len + SEL_CHUNK - 1) / SEL_CHUNK);
  const size_t need = sel_ws_bytes(n_rows, n_chunks);
  if (ws_bytes < need) return fail(ECHO_EWORKSPACE, "echo_topk: workspace %zu < %zu", ws_bytes, need);
  SelWs w;
  w.hist = static_cast<uint32_t *>(ws);
  w.chunk_lt = w.hist + static_cast<size_t>(3) * n_rows * SEL_BINS;
  w.chunk_eq = w.chunk_lt + static_cast<size_t>(n_rows) * n_chunks;
  w.n_chunks = n_chunks;
  TopkSrc src{scores, ld, len, max_len, k};
  const int64_t nz = static_cast<int64_t>(n_rows) * SEL_BINS;
  zero_u32_kernel<<<static_cast<unsigned>(std::min<int64_t>((nz + 255) / 256, 4096)), 256, 0, st>>>(w.hist, nz);
  dim3 grid(n_chunks, n_rows);
  topk_hist_kernel<0><<<grid, SEL_THREADS, 0, st>>>(src, w);
  topk_hist_kernel<1><<<grid, SEL_THREADS, 0, st>>>(src, w);
  topk_hist_kernel<2><<<grid, SEL_THREADS, 0, st>>>(src, w);
  topk_count_kernel<<<grid, SEL_THREADS, 0, st>>>(src, w);
  topk_apply_kernel<<<grid, SEL_THREADS, 0, st>>>(src, w, idx);
  return check_launch("topk");
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
  if (n_rows > 65535) return fail(ECHO_EUNSUPPORTED, "echo_topk: n_rows %d > 65535", n_rows);
  if (n_rows > 0 && (!scores || !len || !idx || !ws)) return fail(ECHO_EINVAL, "echo_topk: NULL pointer");
  return launch_topk(scores, ld, len, n_rows, max_len, k, idx, ws, ws_bytes, S(stream));
}
