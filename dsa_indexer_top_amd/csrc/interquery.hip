// Inter-query prefetch for a chunked prefill (ECHO review page §6.2).  The indexer scores the
// prefill's query blocks in order, so the tokens a block selected can be fetched while the next
// block is scored.  An exact top-k there would slow the indexer, so an approximate top-k gives
// a subset of each row's top-k.  Each score is shifted by a prediction of the k-th score and
// mapped by the top 8 bits of its order key to one of 256 bins.  The highest bins whose total
// stays within k are taken whole, and the next one down is the threshold bin.  The shift puts
// the threshold where the bins are finest, so the threshold bin stays small and the subset
// close to the whole top-k.
//
//   topk_subset_kernel   one workgroup per row: LDS histogram of the shifted keys (the wave's
//                        most common bin peeled off first), threshold bin by a wave scan over
//                        the 256 bins, then an ordered compaction of the tokens above it.
//   union_mark_kernel    the union of index lists as a bitmap over the keys ...
//   union_compact_kernel ... listed in ascending order, segment s = keys [4096 s, 4096 s + 4096),
//                        one workgroup per segment; a fixed shape that the pool step and the
//                        prefetch gather take as 4096-wide "rows" with key_begin 0.
#include <algorithm>

#include "internal.hpp"

namespace echo {

constexpr int SB_T = 1024;           // threads per row
constexpr int UN_SEG = 4096;         // keys per union segment
constexpr int UN_T = 256;            // threads per segment: 16 keys each

// Bin of a shifted score: the top 8 bits of its order key (-0 folded onto +0).
ECHO_DEV uint32_t shifted_bin(float s, float shift) { return f32_key(s - shift) >> 24; }

__global__ __launch_bounds__(SB_T) void topk_subset_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ len, int32_t max_len,
    int32_t k, const float *__restrict__ shift_p, int32_t *__restrict__ subset,
    int32_t *__restrict__ subset_cnt, int32_t *__restrict__ thr_cnt) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[48];
  __shared__ int32_t thr_s[2];
  const int r = blockIdx.x, t = threadIdx.x;
  const int32_t L = min(max(len[r], 0), max_len);
  float shift = shift_p ? *shift_p : 0.f;
  if (__builtin_isnan(shift)) shift = 0.f;             // no prediction yet
  const float *__restrict__ row = scores + static_cast<int64_t>(r) * ld;
  if (t < 256) hist[t] = 0;
  __syncthreads();
  for (int32_t j0 = 0; j0 < L; j0 += SB_T) {
    const int32_t j = j0 + t;
    const bool act = j < L;
    hist_add_peeled(hist, act ? shifted_bin(row[j], shift) : 0u, act);
  }
  __syncthreads();
  // threshold bin: lane l of wave 0 holds bins 255-4l .. 252-4l (descending); the first lane
  // whose running total passes k holds it
  if (t < 64) {
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = hist[255 - 4 * t - i];
      sum += c[i];
    }
    const uint32_t incl = wave_incl_scan(sum);
    const uint64_t over = __ballot(incl > static_cast<uint32_t>(k));
    // in every lane: the bin of its group where the running total would pass k
    uint32_t run = incl - sum;
    int b = 255 - 4 * t;
    for (int i = 0; i < 4; ++i, --b) {
      if (run + c[i] > static_cast<uint32_t>(k)) break;
      run += c[i];
    }
    // the threshold bin is the first such lane's; none when every bin fits
    const int first = over ? __ffsll(static_cast<unsigned long long>(over)) - 1 : 0;
    const int thr = over ? __builtin_amdgcn_readlane(b, first) : -1;
    if (t == 0) thr_s[0] = thr;
  }
  __syncthreads();
  const int32_t thr = thr_s[0];
  // the tokens above the threshold bin, in ascending order
  uint32_t base = 0;
  for (int32_t j0 = 0; j0 < L; j0 += SB_T) {
    const int32_t j = j0 + t;
    const bool take = j < L && static_cast<int32_t>(shifted_bin(row[j], shift)) > thr;
    uint32_t tot;
    const uint32_t pos = base + block_excl_scan<SB_T>(take ? 1u : 0u, tmp, &tot);
    if (take) subset[static_cast<int64_t>(r) * k + pos] = j;
    base += tot;
  }
  for (int32_t j = static_cast<int32_t>(base) + t; j < k; j += SB_T) subset[static_cast<int64_t>(r) * k + j] = -1;
  if (t == 0) {
    subset_cnt[r] = static_cast<int32_t>(base);
    if (thr_cnt) thr_cnt[r] = thr >= 0 ? static_cast<int32_t>(hist[thr]) : 0;
  }
}

__global__ __launch_bounds__(256) void union_mark_kernel(const int32_t *__restrict__ idx, int64_t n,
                                                         int32_t n_keys, uint32_t *__restrict__ bits) {
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < n; e += static_cast<int64_t>(gridDim.x) * 256) {
    const int32_t v = idx[e];
    if (v >= 0 && v < n_keys) atomicOr(&bits[v >> 5], 1u << (v & 31));
  }
}

__global__ __launch_bounds__(UN_T) void union_compact_kernel(const uint32_t *__restrict__ bits,
                                                             int32_t n_keys, int32_t *__restrict__ out,
                                                             int32_t *__restrict__ cnt) {
  __shared__ uint32_t tmp[48];
  const int s = blockIdx.x, t = threadIdx.x;
  const int32_t key0 = s * UN_SEG + t * 16;               // this thread's 16 keys
  const int32_t word = key0 >> 5;
  uint32_t m = 0;
  if (key0 < n_keys) m = (bits[word] >> (key0 & 31)) & 0xFFFFu;
  const int32_t lim = n_keys - key0;                     // keys past n_keys are never marked
  if (lim < 16) m &= lim <= 0 ? 0u : ((1u << lim) - 1u);
  uint32_t tot;
  uint32_t pos = block_excl_scan<UN_T>(static_cast<uint32_t>(__popc(m)), tmp, &tot);
  int32_t *__restrict__ o = out + static_cast<int64_t>(s) * UN_SEG;
  while (m) {
    const int b = __ffs(m) - 1;
    o[pos++] = key0 + b;
    m &= m - 1;
  }
  for (int32_t j = static_cast<int32_t>(tot) + t; j < UN_SEG; j += UN_T) o[j] = -1;
  if (t == 0) cnt[s] = static_cast<int32_t>(tot);
}

static int32_t n_segments(int32_t n_keys) { return n_keys <= 0 ? 1 : (n_keys + UN_SEG - 1) / UN_SEG; }

}  // namespace echo

using namespace echo;

extern "C" int echo_topk_subset(const float *scores, int64_t ld, const int32_t *len, int32_t n_rows,
                                int32_t max_len, int32_t k, const float *shift, int32_t *subset,
                                int32_t *subset_cnt, int32_t *thr_cnt, void *stream) {
  if (n_rows < 0 || max_len < 0) return fail(ECHO_EINVAL, "echo_topk_subset: negative size");
  if (k < 1 || k > ECHO_MAX_TOPK) return fail(ECHO_EUNSUPPORTED, "echo_topk_subset: k %d outside [1, %d]", k, ECHO_MAX_TOPK);
  if (ld < max_len) return fail(ECHO_EINVAL, "echo_topk_subset: ld < max_len");
  if (n_rows > 0 && (!scores || !len || !subset || !subset_cnt))
    return fail(ECHO_EINVAL, "echo_topk_subset: NULL pointer");
  if (n_rows == 0) return ECHO_OK;
  topk_subset_kernel<<<n_rows, SB_T, 0, S(stream)>>>(scores, ld, len, max_len, k, shift, subset,
                                                     subset_cnt, thr_cnt);
  return check_launch("topk_subset");
}

extern "C" size_t echo_union_workspace_bytes(int32_t n_keys) {
  if (n_keys < 0) return 0;
  return static_cast<size_t>(n_segments(n_keys)) * (UN_SEG / 32) * 4;
}

extern "C" int echo_union_rows(const int32_t *idx, int32_t n_rows, int32_t k, int32_t n_keys,
                               int32_t *out, int32_t *out_cnt, void *ws, size_t ws_bytes,
                               void *stream) {
  if (n_rows < 0 || k < 0 || n_keys < 0) return fail(ECHO_EINVAL, "echo_union_rows: negative size");
  if (n_keys > (1 << 30)) return fail(ECHO_EUNSUPPORTED, "echo_union_rows: more than 2^30 keys");
  if (!out || !out_cnt || !ws || (static_cast<int64_t>(n_rows) * k > 0 && !idx))
    return fail(ECHO_EINVAL, "echo_union_rows: NULL pointer");
  const size_t need = echo_union_workspace_bytes(n_keys);
  if (ws_bytes < need) return fail(ECHO_EWORKSPACE, "echo_union_rows: workspace %zu < %zu", ws_bytes, need);
  hipStream_t st = S(stream);
  const int32_t n_seg = n_segments(n_keys);
  uint32_t *bits = static_cast<uint32_t *>(ws);
  int rc = launch_zero_i32(reinterpret_cast<int32_t *>(bits), static_cast<int64_t>(n_seg) * (UN_SEG / 32), st);
  if (rc) return rc;
  const int64_t n = static_cast<int64_t>(n_rows) * k;
  if (n > 0) {
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    union_mark_kernel<<<static_cast<unsigned>(blocks), 256, 0, st>>>(idx, n, n_keys, bits);
    if ((rc = check_launch("union_mark"))) return rc;
  }
  union_compact_kernel<<<n_seg, UN_T, 0, st>>>(bits, n_keys, out, out_cnt);
  return check_launch("union_compact");
}

extern "C" int echo_threshold_ema(const float *scores, int64_t ld, const int32_t *idx,
                                  int32_t n_rows, int32_t k, float alpha, float *theta,
                                  float *kth, void *stream) {
  if (n_rows < 0 || ld < 0) return fail(ECHO_EINVAL, "echo_threshold_ema: negative size");
  if (k < 1 || k > ECHO_MAX_TOPK) return fail(ECHO_EUNSUPPORTED, "echo_threshold_ema: k %d outside [1, %d]", k, ECHO_MAX_TOPK);
  if (!(alpha >= 0.f && alpha <= 1.f)) return fail(ECHO_EINVAL, "echo_threshold_ema: alpha outside [0, 1]");
  if (n_rows > 0 && (!scores || !idx || (!theta && !kth)))
    return fail(ECHO_EINVAL, "echo_threshold_ema: NULL pointer");
  return launch_kth_ema(scores, ld, idx, n_rows, k, alpha, theta, kth, S(stream));
}
