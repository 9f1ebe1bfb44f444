// Prefill (causal) lightning-indexer scores on gfx950 (ECHO review page §2 score definition;
// §3.4: the indexer is quadratic in the context, every query against every earlier key).
//
// Query rows t in [0, n_q) sit at absolute positions q_pos0 + t and see keys [0, lim_t),
// lim_t = min(n_k, q_pos0 + t + 1); the diagonal is included.
//
// Work split: one query per wave (its 64 x 128 FP8 q and 64 weights stay in VGPRs in MFMA
// layout), 16 consecutive queries per 1024-thread workgroup.  The workgroup streams the keys
// [0, lim of its last query) through an LDS double buffer of 256-key stages (32 KB, loaded
// with coalesced 16-byte loads into the same swizzled layout the decode kernel uses), and
// every wave scores its query against each 16-key tile with four
// v_mfma_f32_16x16x128_f8f6f4 (one per 16-head block) followed by the ReLU * w reduction;
// tiles entirely past a wave's causal limit are skipped.  Workgroups are launched heaviest
// (latest queries) first.  Groups of four tiles are reduced so that the 64 lanes of a wave
// write 64 consecutive scores.
#include "internal.hpp"
#include "score_tile.cuh"

namespace echo {

constexpr int PF_THREADS = 1024;
constexpr int PF_QPB = PF_THREADS / 64;                 // 16 queries per workgroup
constexpr int PF_STAGE = 256;                           // keys per LDS stage
constexpr int PF_UNITS = PF_STAGE * D / 16;             // 2048 x 16 B
constexpr int PF_LOADS = PF_UNITS / PF_THREADS;         // 2 per thread

ECHO_DEV int pswz(int tok, int seg) { return tok * 128 + ((seg ^ ((tok >> 1) & 7)) << 4); }

__global__ __launch_bounds__(PF_THREADS) void score_prefill_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ w, const uint8_t *__restrict__ k,
    int32_t n_q, int32_t n_k, int32_t q_pos0, float *__restrict__ scores, int64_t ld) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][PF_STAGE * D];
  const int nblk = (n_q + PF_QPB - 1) / PF_QPB;
  const int blk = nblk - 1 - static_cast<int>(blockIdx.x);     // heaviest first
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int j = l & 15, g = l >> 4;
  const int32_t t = blk * PF_QPB + wv;
  const bool active = t < n_q;
  const int32_t lim = active ? min(n_k, q_pos0 + t + 1) : 0;
  const int32_t t_last = min(n_q - 1, blk * PF_QPB + PF_QPB - 1);
  const int32_t wg_lim = min(n_k, q_pos0 + t_last + 1);
  if (wg_lim <= 0) return;

  QOperand qo;
  if (active) load_q_operand(q, w, t, qo);
  float *__restrict__ srow = scores + static_cast<int64_t>(active ? t : 0) * ld;

  int4 pre[PF_LOADS];
  auto fetch = [&](int32_t c0) {
#pragma unroll
    for (int m = 0; m < PF_LOADS; ++m) {
      const int e = tid + m * PF_THREADS;
      const int32_t s = c0 + (e >> 3);
      if (s < wg_lim)
        pre[m] = *reinterpret_cast<const int4 *>(k + static_cast<int64_t>(s) * D + ((e & 7) << 4));
      else
        pre[m] = int4{0, 0, 0, 0};
    }
  };

  fetch(0);
  int buf = 0;
  for (int32_t c0 = 0; c0 < wg_lim; c0 += PF_STAGE) {
    uint8_t *sb = lds[buf];
#pragma unroll
    for (int m = 0; m < PF_LOADS; ++m) {
      const int e = tid + m * PF_THREADS;
      *reinterpret_cast<int4 *>(sb + pswz(e >> 3, e & 7)) = pre[m];
    }
    __syncthreads();
    if (c0 + PF_STAGE < wg_lim) fetch(c0 + PF_STAGE);
    // four 16-key tiles at a time: lane group g writes tile g's 16 scores
    for (int q4 = 0; q4 < PF_STAGE / 64; ++q4) {
      const int32_t base = c0 + q4 * 64;
      if (base >= lim) break;                       // wave-uniform: causal skip
      float part[4];
#pragma unroll
      for (int tile = 0; tile < 4; ++tile) {
        const int tt = q4 * 64 + tile * 16 + j;
        if (base + tile * 16 < lim) {
          const int4 b0 = *reinterpret_cast<const int4 *>(sb + pswz(tt, 2 * g));
          const int4 b1 = *reinterpret_cast<const int4 *>(sb + pswz(tt, 2 * g + 1));
          part[tile] = reduce_groups(score_tile_partial(qo, v8i{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w}));
        } else {
          part[tile] = 0.f;
        }
      }
      const int32_t s = base + g * 16 + j;
      const float v = g == 0 ? part[0] : (g == 1 ? part[1] : (g == 2 ? part[2] : part[3]));
      if (s < lim) srow[s] = v;
    }
    __syncthreads();
    buf ^= 1;
  }
}

int launch_score_prefill(const uint8_t *q, const float *w, const uint8_t *k, int32_t n_q,
                         int32_t n_k, int32_t q_pos0, float *scores, int64_t ld, hipStream_t st) {
  if (n_q == 0 || n_k == 0) return ECHO_OK;
  const int nblk = (n_q + PF_QPB - 1) / PF_QPB;
  score_prefill_kernel<<<nblk, PF_THREADS, 0, st>>>(q, w, k, n_q, n_k, q_pos0, scores, ld);
  return check_launch("score_prefill");
}

}  // namespace echo

using namespace echo;

extern "C" int echo_index_scores_prefill(const uint8_t *q, const float *w, const uint8_t *k,
                                         int32_t n_q, int32_t n_k, int32_t q_pos0, float *scores,
                                         int64_t ld, void *stream) {
  if (n_q < 0 || n_k < 0 || q_pos0 < 0) return fail(ECHO_EINVAL, "echo_index_scores_prefill: negative size");
  if (ld < n_k) return fail(ECHO_EINVAL, "echo_index_scores_prefill: ld < n_k");
  if (n_q > 0 && n_k > 0 && (!q || !w || !k || !scores)) return fail(ECHO_EINVAL, "echo_index_scores_prefill: NULL pointer");
  return launch_score_prefill(q, w, k, n_q, n_k, q_pos0, scores, ld, S(stream));
}
