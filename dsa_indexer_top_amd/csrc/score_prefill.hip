// Prefill (causal) lightning-indexer scores on gfx950 (ECHO review page §2 score definition;
// §3.4: the indexer is quadratic in the context, every query against every earlier key).
//
// Query rows t in [0, n_q) sit at absolute positions q_pos0 + t and see keys [0, lim_t),
// lim_t = min(n_k, q_pos0 + t + 1); the diagonal is included.
//
// Work split: two consecutive queries per wave (their 64 x 128 FP8 q and 64 weights stay in
// VGPRs in MFMA layout, and each B operand read from LDS serves both), 24 queries per
// 768-thread workgroup (3 waves per SIMD).  The workgroup streams the keys [0, lim of its last
// query) through three LDS buffers of 192-key stages (24 KB each, filled with coalesced 16-byte
// loads into the swizzled layout the decode kernel uses; one barrier per stage): while stage n
// is scored, stage n+1 is already in LDS and stage n+2 in registers.  Workgroups are launched
// heaviest (latest queries) first.
//
// Per 64-key group a wave runs 32 units (four 16-key tiles x four 16-head blocks x two
// queries), each one v_mfma_f32_16x16x128_f8f6f4 and its epilogue.  The kernel is bound by the ratio of epilogue
// VALU work to MFMA work: every (head, key) product needs its ReLU and its weighted add, while
// one MFMA covers 16 heads x 16 keys x 128 bytes in the time of about 8 wave-wide VALU
// instructions.  So:
//   * the epilogue is two VALU instructions per element: the ReLU is an integer max on the
//     float's bits (a negative float, -0 included, has its sign bit set and so is below 0 as an
//     int32; this avoids the NaN canonicalisation an IEEE float max costs), then one FMA;
//   * the MFMA of unit u+PF_AHEAD is issued before the epilogue of unit u, across tile, group
//     and stage boundaries, so the matrix core multiplies while the VALU reduces;
//   * the four tiles' per-lane-group partial sums are combined with one butterfly of gfx950
//     lane swaps (3 swaps + 3 adds per 64 keys), after which the 64 lanes hold 64 consecutive
//     scores of the group.
// The group that crosses a wave's causal limit is computed whole and its writes are masked.
#include "internal.hpp"
#include "score_tile.cuh"

namespace echo {

constexpr int PF_THREADS = 768;
constexpr int PF_QPW = 2;                               // queries per wave
constexpr int PF_QPB = PF_THREADS / 64 * PF_QPW;        // 24 queries per workgroup
constexpr int PF_STAGE = 192;                           // keys per LDS stage (3 groups of 64)
constexpr int PF_UNITS = PF_STAGE * D / 16;             // 1536 x 16 B
constexpr int PF_LOADS = PF_UNITS / PF_THREADS;         // 2 per thread
constexpr int PF_BUFS = 3;                              // stage buffers in LDS (72 KB)
constexpr int PF_AHEAD = 2;                             // MFMAs in flight ahead of the epilogue
static_assert(PF_STAGE % 64 == 0 && PF_UNITS % PF_THREADS == 0, "stage shape");


ECHO_DEV int pswz(int tok, int seg) { return tok * 128 + ((seg ^ ((tok >> 1) & 7)) << 4); }


ECHO_DEV v4f unit_mfma(const v8i &qa, const v8i &bv) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, bv, z, 0, 0, 0, 0, 0, 0);
}
// acc + sum over the lane's 4 rows of one head block: w * ReLU(c)
ECHO_DEV float unit_epilogue(const float (&wr)[4], const v4f &c, float acc) {
#pragma unroll
  for (int v = 0; v < 4; ++v) acc = fmaf(wr[v], relu_bits(c[v]), acc);
  return acc;
}
ECHO_DEV v8i tile_b(const uint8_t *sb, int tt, int g) {
  const int4 b0 = *reinterpret_cast<const int4 *>(sb + pswz(tt, 2 * g));
  const int4 b1 = *reinterpret_cast<const int4 *>(sb + pswz(tt, 2 * g + 1));
  return v8i{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
}


// One 64-key group of a wave: 32 units (4 tiles x 4 head blocks x the wave's 2 queries), one
// MFMA and 8 VALU instructions each, the two queries alternating so that each B operand read
// from LDS serves two MFMAs.  The MFMA of unit u+PF_AHEAD is issued before the epilogue of unit
// u, so the matrix core multiplies while the VALU reduces and an epilogue never waits on the
// MFMA just issued; c[] carries the accumulator sets in flight (c[0] the oldest) and bt the B
// operand of the current tile, from group to group and from stage to stage.  gb is the group's
// 64 keys in LDS, nb the next group's (possibly in the next stage's buffer).  On entry c[]
// holds units 0 .. PF_AHEAD-1 of this group, on return those of the next one.  v[q] returns
// query q's score of key 16*tsel + l%16 of the group; each query's sum is taken in the same
// order as with one query per wave.
//
// The order is pinned with empty asm statements, which the compiler keeps in program order
// and which emit nothing: each MFMA takes its B operand from one, hands its result to the
// next, and the epilogue reads its accumulators from that one and hands its sum to the next
// unit's first.  Without them the compiler issued most of a group's MFMAs back to back before
// any epilogue, holding as many accumulator sets.  The distance from an MFMA to the first read
// of its result stays PF_AHEAD units (at least 17 instructions), beyond the result's latency.
ECHO_DEV void prefill_group(const QOperand (&qo)[PF_QPW], const uint8_t *gb, const uint8_t *nb,
                            int j, int g, v8i &bt, v4f (&c)[PF_AHEAD], float (&v)[PF_QPW]) {
  static_assert(PF_AHEAD == PF_QPW, "unit u+PF_AHEAD is the same query's next head block");
  float p[PF_QPW][4];
  float acc[PF_QPW] = {};              // the running sums of the previous units
#pragma unroll
  for (int tile = 0; tile < 4; ++tile) {
    v8i bn = tile < 3 ? tile_b(gb, (tile + 1) * 16 + j, g) : tile_b(nb, j, g);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
      for (int qi = 0; qi < PF_QPW; ++qi) {
        // unit u+PF_AHEAD is head block hb+1 of the same query, in this tile or the next one
        const bool this_tile = hb + 1 < 4;
        v8i bb = this_tile ? bt : bn;
        asm volatile("" : "+v"(bb), "+v"(acc[qi]));
        if (hb == 0) {                  // this query's sum of the previous tile is complete
          if (tile > 0) p[qi][tile - 1] = acc[qi];
          acc[qi] = 0.f;
        }
        v4f cn = unit_mfma(qo[qi].qa[(hb + 1) & 3], bb);
        if (this_tile) bt = bb; else bn = bb;
        v4f co = c[0];
        asm volatile("" : "+v"(cn), "+v"(co));
        acc[qi] = unit_epilogue(qo[qi].wr[hb], co, acc[qi]);
#pragma unroll
        for (int i = 0; i + 1 < PF_AHEAD; ++i) c[i] = c[i + 1];
        c[PF_AHEAD - 1] = cn;
      }
    }
    bt = bn;
  }
  // lanes of groups {g, g^2} exchange so each keeps two tiles summed over both groups, then
  // groups {g, g^1} exchange so each keeps one tile summed over all four
#pragma unroll
  for (int qi = 0; qi < PF_QPW; ++qi) {
    p[qi][3] = acc[qi];
    const float a = swap_sum32(p[qi][0], p[qi][2]);
    const float b = swap_sum32(p[qi][1], p[qi][3]);
    v[qi] = swap_sum16(a, b);
  }
}

__global__ __launch_bounds__(PF_THREADS) void score_prefill_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ w, const uint8_t *__restrict__ k,
    int32_t n_q, int32_t n_k, int32_t q_pos0, float *__restrict__ scores, int64_t ld) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[PF_BUFS][PF_STAGE * D];
  const int nblk = (n_q + PF_QPB - 1) / PF_QPB;
  const int blk = nblk - 1 - static_cast<int>(blockIdx.x);     // heaviest first
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int j = l & 15, g = l >> 4;
  // the wave's queries t0 and t0 + 1 (a query past n_q scores with a copy of the operand of
  // query min(t0, n_q - 1) and writes nothing)
  const int32_t t0 = blk * PF_QPB + PF_QPW * __builtin_amdgcn_readfirstlane(wv);
  int32_t lim[PF_QPW];
#pragma unroll
  for (int qi = 0; qi < PF_QPW; ++qi) lim[qi] = t0 + qi < n_q ? min(n_k, q_pos0 + t0 + qi + 1) : 0;
  const int32_t t_last = min(n_q - 1, blk * PF_QPB + PF_QPB - 1);
  const int32_t wg_lim = min(n_k, q_pos0 + t_last + 1);
  if (wg_lim <= 0) return;

  // Which tile of a 64-key group this lane's score belongs to after the butterfly.  A 32-lane
  // swap pairs lane group g with g^2 and a 16-lane swap pairs g with g^1; the half (row) of
  // the wave that keeps its own first operand depends on the swap direction, which one probe
  // swap of known values reads (the sums themselves do not depend on it).
  const v2u p32 = __builtin_amdgcn_permlane32_swap(0u, 1u, false, false);
  const v2u p16 = __builtin_amdgcn_permlane16_swap(0u, 1u, false, false);
  const int flip32 = __builtin_amdgcn_readfirstlane(static_cast<int>(p32[0]));
  const int flip16 = __builtin_amdgcn_readfirstlane(static_cast<int>(p16[0]));
  const int tsel = ((((g >> 1) ^ flip32) & 1) << 1) | ((g ^ flip16) & 1);

  QOperand qo[PF_QPW];
  float *__restrict__ srow[PF_QPW];
#pragma unroll
  for (int qi = 0; qi < PF_QPW; ++qi) {
    const int32_t tq = t0 + qi < n_q ? t0 + qi : min(t0, n_q - 1);
    load_q_operand(q, w, tq, qo[qi]);
    srow[qi] = scores + static_cast<int64_t>(tq) * ld;
  }

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

  auto stash = [&](uint8_t *sb) {
#pragma unroll
    for (int m = 0; m < PF_LOADS; ++m) {
      const int e = tid + m * PF_THREADS;
      *reinterpret_cast<int4 *>(sb + pswz(e >> 3, e & 7)) = pre[m];
    }
  };

  // Three stage buffers: while stage n is scored, stage n+1 is already published (the
  // look-ahead of a wave's last group of stage n reads it) and stage n+2 is in registers.
  fetch(0);
  stash(lds[0]);
  __syncthreads();
  if (PF_STAGE < wg_lim) fetch(PF_STAGE);

  int32_t lim_w = 0;                              // the furthest limit of the wave's queries
#pragma unroll
  for (int qi = 0; qi < PF_QPW; ++qi) lim_w = max(lim_w, lim[qi]);
  const int ngw = (lim_w + 63) >> 6;              // 64-key groups this wave scores
  v8i bt = {0, 0, 0, 0, 0, 0, 0, 0};
  v4f c[PF_AHEAD];
#pragma unroll
  for (int i = 0; i < PF_AHEAD; ++i) c[i] = v4f{0.f, 0.f, 0.f, 0.f};
  if (ngw > 0) {
    bt = tile_b(lds[0], j, g);
#pragma unroll
    for (int i = 0; i < PF_AHEAD; ++i) c[i] = unit_mfma(qo[i].qa[0], bt);
  }
  int cur = 0;
  for (int32_t c0 = 0; c0 < wg_lim; c0 += PF_STAGE) {
    const int nxt = cur == PF_BUFS - 1 ? 0 : cur + 1;
    // lds[nxt] was last read while stage c0 - 2*PF_STAGE was scored, before the last barrier
    if (c0 + PF_STAGE < wg_lim) stash(lds[nxt]);
    __syncthreads();
    if (c0 + 2 * PF_STAGE < wg_lim) fetch(c0 + 2 * PF_STAGE);
    const int G0 = c0 >> 6, G1 = min(ngw, G0 + PF_STAGE / 64);   // wave-uniform causal skip
    for (int G = G0; G < G1; ++G) {
      const int gi = G - G0;
      const uint8_t *gb = lds[cur] + gi * 64 * D;
      const uint8_t *nb = gi == PF_STAGE / 64 - 1 ? lds[nxt] : gb + 64 * D;
      float v[PF_QPW];
      prefill_group(qo, gb, nb, j, g, bt, c, v);
      const int32_t s = G * 64 + tsel * 16 + j;      // the group crossing lim is masked here
#pragma unroll
      for (int qi = 0; qi < PF_QPW; ++qi)
        if (s < lim[qi]) srow[qi][s] = v[qi];
    }
    cur = nxt;
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
