// One 64-head x 16-token tile of lightning-indexer scores on gfx950 (ECHO review page §2).
//
// v_mfma_f32_16x16x128_f8f6f4: A = q of 16 heads (16 x 128 FP8), B = k of 16 tokens
// (128 x 16 FP8), C = 16 x 16 fp32.  Lane l supplies A row l%16 and B column l%16; its lane
// group g = l/16 supplies the K slice.  A and B use the same lane-group -> K mapping, so any
// assignment of the 128 bytes of a row to (group, byte) works as long as q and k share it:
// group g carries bytes [32g, 32g+32).  The result C[4g+v][l%16] lands in lane l, element v.
#pragma once

#include "common.hpp"

namespace echo {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct QOperand {
  v8i qa[4];       // head block hb: heads hb*16 + l%16, bytes [32g, 32g+32)
  float wr[4][4];  // weights of the output rows this lane holds: heads hb*16 + 4g + v
};

// Loads request r's q (64 x 128 FP8) and w (64 fp32) in MFMA layout for the calling lane.
ECHO_DEV void load_q_operand(const uint8_t *__restrict__ q, const float *__restrict__ w,
                             int64_t r, QOperand &o) {
  const int l = lane_id(), j = l & 15, g = l >> 4;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int4 *p = reinterpret_cast<const int4 *>(q + ((r * H + hb * 16 + j) * D + 32 * g));
    const int4 a0 = p[0], a1 = p[1];
    o.qa[hb] = v8i{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int v = 0; v < 4; ++v) o.wr[hb][v] = w[r * H + hb * 16 + 4 * g + v];
  }
}

// ReLU(x) as an integer max on the bits: -0 and every negative float map to +0.
ECHO_DEV float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Partial score of token l%16 over the 16 heads this lane group holds:
// sum over hb, v of w * ReLU(q . k).  The full score is the sum over the four lane groups.
ECHO_DEV float score_tile_partial(const QOperand &o, const v8i &bv) {
  float acc = 0.f;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    v4f c = {0.f, 0.f, 0.f, 0.f};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.qa[hb], bv, c, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc = fmaf(o.wr[hb][v], relu_bits(c[v]), acc);
  }
  return acc;
}

// Sum of the four lane groups' partials (lanes l, l^16, l^32, l^48): every lane of the wave
// then holds the score of token l%16.  Groups {g, g^2} are added first, then the two pairs:
// the same association as butterfly4 below, so every kernel that scores with either gets the
// same float32 value for a token.
ECHO_DEV float reduce_groups(float p) {
  p += __shfl_xor(p, 32, 64);
  p += __shfl_xor(p, 16, 64);
  return p;
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// The same partial as score_tile_partial with the four head-block MFMAs issued before the
// epilogue (independent accumulators, so the matrix core runs them back to back).
ECHO_DEV float score_tile_partial_mf(const QOperand &o, const v8i &bv) {
  v4f c[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
    c[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.qa[hb], bv, v4f{0.f, 0.f, 0.f, 0.f},
                                                            0, 0, 0, 0, 0, 0);
  float acc = 0.f;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc = fmaf(o.wr[hb][v], relu_bits(c[hb][v]), acc);
  return acc;
}

// Lane swaps (gfx950 v_permlane32_swap / v_permlane16_swap) that sum a pair of values across
// the two halves of the wave, or across neighbouring 16-lane rows.
ECHO_DEV float swap_sum32(float a, float b) {
  const v2u s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
ECHO_DEV float swap_sum16(float a, float b) {
  const v2u s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Four tiles' partials p[0..3] (tile = 16 consecutive keys, lane group g = l/16 holding the
// partial over its heads) summed over the lane groups by a butterfly of three swaps: lane
// groups {g, g^2} exchange so each keeps two tiles summed over both, then {g, g^1} so each keeps
// one tile summed over all four.  The lane then holds the score of key 16*tile_sel + l%16 of
// the 64, tile_sel from group_tile_sel().
ECHO_DEV float butterfly4(const float (&p)[4]) {
  const float a = swap_sum32(p[0], p[2]);
  const float b = swap_sum32(p[1], p[3]);
  return swap_sum16(a, b);
}
// Which tile the butterfly leaves in this lane.  The half (row) of the wave that keeps its own
// first operand depends on the swap direction, which one probe swap of known values reads; the
// sums themselves do not depend on it.  Every lane of the wave must be active.
ECHO_DEV int group_tile_sel() {
  const int g = lane_id() >> 4;
  const v2u p32 = __builtin_amdgcn_permlane32_swap(0u, 1u, false, false);
  const v2u p16 = __builtin_amdgcn_permlane16_swap(0u, 1u, false, false);
  const int flip32 = __builtin_amdgcn_readfirstlane(static_cast<int>(p32[0]));
  const int flip16 = __builtin_amdgcn_readfirstlane(static_cast<int>(p16[0]));
  return ((((g >> 1) ^ flip32) & 1) << 1) | ((g ^ flip16) & 1);
}

}  // namespace echo
