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

// Partial score of token l%16 over the 16 heads this lane group holds:
// sum over hb, v of w * ReLU(q . k).  The full score is the sum over the four lane groups.
ECHO_DEV float score_tile_partial(const QOperand &o, const v8i &bv) {
  float acc = 0.f;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    v4f c = {0.f, 0.f, 0.f, 0.f};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.qa[hb], bv, c, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc = fmaf(o.wr[hb][v], fmaxf(c[v], 0.f), acc);
  }
  return acc;
}

// Sum of the four lane groups' partials (lanes l, l^16, l^32, l^48): every lane of the wave
// then holds the score of token l%16.
ECHO_DEV float reduce_groups(float p) {
  p += __shfl_xor(p, 16, 64);
  p += __shfl_xor(p, 32, 64);
  return p;
}

}  // namespace echo
