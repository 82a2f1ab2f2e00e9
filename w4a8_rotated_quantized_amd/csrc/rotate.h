// ConvRot rotation helpers shared by the rotate+quantize kernels and the
// weight dequantize/merge kernel (gfx950).
//
// The regular Hadamard matrix of order n = 4^d (16, 64, 256, 1024) as the
// "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4" page (intro) and the
// "Qwen-Image-Edit-2511-W4A8-ConvRot" card (group-size notes) use it, in the
// lane layout and butterfly order described at the top of rq.hip.
#pragma once

#include "common.h"

namespace cr {

// f(d) of the digit-sign vector: -1 for a zero base-4 digit.
CR_DEV float fdig(int d) { return d == 0 ? -1.f : 1.f; }
constexpr float fdig_c(int d) { return d == 0 ? -1.f : 1.f; }
// per-register part of D: digits (b1 b0) and (b3 b2) of e = b0 + 2b1 + 4b2 + 8b3
constexpr bool dreg_neg(int e) { return fdig_c(e & 3) * fdig_c(e >> 2) < 0; }

struct LaneRot {
  int gL;          // element bits b4..b7 of this lane, packed (b4 + 2b5 + 4b6 + 8b7)
  float c[4];      // cross-lane butterfly multipliers for bits b4..b7
  float tau;       // final per-lane sign
};

// Rotation sizes n = 4^d: 16, 64 and 256 live inside one 256-element chunk
// (a 16-lane segment); 1024 is four consecutive chunks held by the same lanes.
template <int NR>
struct RotSize {
  static_assert(NR == 16 || NR == 64 || NR == 256 || NR == 1024, "rotation group of 16, 64, 256 or 1024");
  static constexpr int digits = NR == 16 ? 2 : NR == 64 ? 3 : NR == 256 ? 4 : 5;
  static constexpr int lane_bits = NR == 16 ? 0 : NR == 64 ? 2 : 4;     // element bits b4.. inside the group
  static constexpr float inv_sqrt = NR == 16 ? 0.25f : NR == 64 ? 0.125f : NR == 256 ? 0.0625f : 0.03125f;
};

template <int NR>
CR_DEV LaneRot lane_rot(int L) {
  LaneRot r;
  const int b4 = (L ^ (L >> 2)) & 1;
  const int b5 = ((L >> 1) ^ (L >> 2)) & 1;
  const int b6 = (L >> 2) & 1;
  const int b7 = (L >> 3) & 1;
  r.gL = b4 | (b5 << 1) | (b6 << 2) | (b7 << 3);
  const int bits[4] = {b4, b5, b6, b7};
  // stage s flips element bit b_{4+s}; its digit is (b5 b4) for s < 2, (b7 b6) for s >= 2.
  // With sigma the per-lane sign (true = sigma * stored): the lane holding
  // bit 0 keeps sigma and adds sigma_L*sigma_P*partner; the lane holding bit 1
  // computes partner - self = -sigma_L*(self - sigma_L*sigma_P*partner) and
  // flips sigma. sigma_L*sigma_P only depends on the digit-sign factors.
  for (int s = 0; s < 4; ++s) {
    int lo = (s < 2) ? 0 : 2;
    int d = bits[lo] + 2 * bits[lo + 1];
    int dp = d ^ (1 << (s - lo));
    float sign = bits[s] ? -1.f : 1.f;
    r.c[s] = sign * fdig(d) * fdig(dp);
  }
  // overall sign (-1)^d times the flips of the lane stages inside the group
  constexpr int lane_mask = (1 << RotSize<NR>::lane_bits) - 1;
  r.tau = ((RotSize<NR>::digits + __popc(r.gL & lane_mask)) & 1) ? -1.f : 1.f;
  return r;
}

// In-register butterflies over register bit RB (1, 2, 4, 8).
template <int RB>
CR_DEV void bfly_reg(float (&v)[16]) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (e & RB) continue;
    float a = v[e], b = v[e | RB];
    v[e] = __fadd_rn(a, b);
    v[e | RB] = __fsub_rn(a, b);
  }
}

// Cross-lane butterfly stage: v[e] += c * v[e] of the partner lane, one
// v_fmac_f32_dpp per register (the compiler does not fuse a DPP move into
// fmac, so the stage is written out; the leading s_nop covers the
// VALU-write -> DPP-read hazard of the instructions before the block).
#define CR_FD(i, CTRL) "v_fmac_f32_dpp %" #i ", %" #i ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
#define CR_BFLY_LANE(NAME, CTRL)                                                                  \
  CR_DEV void NAME(float(&v)[16], float c) {                                                      \
    asm volatile("s_nop 1\n\t" CR_FD(0, CTRL) CR_FD(1, CTRL) CR_FD(2, CTRL) CR_FD(3, CTRL)          \
                 CR_FD(4, CTRL) CR_FD(5, CTRL) CR_FD(6, CTRL) CR_FD(7, CTRL) CR_FD(8, CTRL)           \
                 CR_FD(9, CTRL) CR_FD(10, CTRL) CR_FD(11, CTRL) CR_FD(12, CTRL) CR_FD(13, CTRL)       \
                 CR_FD(14, CTRL) CR_FD(15, CTRL)                                                   \
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),        \
                   "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),      \
                   "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])                             \
                 : "v"(c));                                                                        \
  }
CR_BFLY_LANE(bfly_lane_x1, "quad_perm:[1,0,3,2]")
CR_BFLY_LANE(bfly_lane_x2, "quad_perm:[2,3,0,1]")
CR_BFLY_LANE(bfly_lane_x7, "row_half_mirror")
CR_BFLY_LANE(bfly_lane_x8, "row_ror:8")

// The butterfly stages of an NR-point group that lie inside one 256-element
// chunk (all of them for NR <= 256), on values that already carry the
// per-register signs of D (dreg_neg, and the chunk sign for NR = 1024).
template <int NR>
CR_DEV void butterflies(float (&v)[16], const LaneRot& lr) {
  bfly_reg<1>(v);                      // h = 1   (b0)
  bfly_reg<2>(v);                      // h = 2   (b1)
  bfly_reg<4>(v);                      // h = 4   (b2)
  bfly_reg<8>(v);                      // h = 8   (b3)
  if constexpr (NR >= 64) {
    bfly_lane_x1(v, lr.c[0]);          // h = 16  (b4): partner lane ^ 1
    bfly_lane_x2(v, lr.c[1]);          // h = 32  (b5): partner lane ^ 2
  }
  if constexpr (NR >= 256) {
    bfly_lane_x7(v, lr.c[2]);          // h = 64  (b6): partner lane ^ 7
    bfly_lane_x8(v, lr.c[3]);          // h = 128 (b7): partner lane ^ 8
  }
}

// bf16 words (2 x 16 bytes = elements 0..15 of this lane) -> the same stages.
// NEG negates the chunk first (NR = 1024: the digit (b9 b8) of D for chunk 0
// of each group).
// SM: multiply by the per-channel factors sm[0..15] of these elements first
// (one float32 rounding per element, before any butterfly).
template <int NR, bool NEG = false, bool SM = false>
CR_DEV void rotate_group(const u32x4 (&w)[2], const LaneRot& lr, float (&v)[16], const float* sm = nullptr) {
  v4f m[4];
  if constexpr (SM) {
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = reinterpret_cast<const v4f*>(sm)[q];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 8 * h + 2 * j;
      float lo = bf16_lo(w[h][j]), hi = bf16_hi(w[h][j]);
      if constexpr (SM) {
        lo = __fmul_rn(lo, m[e >> 2][e & 3]);
        hi = __fmul_rn(hi, m[(e + 1) >> 2][(e + 1) & 3]);
      }
      v[e] = (dreg_neg(e) != NEG) ? -lo : lo;
      v[e + 1] = (dreg_neg(e + 1) != NEG) ? -hi : hi;
    }
  butterflies<NR>(v, lr);
}

// NR = 1024: the last two stages (h = 256, 512: bits b8, b9 = the chunk index
// within the group) between the NC chunks a lane holds, NC a multiple of 4
// (chunks 4q .. 4q+3 form one group). The chunks share the lane's sign, so
// plain float32 sums of the stored values are the butterflies.
template <int NC>
CR_DEV void bfly_chunks(float (&v)[NC][16]) {
  static_assert(NC % 4 == 0, "whole 1024-groups");
#pragma unroll
  for (int q = 0; q < NC; q += 4)
#pragma unroll
    for (int hb = 1; hb <= 2; hb <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j & hb) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float a = v[q + j][e], b = v[q + j + hb][e];
          v[q + j][e] = __fadd_rn(a, b);
          v[q + j + hb][e] = __fsub_rn(a, b);
        }
      }
}

// sign of chunk c of a 1024-group in D (its digit b9 b8 = c % 4)
CR_DEV constexpr bool chunk_neg(int c) { return (c & 3) == 0; }

}  // namespace cr
