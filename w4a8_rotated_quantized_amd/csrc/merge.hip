// Weight dequantization back to the original basis, with an optional
// low-rank delta: the device side of merging a LoRA into quantized weights
// (gfx950). "Qwen-Image-Edit-2511-W4A8-ConvRot" card, passage on LoRA merge
// versus bypass: a LoRA loaded onto a quantized weight dequantizes it, adds
// the delta and quantizes the result again. The requantization is the
// library's own convrot_rotate_quantize + w4_pack_weights on this output.
//
// Per weight row n and element k (all float32, then one bf16 rounding):
//   r[k]   = fl(s * q)            (symmetric; asymmetric: s16 * (q - z), exact)
//   w[k]   = (H r)[k] / sqrt(n_rot) per rotation group (the rotation is its
//            own inverse up to the 1/sqrt(n) factor; same butterflies and
//            order as the forward rotation; no rotation: w = r)
//   d[k]   = sum_{j < R} up[n, j] * down[j, k], accumulated in float32 in j
//            order (bf16 x bf16 products are exact)
//   out[k] = bf16_rne(fl(w[k] + d[k])), a zero as +0
#include "common.h"
#include "kernels.h"
#include "rotate.h"

namespace cr {

enum { MK_S4 = 0, MK_S8 = 1, MK_ASYM = 2 };

// the 16 dequantized values of one lane: row n, elements k0 .. k0 + 15
template <int KIND>
CR_DEV void dequant16(const MergeParams& p, int64_t n, int64_t k0, float (&v)[16]) {
  const int64_t K = p.K;
  if constexpr (KIND == MK_ASYM) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(p.codes + n * (K / 2) + k0 / 2);
    const float s = (float)reinterpret_cast<const _Float16*>(p.scales)[n * (K / 16) + k0 / 16];
    const int zb = p.zeros[n * (K / 32) + k0 / 32];
    const int z = ((k0 / 16) & 1) ? (zb >> 4) : (zb & 0xF);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int q = (x[e >> 3] >> (4 * (e & 7))) & 0xF;
      v[e] = s * (float)(q - z);                  // exact: 11-bit scale times a 5-bit integer
    }
  } else {
    float s;
    const float* sc = reinterpret_cast<const float*>(p.scales);
    if (p.gran == CR_GRAN_TENSOR) s = sc[0];
    else if (p.gran == CR_GRAN_ROW) s = sc[n];
    else s = sc[n * (K / 64) + k0 / 64];
    if constexpr (KIND == MK_S8) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(p.codes + n * K + k0);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int q = (int)(int8_t)((x[e >> 2] >> (8 * (e & 3))) & 0xFF);
        v[e] = __fmul_rn(s, (float)q);
      }
    } else {
      const u32x2 x = *reinterpret_cast<const u32x2*>(p.codes + n * (K / 2) + k0 / 2);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int q = (int)(((x[e >> 3] >> (4 * (e & 7))) & 0xF) ^ 8) - 8;
        v[e] = __fmul_rn(s, (float)q);
      }
    }
  }
}

// Segment (16 lanes) = one row and GPS consecutive 256-element chunks (four
// for the 1024 rotation); the lane holds elements 16 gL .. 16 gL + 15 of each.
template <int NR, int KIND>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int GPS = NR == 1024 ? 4 : 1;
  constexpr int LNR = NR == 0 ? 256 : NR;          // lane layout of the rotation (any for none)
  const int tid = threadIdx.x;
  const int seg = tid >> 4;
  const LaneRot lr = lane_rot<LNR>(tid & 15);
  const int64_t per_row = (p.K / 256) / GPS;
  const int64_t total = p.N * per_row;
  const int64_t item = (int64_t)blockIdx.x * 16 + seg;
  const bool ok = item < total;
  const int64_t it = ok ? item : total - 1;        // past the end: recompute the last item, store nothing
  const int64_t n = it / per_row;
  const int64_t c0 = (it % per_row) * GPS;

  float v[GPS][16];
#pragma unroll
  for (int g = 0; g < GPS; ++g) {
    dequant16<KIND>(p, n, (c0 + g) * 256 + 16 * lr.gL, v[g]);
    if constexpr (NR != 0) {
      const bool cneg = NR == 1024 && chunk_neg(g);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (dreg_neg(e) != cneg) v[g][e] = -v[g][e];
      butterflies<NR>(v[g], lr);
    }
  }
  if constexpr (NR == 1024) bfly_chunks<GPS>(v);

#pragma unroll
  for (int g = 0; g < GPS; ++g) {
    const int64_t k0 = (c0 + g) * 256 + 16 * lr.gL;
    float w[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      w[e] = v[g][e];
      if constexpr (NR != 0) {
        const bool neg = (lr.tau < 0.f) != (dreg_neg(e) != (NR == 1024 && chunk_neg(g)));
        w[e] = (neg ? -w[e] : w[e]) * RotSize<NR>::inv_sqrt;   // sign and power of two: exact
      }
    }
    if (p.up) {
      float d[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) d[e] = 0.f;
      const uint16_t* up = p.up + n * p.R;
      for (int j = 0; j < p.R; ++j) {
        const float u = bf16_lo(up[j]);
        const u32x4* dp = reinterpret_cast<const u32x4*>(p.down + (int64_t)j * p.K + k0);
        const u32x4 d0 = dp[0], d1 = dp[1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w0 = d0[e >> 1], w1 = d1[e >> 1];
          d[e] = __builtin_fmaf(u, (e & 1) ? bf16_hi(w0) : bf16_lo(w0), d[e]);
          d[8 + e] = __builtin_fmaf(u, (e & 1) ? bf16_hi(w1) : bf16_lo(w1), d[8 + e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) w[e] = __fadd_rn(w[e], d[e]);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) w[e] = __fadd_rn(w[e], 0.f);   // a zero comes out as +0
    if (ok) {
      u32x4 o[2];
#pragma unroll
      for (int e = 0; e < 16; e += 2)
        o[e >> 3][(e & 7) >> 1] = f32_to_bf16_bits(w[e]) | (f32_to_bf16_bits(w[e + 1]) << 16);
      u32x4* dst = reinterpret_cast<u32x4*>(p.out + n * p.K + k0);
      dst[0] = o[0];
      dst[1] = o[1];
    }
  }
}

template <int NR>
static hipError_t launch_merge_nr(const MergeParams& p, hipStream_t s) {
  constexpr int GPS = NR == 1024 ? 4 : 1;
  const int64_t items = p.N * ((p.K / 256) / GPS);
  const dim3 grid((unsigned)((items + 15) / 16));
  if (p.qtype == CR_Q_ASYM_UINT4) {
    if constexpr (NR == 0 || NR == 256) hipLaunchKernelGGL((merge_kernel<NR, MK_ASYM>), grid, dim3(256), 0, s, p);
  } else if (p.qtype == CR_Q_SYM_INT8) {
    hipLaunchKernelGGL((merge_kernel<NR, MK_S8>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((merge_kernel<NR, MK_S4>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  switch (p.rot_group) {
    case 0: return launch_merge_nr<0>(p, s);
    case 16: return launch_merge_nr<16>(p, s);
    case 64: return launch_merge_nr<64>(p, s);
    case 1024: return launch_merge_nr<1024>(p, s);
    default: return launch_merge_nr<256>(p, s);
  }
}

}  // namespace cr
