// Fused GEMM epilogue shared by the integer-matrix-core GEMMs: for one
// 16x16 output block whose lane holds token m and output channels n..n+3.
// "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Fused LoRA-Up Epilogue
// (low-rank up-projection on bf16 matrix cores inside the INT4 GEMM
// epilogue) and Kernel Engineering (unsigned shifted activations).
#pragma once

#include "common.h"
#include "kernels.h"

namespace cr {

// Fused epilogue for one 16x16 block: lane holds token m and channels n..n+3.
// ---------------------------------------------------------------------------
template <int OUT>
CR_DEV void store4(const GemmParams& p, int64_t m, int64_t n, const float (&y)[4], const int (&raw)[4]) {
  if (m >= p.M) return;
  if constexpr (OUT == CR_OUT_I32_RAW) {
    *reinterpret_cast<v4i*>(reinterpret_cast<int32_t*>(p.out) + m * p.ldc + n) = v4i{raw[0], raw[1], raw[2], raw[3]};
  } else if constexpr (OUT == CR_OUT_F32) {
    *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.out) + m * p.ldc + n) = v4f{y[0], y[1], y[2], y[3]};
  } else {
    u32x2 o;
    o[0] = f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16);
    o[1] = f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldc + n) = o;
  }
}

// y += lora_act[m, :] . L1[n..n+3, :] for the 16x16 block (tokens mb.., channels nb..),
// L1 in the tiled layout [N/128][R][128]
CR_DEV void lora_up_block(const GemmParams& p, int64_t mb, int64_t nb, int l, float (&y)[4]) {
  const int64_t mrow = (mb + (l & 15) < p.M) ? mb + (l & 15) : p.M - 1;
  const int64_t nrow = nb + (l & 15);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const int R = p.R;                       // 32 or 64
  if (!p.lora_f32) {
    for (int r0 = 0; r0 < R; r0 += 32) {
      const uint16_t* la = reinterpret_cast<const uint16_t*>(p.lora_act) + mrow * R + r0 + (l >> 4) * 8;
      v8bf a = lora_up8(p.lora_up, R, nrow, r0 + (l >> 4) * 8);
      v8bf b = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(la));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
  } else {
    const float* la = reinterpret_cast<const float*>(p.lora_act) + mrow * R;
    for (int r0 = 0; r0 < R; r0 += 4) {
      float a = lora_up1(p.lora_up, R, nrow, r0 + (l >> 4));
      float b = la[r0 + (l >> 4)];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] += acc[i];
}

// Everything after the float value s_a*s_w*acc (or the group sum) is known:
// shift correction, low-rank branch and bias, in place.
template <int OUT>
CR_DEV void finish_values(const GemmParams& p, int64_t n, int64_t mb, int l, float (&y)[4]) {
  if constexpr (OUT != CR_OUT_I32_RAW) {
    if (p.act == ACT_U4) {
      const v4f ws = *reinterpret_cast<const v4f*>(p.w_sum + n);
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = __builtin_fmaf(-p.a_shift, ws[i], y[i]);
    }
    if (p.lora_act) lora_up_block(p, mb, n - (l >> 4) * 4, l, y);
    if (p.bias) {
      u32x2 b = *reinterpret_cast<const u32x2*>(p.bias + n);
      y[0] += bf16_lo(b[0]);
      y[1] += bf16_hi(b[0]);
      y[2] += bf16_lo(b[1]);
      y[3] += bf16_hi(b[1]);
    }
  }
}

template <int OUT>
CR_DEV void finish_block(const GemmParams& p, int64_t m, int64_t n, int64_t mb, int l, float (&y)[4],
                         const int (&raw)[4]) {
  finish_values<OUT>(p, n, mb, l, y);
  store4<OUT>(p, m, n, y, raw);
}

}  // namespace cr
