// Shared device helpers for the gfx950 kernels of the ConvRot low-bit linear.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CR_DEV __device__ __forceinline__

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Magic constant 1.5 * 2^23: adding it to a float32 of magnitude < 2^22
// rounds to an integer with the current (half-to-even) rounding mode, and
// the low bits of the sum's bit pattern are that integer in two's complement.
#define CR_MAGIC_RNE 12582912.0f

CR_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
CR_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16 bits, round half to even (finite inputs).
CR_DEV uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

CR_DEV int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// The low-rank up-projection L1 in its tiled layout [N/128][R][128] (for each
// block of 128 output channels, rank-major runs of 128 channels: "Qwen-Image-
// Edit-2511 INT4 (ComfyUI Optimized)", Tile-Packed Weight Format):
// rank entries r .. r+7 of channel n as one bf16 operand fragment (eight
// 2-byte reads 256 bytes apart; the 32 or 16 channels of a fragment row read
// one contiguous run per entry), and one entry as a float.
CR_DEV v8bf lora_up8(const uint16_t* up, int R, int64_t n, int r) {
  const uint16_t* q = up + ((n >> 7) * R + r) * 128 + (n & 127);
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)q[(2 * i) * 128] | ((uint32_t)q[(2 * i + 1) * 128] << 16);
  return __builtin_bit_cast(v8bf, w);
}
CR_DEV float lora_up1(const uint16_t* up, int R, int64_t n, int r) {
  return __uint_as_float((uint32_t)up[((n >> 7) * R + r) * 128 + (n & 127)] << 16);
}

CR_DEV float amax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Correctly rounded float32 quotient: the double quotient of two float32
// values rounded once more to float32 is correctly rounded (53 >= 2*24+2).
CR_DEV float div_rn(float a, float b) { return (float)((double)a / (double)b); }

// DPP lane permutations inside a 16-lane row (gfx9 encodings).
#define DPP_QUAD_1032 0xB1   // quad_perm [1,0,3,2]: lane ^ 1
#define DPP_QUAD_2301 0x4E   // quad_perm [2,3,0,1]: lane ^ 2
#define DPP_HALF_MIRROR 0x141  // lane ^ 7 inside each 8-lane half row
#define DPP_ROW_ROR8 0x128     // lane ^ 8 inside a 16-lane row

template <int CTRL>
CR_DEV float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
CR_DEV int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// max over the 16 lanes of a DPP row (all four XOR directions).
CR_DEV float row16_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_ROR8>(v));
  return v;
}
CR_DEV float row16_min(float v) {
  v = fminf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fminf(v, dpp_f<DPP_QUAD_2301>(v));
  v = fminf(v, dpp_f<DPP_HALF_MIRROR>(v));
  v = fminf(v, dpp_f<DPP_ROW_ROR8>(v));
  return v;
}
CR_DEV float quad_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_2301>(v));
  return v;
}
CR_DEV float quad_min(float v) {
  v = fminf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fminf(v, dpp_f<DPP_QUAD_2301>(v));
  return v;
}

// max over a full 64-lane wave.
CR_DEV float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// ---------------------------------------------------------------------------
// int4 -> int8 widening for the int8 matrix cores. Both operands of one MFMA
// are widened by the same function, so the k order inside a lane's 16 bytes
// (even elements of bytes 0..3, odd elements, then bytes 4..7) matches.
// ---------------------------------------------------------------------------

// signed nibbles -> bytes holding 16*q (exact: 16*q in [-128, 112]).
CR_DEV v4i widen_s4x16(u32x2 x) {
  v4i r;
  r[0] = (int)((x[0] << 4) & 0xF0F0F0F0u);
  r[1] = (int)(x[0] & 0xF0F0F0F0u);
  r[2] = (int)((x[1] << 4) & 0xF0F0F0F0u);
  r[3] = (int)(x[1] & 0xF0F0F0F0u);
  return r;
}
// unsigned nibbles -> bytes holding u in [0, 15].
CR_DEV v4i widen_u4(u32x2 x) {
  v4i r;
  r[0] = (int)(x[0] & 0x0F0F0F0Fu);
  r[1] = (int)((x[0] >> 4) & 0x0F0F0F0Fu);
  r[2] = (int)(x[1] & 0x0F0F0F0Fu);
  r[3] = (int)((x[1] >> 4) & 0x0F0F0F0Fu);
  return r;
}
