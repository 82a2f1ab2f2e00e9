// W4A8 GEMM (gfx950): per-token int8 activations x asymmetric uint4 weights
// with a float16 scale and a uint4 zero point per 16 input channels.
//
// "Qwen-Image-Edit-2511-W4A8-ConvRot" card, build table and file layout
// (asym_w4a8_int8, group_size 16, convrot_groupsize 256, 8-bit activations).
//
// Every 16-deep group is one v_mfma_i32_32x32x16_i8, so each MFMA yields the
// exact per-group partial P[m, n, g] = sum_k qa (qw - z). The weight nibbles
// are widened to the signed bytes (q - z) in registers; the float16 group
// scale is applied by one convert + one fused multiply-add per (m, n, g),
// which makes this format VALU-bound by construction. Operand roles: A = the
// activations (32 tokens), B = the weights (32 channels), so every lane owns
// one output channel and needs one scale per group.
#include "common.h"
#include "kernels.h"

namespace cr {

typedef long v1l;

// 8 weight nibbles of one lane (byte i = q[i] | q[4+i] << 4) -> bytes q - z.
CR_DEV long widen_asym(uint32_t x, uint32_t zz) {
  uint32_t lo = (((x & 0x0F0F0F0Fu) | 0x80808080u) - zz) ^ 0x80808080u;
  uint32_t hi = ((((x >> 4) & 0x0F0F0F0Fu) | 0x80808080u) - zz) ^ 0x80808080u;
  return (long)(((uint64_t)hi << 32) | lo);
}

template <int OUT>
__global__ __launch_bounds__(256) void gemm_w4a8_kernel(GemmParams p) {
  constexpr int BM = 128, BN = 128;
  constexpr bool GRP = OUT != CR_OUT_I32_RAW;
  constexpr int X_ST = 2 * 4 * (BM / 32) * 512;   // [kt][kg][mb][64 x 8 B]
  constexpr int W_ST = 2 * 4096;                  // [kt][kg][nb][64 x 4 B]
  constexpr int S_ST = 2 * 4 * 128 * 2;           // fp16 scales [kt][kg][128]
  constexpr int Z_ST = 2 * 4 * 128;               // zero points  [kt][kg][128]
  constexpr int STAGE = X_ST + W_ST + S_ST + Z_ST;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int ntm = (int)((p.M + BM - 1) / BM);
  const int ntn = (int)(p.N / BN);
  const int ntiles = ntm * ntn;
  int t = blockIdx.x;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  constexpr int GM = 8;
  const int band = t / (GM * ntn);
  const int rows_in_band = min(GM, ntm - band * GM);
  const int within = t - band * GM * ntn;
  const int tn = within / rows_in_band;
  const int tm = band * GM + within % rows_in_band;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t K = p.K;
  const int nkb = (int)(K / 128);
  const int64_t wtile0 = (n0 >> 7) * (K / 64);      // first tile of this channel block

  u32x4 rx[4], rwt[2], rsz;
  auto gload = [&](int kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int pc = tid + j * 256;            // 1024 pieces: row = pc >> 3, group-of-16 = pc & 7
      int row = pc >> 3, part = pc & 7;
      int64_t m = imin64(m0 + row, p.M - 1);
      rx[j] = *reinterpret_cast<const u32x4*>(p.a + m * K + (int64_t)kb * 128 + part * 16);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
      rwt[j] = *reinterpret_cast<const u32x4*>(p.w + (wtile0 + kb * 2) * 4096 + (tid + j * 256) * 16);
    if (tid < 128) {
      rsz = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(p.w_scales16) +
                                            (wtile0 + kb * 2) * 1024 + tid * 16);
    } else if (tid < 192) {
      rsz = *reinterpret_cast<const u32x4*>(p.w_zeros + (wtile0 + kb * 2) * 512 + (tid - 128) * 16);
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* Xs = smem + buf * STAGE;
    uint8_t* Wsm = Xs + X_ST;
    uint8_t* Ssm = Wsm + W_ST;
    uint8_t* Zsm = Ssm + S_ST;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int pc = tid + j * 256;
      int row = pc >> 3, part = pc & 7;
      int kt = part >> 2, kg = part & 3;
      uint8_t* base = Xs + ((kt * 4 + kg) * (BM / 32) + (row >> 5)) * 512;
      *reinterpret_cast<u32x2*>(base + (row & 31) * 8) = u32x2{rx[j][0], rx[j][1]};
      *reinterpret_cast<u32x2*>(base + ((row & 31) + 32) * 8) = u32x2{rx[j][2], rx[j][3]};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(Wsm + (tid + j * 256) * 16) = rwt[j];
    if (tid < 128) *reinterpret_cast<u32x4*>(Ssm + tid * 16) = rsz;
    else if (tid < 192) *reinterpret_cast<u32x4*>(Zsm + (tid - 128) * 16) = rsz;
  };

  v16i acc[2][2];
  float y[2][2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[a][b][r] = 0;
        y[a][b][r] = 0.f;
      }
    }

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
    const uint8_t* Xs = smem + buf * STAGE;
    const uint8_t* Wsm = Xs + X_ST;
    const _Float16* Ssm = reinterpret_cast<const _Float16*>(Wsm + W_ST);
    const uint8_t* Zsm = Wsm + W_ST + S_ST;
#pragma unroll 1
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll 1
      for (int kg = 0; kg < 4; ++kg) {
        long xa[2], wb[2];
        float sc[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          xa[i] = *reinterpret_cast<const long*>(Xs + ((kt * 4 + kg) * (BM / 32) + wm * 2 + i) * 512 + l * 8);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int nl = (wn * 2 + j) * 32 + (l & 31);
          uint32_t z = Zsm[(kt * 4 + kg) * 128 + nl];
          sc[j] = (float)Ssm[(kt * 4 + kg) * 128 + nl];
          uint32_t x = *reinterpret_cast<const uint32_t*>(Wsm + kt * 4096 + kg * 1024 + (wn * 2 + j) * 256 + l * 4);
          wb[j] = widen_asym(x, z * 0x01010101u);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if constexpr (GRP) {
              v16i pp = __builtin_amdgcn_mfma_i32_32x32x16_i8(xa[i], wb[j], v16i{}, 0, 0, 0);
#pragma unroll
              for (int r = 0; r < 16; ++r) y[i][j][r] = __builtin_fmaf((float)pp[r], sc[j], y[i][j][r]);
            } else {
              acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x16_i8(xa[i], wb[j], acc[i][j], 0, 0, 0);
            }
          }
      }
    }
    if (kb + 1 < nkb) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane owns channel n = l%32 of each 32x32 block and tokens
  // 8*(r/4) + 4*(l/32) + r%4
  const float sa_t = (p.a_gran == CR_GRAN_TENSOR) ? p.a_scales[0] : 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + (wn * 2 + j) * 32 + (l & 31);
    float b = 0.f;
    if (GRP && p.bias) b = __uint_as_float((uint32_t)p.bias[n] << 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + (wm * 2 + i) * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        if (m >= p.M) continue;
        if constexpr (OUT == CR_OUT_I32_RAW) {
          reinterpret_cast<int32_t*>(p.out)[m * p.ldc + n] = acc[i][j][r];
        } else {
          float sa = (p.a_gran == CR_GRAN_TENSOR) ? sa_t : p.a_scales[m];
          float v = y[i][j][r] * sa + b;
          if constexpr (OUT == CR_OUT_F32) reinterpret_cast<float*>(p.out)[m * p.ldc + n] = v;
          else reinterpret_cast<uint16_t*>(p.out)[m * p.ldc + n] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Float-output kernel: the weights are dequantized in registers to
// fp16(s * (q - z)) and the int8 activation codes converted exactly to fp16,
// and v_mfma_f32_32x32x16_f16 accumulates over the whole of K in fp32. This
// removes the per-group float epilogue (two VALU operations per output per
// 16-deep group), which on gfx950 costs far more than the matrix work. The
// one extra rounding (of s * (q - z) to fp16, relative 2^-11) stays far below
// the bf16 output rounding. The exact int32 output keeps the kernel above.
//
// Operand layouts are those of the int8 kernel (the fp16 32x32x16 operand
// of a lane is the same 8 k-values of one row / column as the int8 one):
// activations [group][32-row block][64 lanes x 8 B] in LDS, filled by
// 4-byte global_load_lds pieces from the natural int8 rows; weights, fp16
// scales and zero points by 16-byte pieces in their tile-packed order.
// fp16 conversions: 0x6400 | u is the fp16 value 1024 + u for u < 1024, so
// v_perm_b32 against 0x64646464 builds two of them per instruction and one
// packed fp16 subtraction removes the bias exactly.
// ---------------------------------------------------------------------------
typedef _Float16 v8h_ __attribute__((ext_vector_type(8)));
typedef _Float16 v2h_ __attribute__((ext_vector_type(2)));
typedef float v16f_ __attribute__((ext_vector_type(16)));
typedef const void __attribute__((address_space(1)))* gas_ptr_w8;
typedef void __attribute__((address_space(3)))* las_ptr_w8;

CR_DEV uint32_t h2_add(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h_, a) + __builtin_bit_cast(v2h_, b));
}
CR_DEV uint32_t h2_sub_mul(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_bit_cast(uint32_t, (__builtin_bit_cast(v2h_, a) - __builtin_bit_cast(v2h_, b)) *
                                          __builtin_bit_cast(v2h_, c));
}

template <int OUT>
__global__ __launch_bounds__(256, 2) void gemm_w4a8_f16_kernel(GemmParams p) {
  constexpr int BM = 128, BN = 128, NG = 8;                 // 8 groups of 16 = 128 k per stage
  constexpr int A_ST = BM * 16 * NG;                        // [g][mb][64][8 B]   16 KB
  constexpr int W_ST = 2 * 4096;                            // [kt][kg][nb][64][4 B]  8 KB
  constexpr int S_ST = 2 * 4 * 128 * 2;                     // fp16 scales [kt][kg][128]  2 KB
  constexpr int Z_ST = 2 * 4 * 128;                         // zero points [kt][kg][128]  1 KB
  constexpr int STAGE = A_ST + W_ST + S_ST + Z_ST;
  constexpr int LA = A_ST / 256 / 4;                        // 4-byte wave-loads of A per wave (16)
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem_w8[];
  uint8_t* smem = smem_w8;

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int ntm = (int)((p.M + BM - 1) / BM);
  const int ntn = (int)(p.N / BN);
  const int ntiles = ntm * ntn;
  int t = (int)blockIdx.x;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  constexpr int GM = 8;
  const int band = t / (GM * ntn);
  const int rows_in_band = min(GM, ntm - band * GM);
  const int within = t - band * GM * ntn;
  const int tn = within / rows_in_band;
  const int tm = band * GM + within % rows_in_band;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t K = p.K;
  const int64_t KT = K / 64;
  const int nkb = (int)(K / 128);
  const int64_t wtile0 = (n0 >> 7) * KT;

  // A wave-load wl = wave + 4 j covers fragment f = wl >> 1 (group f >> 2,
  // 32-row block f & 3), fragment lanes 32 (wl & 1) + l / 2, dword l & 1:
  // row 32 mb + l / 2, k-bytes 16 g + 8 (wl & 1) + 4 (l & 1) of the stage.
  int64_t rowoff[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) rowoff[mb] = imin64(m0 + 32 * mb + (l >> 1), p.M - 1) * K;
  const int kbyte = 8 * (wave & 1) + 4 * (l & 1);

  auto issue = [&](int kb) {
    uint8_t* st = smem + (kb & 1) * STAGE;
    const uint8_t* ga = p.a + (int64_t)kb * 128 + kbyte;
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int f = (wave >> 1) + 2 * j;                    // fragment index, compile-time up to wave
      __builtin_amdgcn_global_load_lds((gas_ptr_w8)(ga + rowoff[f & 3] + 16 * (f >> 2)),
                                       (las_ptr_w8)(st + (wave + 4 * j) * 256), 4, 0, 0);
    }
    const uint8_t* gw = p.w + (wtile0 + kb * 2) * 4096;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds((gas_ptr_w8)(gw + (wave + 4 * j) * 1024 + l * 16),
                                       (las_ptr_w8)(st + A_ST + (wave + 4 * j) * 1024), 16, 0, 0);
    if (wave < 2)
      __builtin_amdgcn_global_load_lds(
          (gas_ptr_w8)(reinterpret_cast<const uint8_t*>(p.w_scales16) + (wtile0 + kb * 2) * 1024 + wave * 1024 +
                       l * 16),
          (las_ptr_w8)(st + A_ST + W_ST + wave * 1024), 16, 0, 0);
    else if (wave == 2)
      __builtin_amdgcn_global_load_lds((gas_ptr_w8)(p.w_zeros + (wtile0 + kb * 2) * 512 + l * 16),
                                       (las_ptr_w8)(st + A_ST + W_ST + S_ST), 16, 0, 0);
  };

  v16f_ acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  issue(0);
  for (int kb = 0; kb < nkb; ++kb) {
    __builtin_amdgcn_s_waitcnt(0x0070);                     // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (kb + 1 < nkb) issue(kb + 1);
    const uint8_t* As = smem + (kb & 1) * STAGE;
    const uint8_t* Wsm = As + A_ST;
    const uint16_t* Ssm = reinterpret_cast<const uint16_t*>(Wsm + W_ST);
    const uint8_t* Zsm = Wsm + W_ST + S_ST;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int kt = g >> 2, kg = g & 3;
      uint32_t af[2][4], wf[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(As + ((g * 4 + wm * 2 + i) * 64 + l) * 8);
        const uint32_t x0 = x[0] ^ 0x80808080u, x1 = x[1] ^ 0x80808080u;   // a + 128 as unsigned bytes
        const uint32_t nb = 0xE480E480u;                                       // fp16 -1152 in both halves
        af[i][0] = h2_add(__builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u), nb);
        af[i][1] = h2_add(__builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u), nb);
        af[i][2] = h2_add(__builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u), nb);
        af[i][3] = h2_add(__builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u), nb);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nb = wn * 2 + j;
        const int c = (kt * 4 + kg) * 128 + nb * 32 + (l & 31);
        const uint32_t zz = __builtin_amdgcn_perm(0x64646464u, (uint32_t)Zsm[c], 0x04000400u);   // 1024 + z
        const uint32_t sv = Ssm[c];
        const uint32_t ss = sv | (sv << 16);
        const uint32_t x = *reinterpret_cast<const uint32_t*>(Wsm + ((kt * 4 + kg) * 4 + nb) * 256 + l * 4);
        const uint32_t xl = x & 0x0F0F0F0Fu, xh = (x >> 4) & 0x0F0F0F0Fu;      // q[0..3], q[4..7]
        wf[j][0] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, xl, 0x04010400u), zz, ss);
        wf[j][1] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, xl, 0x04030402u), zz, ss);
        wf[j][2] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, xh, 0x04010400u), zz, ss);
        wf[j][3] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, xh, 0x04030402u), zz, ss);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(v8h_, u32x4{af[i][0], af[i][1], af[i][2], af[i][3]}),
              __builtin_bit_cast(v8h_, u32x4{wf[j][0], wf[j][1], wf[j][2], wf[j][3]}), acc[i][j], 0, 0, 0);
    }
  }

  // lane owns channel n = l % 32 of each 32 x 32 block and tokens 8 (r / 4) + 4 (l / 32) + r % 4
  const float sa_t = (p.a_gran == CR_GRAN_TENSOR) ? p.a_scales[0] : 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + (wn * 2 + j) * 32 + (l & 31);
    const float b = p.bias ? __uint_as_float((uint32_t)p.bias[n] << 16) : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + (wm * 2 + i) * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        if (m >= p.M) continue;
        const float sa = (p.a_gran == CR_GRAN_TENSOR) ? sa_t : p.a_scales[m];
        const float v = acc[i][j][r] * sa + b;
        if constexpr (OUT == CR_OUT_F32) reinterpret_cast<float*>(p.out)[m * p.ldc + n] = v;
        else reinterpret_cast<uint16_t*>(p.out)[m * p.ldc + n] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  }
}

template <int OUT>
static hipError_t launch_w4a8_f16(const GemmParams& p, hipStream_t s) {
  constexpr int lds = 2 * (128 * 16 * 8 + 2 * 4096 + 2 * 4 * 128 * 2 + 2 * 4 * 128);
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)gemm_w4a8_f16_kernel<OUT>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = ((p.M + 127) / 128) * (p.N / 128);
  hipLaunchKernelGGL((gemm_w4a8_f16_kernel<OUT>), dim3((unsigned)tiles), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_w4a8(const GemmParams& p, hipStream_t s) {
  const int64_t tiles = ((p.M + 127) / 128) * (p.N / 128);
  switch (p.out_type) {
    case CR_OUT_BF16:
      return launch_w4a8_f16<CR_OUT_BF16>(p, s);
    case CR_OUT_F32:
      return launch_w4a8_f16<CR_OUT_F32>(p, s);
    default:
      hipLaunchKernelGGL((gemm_w4a8_kernel<CR_OUT_I32_RAW>), dim3((unsigned)tiles), dim3(256), 0, s, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace cr
