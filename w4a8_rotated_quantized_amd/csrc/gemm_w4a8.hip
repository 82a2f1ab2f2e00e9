// W4A8 GEMM (gfx950): per-token int8 activations x asymmetric uint4 weights
// with a float16 scale and a uint4 zero point per 16 input channels.
//
// "Qwen-Image-Edit-2511-W4A8-ConvRot" card, build table and file layout
// (asym_w4a8_int8, group_size 16, convrot_groupsize 256, 8-bit activations).
//
// Two kernels:
//  - the exact int32 output (CR_OUT_I32_RAW): every 16-deep group is one
//    v_mfma_i32_32x32x16_i8 over the activation codes and the weight nibbles
//    widened to the signed bytes q - z, accumulated in int32;
//  - bf16 / float32 outputs: the fp16 matrix-core kernel further below.
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

__global__ __launch_bounds__(256) void gemm_w4a8_raw_kernel(GemmParams p) {
  constexpr int BM = 128, BN = 128;
  constexpr int X_ST = 2 * 4 * (BM / 32) * 512;   // [kt][kg][mb][64 x 8 B]
  constexpr int W_ST = 2 * 4096;                  // [kt][kg][nb][64 x 4 B]
  constexpr int Z_ST = 2 * 4 * 128;               // zero points  [kt][kg][128]
  constexpr int STAGE = X_ST + W_ST + Z_ST;
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
    if (tid < 64) rsz = *reinterpret_cast<const u32x4*>(p.w_zeros + (wtile0 + kb * 2) * 512 + tid * 16);
  };
  auto lstore = [&](int buf) {
    uint8_t* Xs = smem + buf * STAGE;
    uint8_t* Wsm = Xs + X_ST;
    uint8_t* Zsm = Wsm + W_ST;
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
    if (tid < 64) *reinterpret_cast<u32x4*>(Zsm + tid * 16) = rsz;
  };

  v16i acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
    const uint8_t* Xs = smem + buf * STAGE;
    const uint8_t* Wsm = Xs + X_ST;
    const uint8_t* Zsm = Wsm + W_ST;
#pragma unroll 1
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll 1
      for (int kg = 0; kg < 4; ++kg) {
        long xa[2], wb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          xa[i] = *reinterpret_cast<const long*>(Xs + ((kt * 4 + kg) * (BM / 32) + wm * 2 + i) * 512 + l * 8);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int nl = (wn * 2 + j) * 32 + (l & 31);
          uint32_t z = Zsm[(kt * 4 + kg) * 128 + nl];
          uint32_t x = *reinterpret_cast<const uint32_t*>(Wsm + kt * 4096 + kg * 1024 + (wn * 2 + j) * 256 + l * 4);
          wb[j] = widen_asym(x, z * 0x01010101u);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x16_i8(xa[i], wb[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kb + 1 < nkb) lstore(buf ^ 1);
    __syncthreads();
  }

  // lane owns channel n = l % 32 of each 32 x 32 block and tokens 8 (r / 4) + 4 (l / 32) + r % 4
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + (wn * 2 + j) * 32 + (l & 31);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + (wm * 2 + i) * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        if (m < p.M) reinterpret_cast<int32_t*>(p.out)[m * p.ldc + n] = acc[i][j][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Float-output kernel on fp16 matrix cores (bf16 / float32 outputs).
//
// Applying a float group scale after every 16-deep int8 product costs two
// VALU operations per output and group, far more than the matrix work. This
// kernel instead dequantizes each weight once per block to fp16(s * (q - z))
// in registers and lets v_mfma_f32_32x32x16_f16 accumulate over all of K in
// float32. The only rounding added to the exact sum is that of s * (q - z)
// to fp16 (relative 2^-11); the exact int32 output keeps the kernel above.
//
// Activation codes become fp16 without arithmetic: a ^ 0x80 is the unsigned
// byte u = a + 128, and 0x64 placed above it is the fp16 value 1024 + u =
// 1152 + a (v_perm_b32 builds two per instruction). The matrix cores thus
// compute sum_k (1152 + a_k) w_k, and the epilogue subtracts 1152 * w_sum[n]
// with w_sum[n] = sum_k fp16(s * (q - z)) (exact, from w4_pack_weights).
// Weights: 0x64 above a nibble is 1024 + q; one packed fp16 subtraction of
// 1024 + z is exact and one packed multiplication by s rounds once.
//
// Block: 256 x 128 outputs, 4 waves of 128 x 64 (4 x 2 blocks of 32 x 32).
// Each 64-deep k-tile is one pipeline stage (3 in flight, loaded straight
// into LDS by 16-byte global_load_lds): activations [row][4 x 16 B] with the
// 16-byte slots XOR-swizzled per row, weights / scales / zero points in their
// tile-packed order. A lane reads 16 activation bytes (one 16-deep group) at
// once and feeds the two 8-deep halves to two MFMAs; in the first, lanes
// 0-31 carry group 2p and lanes 32-63 group 2p + 1 (k 0..7 of each), in the
// second k 8..15 of the same groups, and the weight fragments follow the same
// assignment (the order of a dot product's terms is free). The weights are
// operand A, so a lane ends with one token and four adjacent channels: one
// activation scale per lane and 8-byte bf16 stores.
// ---------------------------------------------------------------------------
typedef _Float16 v8h_ __attribute__((ext_vector_type(8)));
typedef _Float16 v2h_ __attribute__((ext_vector_type(2)));
typedef const void __attribute__((address_space(1)))* gas_ptr_w8;
typedef void __attribute__((address_space(3)))* las_ptr_w8;

typedef float v2f_ __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

CR_DEV uint32_t h2_sub_mul(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_bit_cast(uint32_t, (__builtin_bit_cast(v2h_, a) - __builtin_bit_cast(v2h_, b)) *
                                          __builtin_bit_cast(v2h_, c));
}

template <int N>
CR_DEV void w8_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16-byte slot of group g in row r of an activation stage (4 groups of 16
// bytes per row): XOR-swizzled so that 8 or 16 consecutive rows read at one
// group hit distinct LDS banks.
CR_DEV int w8_slot(int r, int g) { return g ^ (((r >> 1) ^ (r >> 3)) & 3); }

template <int OUT>
__global__ __launch_bounds__(256, 2) void gemm_w4a8_h_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 128, NS = 3;
  constexpr int A_ST = BM * 64;                 // [row][4 slots x 16 B]
  constexpr int W_ST = 4096;                    // [kg][nb][64 x 4 B]
  constexpr int S_ST = 1024;                    // fp16 scales [kg][128]
  constexpr int Z_ST = 1024;                    // zero points [kg][128] (+512 B duplicate)
  constexpr int STAGE = A_ST + W_ST + S_ST + Z_ST;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem_w8h[];
  uint8_t* smem = smem_w8h;

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int ntm = (int)((p.M + BM - 1) / BM);
  const int ntn = (int)(p.N / BN);
  const int ntiles = ntm * ntn;
  int t = (int)blockIdx.x;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  constexpr int GM = 4;
  const int band = t / (GM * ntn);
  const int rows_in_band = min(GM, ntm - band * GM);
  const int within = t - band * GM * ntn;
  const int tn = within / rows_in_band;
  const int tm = band * GM + within % rows_in_band;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t K = p.K;
  const int64_t KT = K / 64;
  const int nst = (int)KT;
  const int64_t wt0 = (int64_t)tn * KT;          // first packed k-tile of this channel block

  // activation wave-load j of this wave: rows 16 (wave + 4 j) + l / 4, slot l % 4
  int64_t aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * (wave + 4 * j) + (l >> 2);
    aoff[j] = imin64(m0 + r, p.M - 1) * K + 16 * w8_slot(r, l & 3);
  }

  auto issue = [&](int s) {
    uint8_t* st = smem + (s % NS) * STAGE;
    const uint8_t* ga = p.a + (int64_t)s * 64;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds((gas_ptr_w8)(ga + aoff[j]), (las_ptr_w8)(st + (wave + 4 * j) * 1024), 16, 0, 0);
    const int64_t tile = wt0 + s;
    __builtin_amdgcn_global_load_lds((gas_ptr_w8)(p.w + tile * 4096 + wave * 1024 + l * 16),
                                     (las_ptr_w8)(st + A_ST + wave * 1024), 16, 0, 0);
    if (wave == 0)
      __builtin_amdgcn_global_load_lds(
          (gas_ptr_w8)(reinterpret_cast<const uint8_t*>(p.w_scales16) + tile * 1024 + l * 16),
          (las_ptr_w8)(st + A_ST + W_ST), 16, 0, 0);
    else if (wave == 1)
      __builtin_amdgcn_global_load_lds((gas_ptr_w8)(p.w_zeros + tile * 512 + (l & 31) * 16),
                                       (las_ptr_w8)(st + A_ST + W_ST + S_ST), 16, 0, 0);
  };

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment addresses inside a stage
  const int lr = l & 31, h = l >> 5;
  const int fl = ((lr >> 1) ^ (lr >> 3)) & 3;
  int abase[2], wbase[2], sbase[2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    const int g = 2 * pp + h;
    abase[pp] = (wm * 128 + lr) * 64 + 16 * (g ^ fl);
    wbase[pp] = A_ST + (g * 4 + wn * 2) * 256 + lr * 4;
    sbase[pp] = g * 128 + wn * 64 + lr;
  }

  issue(0);
  if (nst > 1) issue(1);
  for (int s = 0; s < nst; ++s) {
    if (s + 1 < nst) {
      if (wave < 2) w8_wait_vm<6>();
      else w8_wait_vm<5>();
    } else {
      w8_wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (s + 2 < nst) issue(s + 2);
    const uint8_t* st = smem + (s % NS) * STAGE;
    const uint16_t* Ssm = reinterpret_cast<const uint16_t*>(st + A_ST + W_ST);
    const uint8_t* Zsm = st + A_ST + W_ST + S_ST;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      u32x4 ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = *reinterpret_cast<const u32x4*>(st + abase[pp] + i * 2048);
      uint32_t wa[2][4], wb[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t x0 = *reinterpret_cast<const uint32_t*>(st + wbase[pp] + j * 256);
        const uint32_t x1 = *reinterpret_cast<const uint32_t*>(st + wbase[pp] + j * 256 + 128);
        const uint32_t z = Zsm[sbase[pp] + j * 32];
        const uint32_t sv = Ssm[sbase[pp] + j * 32];
        const uint32_t zz = z * 0x00010001u + 0x64006400u;      // fp16 pair (1024 + z, 1024 + z)
        const uint32_t ss = sv | (sv << 16);
        const uint32_t x0l = x0 & 0x0F0F0F0Fu, x0h = (x0 >> 4) & 0x0F0F0F0Fu;
        const uint32_t x1l = x1 & 0x0F0F0F0Fu, x1h = (x1 >> 4) & 0x0F0F0F0Fu;
        wa[j][0] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, x0l, 0x04010400u), zz, ss);
        wa[j][1] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, x0l, 0x04030402u), zz, ss);
        wa[j][2] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, x0h, 0x04010400u), zz, ss);
        wa[j][3] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, x0h, 0x04030402u), zz, ss);
        wb[j][0] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, x1l, 0x04010400u), zz, ss);
        wb[j][1] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, x1l, 0x04030402u), zz, ss);
        wb[j][2] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, x1h, 0x04010400u), zz, ss);
        wb[j][3] = h2_sub_mul(__builtin_amdgcn_perm(0x64646464u, x1h, 0x04030402u), zz, ss);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t u[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) u[q] = ar[i][q] ^ 0x80808080u;   // a + 128 as unsigned bytes
        // fp16 1152 + a: 0x64 above byte u is the fp16 value 1024 + u
        const v8h_ fa = __builtin_bit_cast(v8h_, u32x4{__builtin_amdgcn_perm(0x64646464u, u[0], 0x04010400u),
                                                       __builtin_amdgcn_perm(0x64646464u, u[0], 0x04030402u),
                                                       __builtin_amdgcn_perm(0x64646464u, u[1], 0x04010400u),
                                                       __builtin_amdgcn_perm(0x64646464u, u[1], 0x04030402u)});
        const v8h_ fb = __builtin_bit_cast(v8h_, u32x4{__builtin_amdgcn_perm(0x64646464u, u[2], 0x04010400u),
                                                       __builtin_amdgcn_perm(0x64646464u, u[2], 0x04030402u),
                                                       __builtin_amdgcn_perm(0x64646464u, u[3], 0x04010400u),
                                                       __builtin_amdgcn_perm(0x64646464u, u[3], 0x04030402u)});
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(v8h_, u32x4{wa[j][0], wa[j][1], wa[j][2], wa[j][3]}), fa, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(v8h_, u32x4{wb[j][0], wb[j][1], wb[j][2], wb[j][3]}), fb, acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // D = W . A^T per 32 x 32 block: lane owns token m = l % 32 and channels
  // 8 (r / 4) + 4 (l / 32) + r % 4. The activations entered as 1152 + a, so
  // 1152 * w_sum[n] comes off first. Phase 1 turns every accumulator into its
  // output value in place, phase 2 stores them: all epilogue loads (scales,
  // column sums, bias, low-rank operands) are issued before the first store,
  // so no load waits on a store. A missing bias reads w_sum's memory and is
  // zeroed.
  float sa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = imin64(m0 + wm * 128 + i * 32 + lr, p.M - 1);
    sa[i] = p.a_scales[p.a_gran == CR_GRAN_TENSOR ? 0 : m];
  }
  v4f cw[2][4];
  u32x2 bw[2][4];
  const bool has_bias = p.bias != nullptr;
  const uint16_t* bsrc = has_bias ? p.bias : reinterpret_cast<const uint16_t*>(p.w_sum);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = n0 + (wn * 2 + j) * 32 + 8 * q + 4 * h;
      cw[j][q] = *reinterpret_cast<const v4f*>(p.w_sum + n);
      bw[j][q] = *reinterpret_cast<const u32x2*>(bsrc + n);
    }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f c = cw[j][q] * 1152.f;
      const u32x2 bb = has_bias ? bw[j][q] : u32x2{0u, 0u};
      const v4f b = v4f{bf16_lo(bb[0]), bf16_hi(bb[0]), bf16_lo(bb[1]), bf16_hi(bb[1])};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][j][4 * q + t] = (acc[i][j][4 * q + t] - c[t]) * sa[i] + b[t];
    }
  }
  if (p.lora_act) {
    // low-rank branch: y[m, n] += sum_r la[m, r] L1[n, r], one
    // v_mfma_f32_32x32x16_bf16 per 16 ranks and 32 x 32 block, whose result
    // layout is that of the main accumulators
    const uint16_t* la = reinterpret_cast<const uint16_t*>(p.lora_act);
    const int R = p.R;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint16_t* lu = p.lora_up + (n0 + (wn * 2 + j) * 32 + lr) * R + 8 * h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t* lam = la + imin64(m0 + wm * 128 + i * 32 + lr, p.M - 1) * R + 8 * h;
        for (int r0 = 0; r0 < R; r0 += 16)        // accumulates onto the finished outputs
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(lu + r0)),
              __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(lam + r0)), acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);          // one block's operands live at a time
      }
    }
  }
  if constexpr (OUT == CR_OUT_BF16) {
    // bf16 (v_cvt_pk_bf16_f32, half to even) through LDS in two halves of 64
    // token rows per wave, so that every store writes whole 128-byte output
    // rows; the fragment layout would scatter 8-byte pieces over 32 rows per
    // store instruction
    constexpr int RS = 144;                          // LDS row stride of a half tile, 16-byte aligned
    static_assert(4 * 64 * RS <= NS * STAGE, "half tiles fit the stage buffers");
    __syncthreads();                                 // every wave is done with the stage buffers
    uint8_t* tile = smem + wave * (64 * RS);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v16f& a = acc[2 * hh + ii][j];
            const v2bf lo = __builtin_convertvector((v2f_){a[4 * q], a[4 * q + 1]}, v2bf);
            const v2bf hi = __builtin_convertvector((v2f_){a[4 * q + 2], a[4 * q + 3]}, v2bf);
            *reinterpret_cast<u32x2*>(tile + (ii * 32 + lr) * RS + (j * 32 + 8 * q + 4 * h) * 2) =
                u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          }
      // this wave's half tile is complete (LDS keeps a wave's order, so the
      // next half's writes also land after these reads)
      __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0)
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) {
        const int r = (l >> 3) + 8 * qq;
        const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * RS + (l & 7) * 16);
        const int64_t m = m0 + wm * 128 + hh * 64 + r;
        if (m < p.M)
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldc + n0 + wn * 64 + (l & 7) * 8) = v;
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = n0 + (wn * 2 + j) * 32 + 8 * q + 4 * h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 128 + i * 32 + lr;
        if (m >= p.M) continue;
        const float y[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if constexpr (OUT == CR_OUT_F32) {
          *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.out) + m * p.ldc + n) = v4f{y[0], y[1], y[2], y[3]};
        } else {
          u32x2 o;
          o[0] = f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16);
          o[1] = f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16);
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldc + n) = o;
        }
      }
    }
  }
}

template <int OUT>
static hipError_t launch_w4a8_h(const GemmParams& p, hipStream_t s) {
  constexpr int lds = 3 * (256 * 64 + 4096 + 1024 + 1024);
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)gemm_w4a8_h_kernel<OUT>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = ((p.M + 255) / 256) * (p.N / 128);
  hipLaunchKernelGGL((gemm_w4a8_h_kernel<OUT>), dim3((unsigned)tiles), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_w4a8(const GemmParams& p, hipStream_t s) {
  switch (p.out_type) {
    case CR_OUT_BF16:
      return launch_w4a8_h<CR_OUT_BF16>(p, s);
    case CR_OUT_F32:
      return launch_w4a8_h<CR_OUT_F32>(p, s);
    default: {
      const int64_t tiles = ((p.M + 127) / 128) * (p.N / 128);
      hipLaunchKernelGGL(gemm_w4a8_raw_kernel, dim3((unsigned)tiles), dim3(256), 0, s, p);
      return hipGetLastError();
    }
  }
}

}  // namespace cr
