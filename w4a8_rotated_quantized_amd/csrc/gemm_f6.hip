// W4A4 GEMM on the fp6 matrix cores (gfx950): int4 codes carried as fp6
// E2M3 values, exact products and exact float32 sums.
//
// "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4" page, Measurements: a fused
// INT4 matrix multiply with a rank-one (s_a x s_w) rescale.
// "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Key Technical
// Optimizations (tile-packed weights, fused LoRA-up) and Kernel Engineering
// (multi-stage global->shared pipeline).
//
// Why fp6. A symmetric int4 code lies in [-7, 7], and every integer of that
// range is an E2M3 value (sign, 2 exponent bits with bias 1, 3 mantissa
// bits: 0, 1, 2, 3 = 2 x 1.5, 4, 5 = 4 x 1.25, 6, 7 = 4 x 1.75). A product of
// two codes is an integer of magnitude <= 49 and the matrix cores add such
// products in float32, which stays exact while every partial sum is below
// 2^24 in magnitude: K * 49 < 2^24 for K <= 342392. So
// v_mfma_f32_32x32x64_f8f6f4 on E2M3 operands yields exactly the integer
// sum_k qa * qw, at twice the rate of the int8 instruction and with no
// widening work in the loop.
//
// Operand fragment (one 32 x 64 block of codes, 1536 bytes): lane l (row
// l % 32, k-half l / 32) holds 32 consecutive codes as six-bit fields,
// field i at bits 6i..6i+5 of its 24 bytes; bytes 0..15 sit at l * 16,
// bytes 16..23 at 1024 + l * 8. Activations and weights share the layout
// [rows/32][K/64][1536 B], so both operands of a block stage are runs of
// 3 KB (two 64-deep k-tiles of one 32-row block).
//
// Operand roles: MFMA A = weights (32 output channels), B = activations (32
// tokens). Lane l of the 32x32 result holds token l % 32 and, in register
// r, channel 8 (r / 4) + 4 (l / 32) + r % 4: four runs of four consecutive
// channels, each one 8-byte bf16 store.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace cr {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef const void __attribute__((address_space(1)))* f6_gptr;
typedef void __attribute__((address_space(3)))* f6_lptr;

constexpr int F6_FRAG = 1536;

// E2M3 on both operands (format code 2), no block scale
CR_DEV v16f mfma_f6_32(v8i w, v8i a, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, a, c, 2, 2, 0, 0, 0, 0);
}
CR_DEV v4f mfma_f6_16(v8i w, v8i a, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, c, 2, 2, 0, 0, 0, 0);
}

// one lane's 24 bytes of a fragment (two reads; the last two dwords unused)
CR_DEV v8i frag_f6(const uint8_t* frag, int lane) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(frag + lane * 16);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(frag + 1024 + lane * 8);
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], 0, 0};
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] in bits 3:0,
// vmcnt[5:4] in bits 15:14, expcnt in bits 6:4 left at its maximum).
template <int N>
CR_DEV void f6_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// ---------------------------------------------------------------------------
// Block BM x BN (tokens x channels) of waves with TM x TN MFMAs of
// 32 x 32 x 64 each (64 x 64 wave tiles in the large blocks, 32 x 32 in the
// mid-size 64 x 64 block), WN waves along the channels. A stage holds BKT 64-deep
// k-tiles of both operands ((BM + BN) * BKT * 48 bytes) and is filled by
// direct global -> LDS loads in 1 KB wave-loads; S stages rotate, S - 1 of
// them in flight ahead of the one being consumed.
// Scales per tensor or per row on either side; no low-rank branch.
// ---------------------------------------------------------------------------
template <int L>
CR_DEV void f6_wait_stage(int ahead) {   // at most `ahead` later stages (L loads each) left in flight
  if (ahead >= 4) f6_wait_vmcnt<4 * L>();
  else if (ahead == 3) f6_wait_vmcnt<3 * L>();
  else if (ahead == 2) f6_wait_vmcnt<2 * L>();
  else if (ahead == 1) f6_wait_vmcnt<L>();
  else f6_wait_vmcnt<0>();
}

template <int BM, int BN, int TM, int TN, int BKT, int S, int MINB, int OUT>
__global__ __launch_bounds__((BM / (32 * TM)) * (BN / (32 * TN)) * 64, MINB) void gemm_f6_kernel(GemmParams p) {
  constexpr int WN = BN / (32 * TN);                   // waves along the channels
  constexpr int NW = (BM / (32 * TM)) * WN;
  static_assert(BM % (32 * TM) == 0 && BN % (32 * TN) == 0, "whole wave tiles");
  static_assert(S >= 2 && S <= 6, "stages in flight ahead of the current one: 0 to 4");
  constexpr int A_ST = (BM / 32) * BKT * F6_FRAG, W_ST = (BN / 32) * BKT * F6_FRAG;
  constexpr int STAGE = A_ST + W_ST;
  constexpr int NA = A_ST / 1024, NL = STAGE / 1024;   // 1 KB wave-loads per stage (activation part first)
  static_assert(A_ST % 1024 == 0 && W_ST % 1024 == 0, "whole wave-loads");
  constexpr int LPW = (NL + NW - 1) / NW;              // wave-loads of the busiest waves
  constexpr int NHI = NL - (LPW - 1) * NW;             // waves 0 .. NHI-1 take LPW, the others LPW - 1
  constexpr int RUN = BKT * F6_FRAG / 16;              // 16-byte pieces per 32-row block and stage
  constexpr int RS = TN * 64 + 16;                     // epilogue: LDS row stride of a wave's bf16 tile
  constexpr int SMEM = (S * STAGE > NW * TM * 32 * RS) ? S * STAGE : NW * TM * 32 * RS;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;

  // block -> tile: XCD-aware (consecutive blocks go round robin over the 8
  // XCDs), then bands of 8 tile rows walked column by column
  const int ntm = (int)((p.M + BM - 1) / BM);
  const int ntn = (int)(p.N / BN);
  const int ntiles = ntm * ntn;
  int t = (int)blockIdx.x;
  if (ntiles % 8 == 0) t = (t & 7) * (ntiles / 8) + (t >> 3);
  constexpr int GM = 8;
  const int band = t / (GM * ntn);
  const int rows_in_band = min(GM, ntm - band * GM);
  const int within = t - band * GM * ntn;
  const int tn = within / rows_in_band;
  const int tm = band * GM + within % rows_in_band;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t KT = p.K / 64;
  const int nkb = (int)(p.K / (64 * BKT));
  const int64_t MB = (p.M + 31) / 32;

  // wave-load idx = wave + NW j fills stage bytes [idx KB, +1 KB): the
  // activation part for idx < NA, else the weight part. Piece
  // pc = (idx or idx - NA) * 64 + l of a part is byte (pc % RUN) * 16 of the
  // stage's run of 32-row block pc / RUN. Both operands advance by the same
  // BKT * 1536 bytes per stage.
  const uint8_t* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int idx = min(wave + NW * j, NL - 1);
    if (idx < NA) {
      const int pc = idx * 64 + l;
      const int64_t b = imin64(m0 / 32 + pc / RUN, MB - 1);   // blocks past M: the last one, never stored
      src[j] = p.a + b * KT * F6_FRAG + (pc % RUN) * 16;
    } else {
      const int pc = (idx - NA) * 64 + l;
      src[j] = p.w + (n0 / 32 + pc / RUN) * KT * F6_FRAG + (pc % RUN) * 16;
    }
  }
  auto issue = [&](int kb) {
    uint8_t* st = smem + (kb % S) * STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      if (j < LPW - 1 || wave < NHI)
        __builtin_amdgcn_global_load_lds((f6_gptr)(src[j] + (size_t)kb * (BKT * F6_FRAG)),
                                         (f6_lptr)(st + (wave + NW * j) * 1024), 16, 0, 0);
  };
  auto wait_stage = [&](int ahead) {
    if constexpr (NHI == NW) {
      f6_wait_stage<LPW>(ahead);
    } else {
      if (wave < NHI) f6_wait_stage<LPW>(ahead);
      else f6_wait_stage<LPW - 1>(ahead);
    }
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nkb) issue(s);
  for (int kb = 0; kb < nkb; ++kb) {
    wait_stage(min(S - 2, nkb - 1 - kb));           // this wave's loads of stage kb have landed
    __builtin_amdgcn_s_barrier();                    // ... and every wave's; stage kb - 1 is consumed
    if (kb + S - 1 < nkb) issue(kb + S - 1);
    const uint8_t* As = smem + (kb % S) * STAGE;
    const uint8_t* Ws = As + A_ST;
    v8i av[2][TM], wv[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) av[0][i] = frag_f6(As + ((wm * TM + i) * BKT) * F6_FRAG, l);
#pragma unroll
    for (int j = 0; j < TN; ++j) wv[0][j] = frag_f6(Ws + ((wn * TN + j) * BKT) * F6_FRAG, l);
#pragma unroll
    for (int kt = 0; kt < BKT; ++kt) {
      const int cb = kt & 1;
      if (kt + 1 < BKT) {
#pragma unroll
        for (int i = 0; i < TM; ++i) av[cb ^ 1][i] = frag_f6(As + ((wm * TM + i) * BKT + kt + 1) * F6_FRAG, l);
#pragma unroll
        for (int j = 0; j < TN; ++j) wv[cb ^ 1][j] = frag_f6(Ws + ((wn * TN + j) * BKT + kt + 1) * F6_FRAG, l);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_f6_32(wv[cb][j], av[cb][i], acc[i][j]);
    }
  }

  // ---- epilogue: every input loaded before the first store ----
  if constexpr (OUT == CR_OUT_I32_RAW) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + (wm * TM + i) * 32 + (l & 31);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + (wn * TN + j) * 32 + 8 * g + 4 * (l >> 5);
          float y[4] = {0.f, 0.f, 0.f, 0.f};
          int raw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) raw[e] = (int)acc[i][j][4 * g + e];
          store4<OUT>(p, m, n, y, raw);
        }
    }
  } else {
    const float sa_t = (p.a_gran == CR_GRAN_TENSOR) ? p.a_scales[0] : 0.f;
    const float sw_t = (p.w_gran == CR_GRAN_TENSOR) ? p.w_scales[0] : 0.f;
    float sa[TM];
    v4f sw[TN][4];
    u32x2 bias[TN][4];
    if constexpr (OUT == CR_OUT_BF16) {
      // y = s_a s_w acc + bias, rounded to bf16 (v_cvt_pk_bf16_f32, half to
      // even), then the wave's 64 x 64 tile passes through LDS so that every
      // store writes whole 128-byte output rows (the fragment layout would
      // scatter 16-byte pieces over 32 rows per instruction)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + (wm * TM + i) * 32 + (l & 31);
        sa[i] = (p.a_gran == CR_GRAN_TENSOR) ? sa_t : p.a_scales[m < p.M ? m : p.M - 1];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + (wn * TN + j) * 32 + 8 * g + 4 * (l >> 5);
          sw[j][g] = (p.w_gran == CR_GRAN_TENSOR) ? v4f{sw_t, sw_t, sw_t, sw_t}
                                                  : *reinterpret_cast<const v4f*>(p.w_scales + n);
          bias[j][g] = p.bias ? *reinterpret_cast<const u32x2*>(p.bias + n) : u32x2{0u, 0u};
        }
      __syncthreads();                              // every wave is done with the stage buffers
      uint8_t* tile = smem + wave * (TM * 32 * RS);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * g + e] * (sa[i] * sw[j][g][e]);
            y[0] += bf16_lo(bias[j][g][0]);
            y[1] += bf16_hi(bias[j][g][0]);
            y[2] += bf16_lo(bias[j][g][1]);
            y[3] += bf16_hi(bias[j][g][1]);
            const v2bf lo = __builtin_convertvector((v2f){y[0], y[1]}, v2bf);
            const v2bf hi = __builtin_convertvector((v2f){y[2], y[3]}, v2bf);
            const int r = i * 32 + (l & 31);
            const int cb = (j * 32 + 8 * g + 4 * (l >> 5)) * 2;
            *reinterpret_cast<u32x2*>(tile + r * RS + cb) =
                u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          }
      f6_wait_vmcnt<63>();                          // this wave's tile writes are done (LDS is in order per wave)
      constexpr int PR = TN * 4;                    // 16-byte pieces per tile row
#pragma unroll
      for (int q = 0; q < TM * 32 * PR / 64; ++q) {
        const int pc = q * 64 + l;
        const int r = pc / PR, c = pc % PR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * RS + c * 16);
        const int64_t m = m0 + wm * TM * 32 + r;
        if (m < p.M)
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldc + n0 + wn * TN * 32 + c * 8) = v;
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + (wm * TM + i) * 32 + (l & 31);
      sa[i] = (p.a_gran == CR_GRAN_TENSOR) ? sa_t : p.a_scales[m < p.M ? m : p.M - 1];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + (wn * TN + j) * 32 + 8 * g + 4 * (l >> 5);
        sw[j][g] = (p.w_gran == CR_GRAN_TENSOR) ? v4f{sw_t, sw_t, sw_t, sw_t}
                                                : *reinterpret_cast<const v4f*>(p.w_scales + n);
        bias[j][g] = p.bias ? *reinterpret_cast<const u32x2*>(p.bias + n) : u32x2{0u, 0u};
      }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + (wm * TM + i) * 32 + (l & 31);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + (wn * TN + j) * 32 + 8 * g + 4 * (l >> 5);
          float y[4];
          const int raw[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * g + e] * (sa[i] * sw[j][g][e]);
          y[0] += bf16_lo(bias[j][g][0]);
          y[1] += bf16_hi(bias[j][g][0]);
          y[2] += bf16_lo(bias[j][g][1]);
          y[3] += bf16_hi(bias[j][g][1]);
          store4<OUT>(p, m, n, y, raw);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// 64-group scales on both sides (the SVDQuant format): one 32 x 32 x 64 matrix
// op covers exactly one group, so its float32 result P (exact) is scaled
// right away: y += P * (s_a[m, g] * s_w[n, g]). The scale products come from
// a two-block outer-product matrix op (see the loop), which leaves one VALU
// FMA per output and group. Unsigned shifted activations (codes u in
// [0, 15]) come as the E2M3 values u/2, so P is half the integer sum and the
// factor 2 joins the scale.
// Block 128 x 128, 2 x 2 waves of 64 x 64, stages of two k-tiles with their
// scales (26 KB: activation scales gathered as 4-byte pieces of the row-major
// [M, K/64] array, weight scales a contiguous 1 KB run of the packed
// [N/128][K/64][128] array), two in the ring, three blocks per CU (167
// VGPRs: one channel column's scale products and group sums are live at a
// time beside the 64 sums). Epilogue: shift correction, low-rank branch
// (32 x 32 x 16 bf16 or 32 x 32 x 2 f32 matrix ops onto the outputs), bias,
// bf16 rows through LDS.
// ---------------------------------------------------------------------------
template <bool UNS>
CR_DEV void f6_lowrank_32(const GemmParams& p, int64_t m0w, int64_t n0w, int l, v16f (&y)[2][2]) {
  const int lr = l & 31, h = l >> 5;
  const int R = p.R;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0w + j * 32 + lr;   // L1 in the tiled layout [N/128][R][128]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t mr = imin64(m0w + i * 32 + lr, p.M - 1);
      if (!p.lora_f32) {
        const uint16_t* la = reinterpret_cast<const uint16_t*>(p.lora_act) + mr * R;
        for (int r0 = 0; r0 < R; r0 += 16)
          y[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lora_up8(p.lora_up, R, n, r0 + 8 * h),
              __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(la + r0 + 8 * h)), y[i][j], 0, 0, 0);
      } else {
        const float* la = reinterpret_cast<const float*>(p.lora_act) + mr * R;
        for (int r0 = 0; r0 < R; r0 += 2)
          y[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(lora_up1(p.lora_up, R, n, r0 + h), la[r0 + h],
                                                         y[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int OUT, bool UNS>
__global__ __launch_bounds__(256, 3) void gemm_f6_grp_kernel(GemmParams p) {
  constexpr int BM = 128, BN = 128, BKT = 2, NW = 4, WN = 2;
  constexpr int A_ST = (BM / 32) * BKT * F6_FRAG, W_ST = (BN / 32) * BKT * F6_FRAG;
  constexpr int SA_ST = BKT * BM * 4, SW_ST = BKT * BN * 4;
  constexpr int STAGE = A_ST + W_ST + SA_ST + SW_ST;
  constexpr int NL = (A_ST + W_ST) / 1024, NA = A_ST / 1024, LPW = NL / NW;
  static_assert(NL % NW == 0 && SA_ST == 256 * NW && SW_ST == 256 * NW, "loads split evenly over the waves");
  constexpr int RUN = BKT * F6_FRAG / 16;
  constexpr int RS = 144;                              // epilogue: LDS row stride of a 64 x 64 bf16 tile
  static_assert(NW * 64 * RS <= 2 * STAGE, "epilogue tiles fit the stage buffers");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int l = tid & 63, lr = l & 31, h = l >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  const int ntm = (int)((p.M + BM - 1) / BM);
  const int ntn = (int)(p.N / BN);
  const int ntiles = ntm * ntn;
  int t = (int)blockIdx.x;
  if (ntiles % 8 == 0) t = (t & 7) * (ntiles / 8) + (t >> 3);
  constexpr int GM = 8;
  const int band = t / (GM * ntn);
  const int rows_in_band = min(GM, ntm - band * GM);
  const int within = t - band * GM * ntn;
  const int tn = within / rows_in_band;
  const int tm = band * GM + within % rows_in_band;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t KT = p.K / 64;
  const int nkb = (int)(p.K / (64 * BKT));
  const int64_t MB = (p.M + 31) / 32;

  const uint8_t* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int idx = wave + NW * j;
    if (idx < NA) {
      const int pc = idx * 64 + l;
      const int64_t b = imin64(m0 / 32 + pc / RUN, MB - 1);
      src[j] = p.a + b * KT * F6_FRAG + (pc % RUN) * 16;
    } else {
      const int pc = (idx - NA) * 64 + l;
      src[j] = p.w + (n0 / 32 + pc / RUN) * KT * F6_FRAG + (pc % RUN) * 16;
    }
  }
  // scale entry e = wave * 64 + l of a stage: k-tile e / 128, row (column) e % 128
  const int ske = wave * 64 + l;
  const float* sa_src = p.a_scales + imin64(m0 + ske % BM, p.M - 1) * KT + ske / BM;
  const float* sw_src = p.w_scales + n0 * KT + ske;   // packed: [N/128][K/64][128]
  auto issue = [&](int kb) {
    uint8_t* st = smem + (kb % 2) * STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_global_load_lds((f6_gptr)(src[j] + (size_t)kb * (BKT * F6_FRAG)),
                                       (f6_lptr)(st + (wave + NW * j) * 1024), 16, 0, 0);
    if constexpr (OUT != CR_OUT_I32_RAW) {
      __builtin_amdgcn_global_load_lds((f6_gptr)(sa_src + kb * BKT), (f6_lptr)(st + A_ST + W_ST + wave * 256), 4, 0, 0);
      __builtin_amdgcn_global_load_lds((f6_gptr)(sw_src + (size_t)kb * (BKT * BN)),
                                       (f6_lptr)(st + A_ST + W_ST + SA_ST + wave * 256), 4, 0, 0);
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
  constexpr float UF = UNS ? 2.f : 1.f;

  issue(0);
  for (int kb = 0; kb < nkb; ++kb) {
    f6_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kb + 1 < nkb) issue(kb + 1);
    const uint8_t* As = smem + (kb % 2) * STAGE;
    const uint8_t* Ws = As + A_ST;
    const float* Sa = reinterpret_cast<const float*>(As + A_ST + W_ST);
    const float* Sw = Sa + BKT * BM;
#pragma unroll
    for (int kt = 0; kt < BKT; ++kt) {
      v8i av[2], wv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = frag_f6(As + ((wm * 2 + i) * BKT + kt) * F6_FRAG, l);
#pragma unroll
      for (int j = 0; j < 2; ++j) wv[j] = frag_f6(Ws + ((wn * 2 + j) * BKT + kt) * F6_FRAG, l);
      if constexpr (OUT == CR_OUT_I32_RAW) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f6_32(wv[j], av[i], acc[i][j]);
      } else {
        // the scale products s_a[m] s_w[n] of both 32 x 32 tiles of column j
        // come from one two-block outer-product matrix op (block i = tokens
        // 32 i .., lane l gives s_a of token l and s_w of channel l % 32), in
        // the 32 x 32 output layout of the fp6 op: one FMA per output and
        // group is left on the vector ALUs
        const float sa = Sa[kt * BM + wm * 64 + l] * UF;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const v32f c = __builtin_amdgcn_mfma_f32_32x32x1f32(Sw[kt * BN + (wn * 2 + j) * 32 + lr], sa, v32f{}, 0, 0, 0);
          const v16f p0 = mfma_f6_32(wv[j], av[0], v16f{});
          const v16f p1 = mfma_f6_32(wv[j], av[1], v16f{});
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[0][j][r] = __builtin_fmaf(p0[r], c[r], acc[0][j][r]);
            acc[1][j][r] = __builtin_fmaf(p1[r], c[16 + r], acc[1][j][r]);
          }
          asm volatile("" : "+v"(acc[0][j]), "+v"(acc[1][j]));   // one column's products live at a time
        }
      }
    }
  }

  const int64_t m0w = m0 + wm * 64, n0w = n0 + wn * 64;
  if constexpr (OUT == CR_OUT_I32_RAW) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float y[4] = {0.f, 0.f, 0.f, 0.f};
          int raw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) raw[e] = (int)(acc[i][j][4 * g + e] * UF);
          store4<OUT>(p, m0w + i * 32 + lr, n0w + j * 32 + 8 * g + 4 * h, y, raw);
        }
    return;
  } else {
    // shift correction and bias first (loads before any store), then the low-rank branch
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0w + j * 32 + 8 * g + 4 * h;
        v4f c = v4f{0.f, 0.f, 0.f, 0.f};
        if constexpr (UNS) {
          const v4f ws = *reinterpret_cast<const v4f*>(p.w_sum + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) c[e] = -p.a_shift * ws[e];
        }
        const u32x2 bb = p.bias ? *reinterpret_cast<const u32x2*>(p.bias + n) : u32x2{0u, 0u};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          acc[i][j][4 * g + 0] = __builtin_fmaf(1.f, c[0], acc[i][j][4 * g + 0]) + bf16_lo(bb[0]);
          acc[i][j][4 * g + 1] = __builtin_fmaf(1.f, c[1], acc[i][j][4 * g + 1]) + bf16_hi(bb[0]);
          acc[i][j][4 * g + 2] = __builtin_fmaf(1.f, c[2], acc[i][j][4 * g + 2]) + bf16_lo(bb[1]);
          acc[i][j][4 * g + 3] = __builtin_fmaf(1.f, c[3], acc[i][j][4 * g + 3]) + bf16_hi(bb[1]);
        }
      }
    if (p.lora_act) f6_lowrank_32<UNS>(p, m0w, n0w, l, acc);
    if constexpr (OUT == CR_OUT_F32) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int64_t m = m0w + i * 32 + lr;
            if (m < p.M)
              *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.out) + m * p.ldc + n0w + j * 32 + 8 * g + 4 * h) =
                  v4f{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          }
    } else {
      __syncthreads();                                 // every wave is done with the stage buffers
      uint8_t* tile = smem + wave * (64 * RS);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v2bf lo = __builtin_convertvector((v2f){acc[i][j][4 * g], acc[i][j][4 * g + 1]}, v2bf);
            const v2bf hi = __builtin_convertvector((v2f){acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]}, v2bf);
            *reinterpret_cast<u32x2*>(tile + (i * 32 + lr) * RS + (j * 32 + 8 * g + 4 * h) * 2) =
                u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          }
      f6_wait_vmcnt<63>();                             // this wave's tile writes are done
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = (l >> 3) + 8 * q;
        const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * RS + (l & 7) * 16);
        const int64_t m = m0w + r;
        if (m < p.M) *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldc + n0w + (l & 7) * 8) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small-M kernel (M <= 64): weight streaming. A block owns 16 output channels
// (half of a 32-row weight block); its SK waves take the 128-deep k-steps
// round robin and read their fragments straight from global memory in the
// 16 x 16 x 128 operand order (lane l: row l % 16, k-quarter l / 16, which is
// k-half (l / 16) % 2 of k-tile 2 s + l / 32 in the 32 x 64 fragment layout).
// Partial sums are reduced through LDS in a fixed order; the 16 x 16 result
// layout is that of the int8 kernels, so the shared epilogue (low-rank
// branch included) applies unchanged.
// ---------------------------------------------------------------------------
constexpr int F6_SK_WAVES = 16;

// lane l's 24 bytes for rows r0 .. r0+15 (r0 = 0 or 16 inside a 32-row block)
// and k-step s (128 deep) of the [rows/32][K/64][1536 B] array at `blk`
CR_DEV v8i frag_f6_16(const uint8_t* blk, int64_t s, int r0, int l) {
  const int q = l >> 4;                              // k-quarter 0..3
  const uint8_t* frag = blk + (2 * s + (q >> 1)) * F6_FRAG;
  return frag_f6(frag, ((q & 1) << 5) + r0 + (l & 15));
}

template <int FM, int OUT>
__global__ __launch_bounds__(F6_SK_WAVES * 64) void gemm_f6_skinny_kernel(GemmParams p) {
  constexpr int NW = F6_SK_WAVES;
  constexpr int U = 2;                               // k-steps in flight per wave
  __shared__ __attribute__((aligned(16))) float red[NW][FM][64][4];
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t KT = p.K / 64;
  const int nks = (int)(p.K / 128);
  const uint8_t* wblk = p.w + (n0 >> 5) * KT * F6_FRAG;
  const int wr0 = (int)(n0 & 16);

  v4f acc[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int s0 = wave * U; s0 < nks; s0 += NW * U) {
    v8i wr[U], ar[U][FM];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      if (s >= nks) break;
      wr[u] = frag_f6_16(wblk, s, wr0, l);
#pragma unroll
      for (int i = 0; i < FM; ++i) ar[u][i] = frag_f6_16(p.a + (int64_t)(i >> 1) * KT * F6_FRAG, s, (i & 1) * 16, l);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u >= nks) break;
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[i] = mfma_f6_16(wr[u], ar[u][i], acc[i]);
    }
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][i][l][e] = acc[i][e];
  __syncthreads();
  if (wave < FM) {
    const int i = wave;
    float y[4];
    int raw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float t = red[0][i][l][e];
#pragma unroll
      for (int w = 1; w < NW; ++w) t += red[w][i][l][e];   // exact: integers below 2^24
      raw[e] = (int)t;
      y[e] = t;
    }
    const int64_t mb = i * 16;
    const int64_t m = mb + (l & 15);
    const int64_t n = n0 + (l >> 4) * 4;
    if constexpr (OUT != CR_OUT_I32_RAW) {
      const int64_t mc = m < p.M ? m : p.M - 1;
      const float sa = (p.a_gran == CR_GRAN_TENSOR) ? p.a_scales[0] : p.a_scales[mc];
      v4f sw;
      if (p.w_gran == CR_GRAN_TENSOR) {
        const float t = p.w_scales[0];
        sw = v4f{t, t, t, t};
      } else {
        sw = *reinterpret_cast<const v4f*>(p.w_scales + n);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = y[e] * (sa * sw[e]);
    }
    finish_block<OUT>(p, m, n, mb, l, y, raw);
  }
}

template <int OUT>
static hipError_t launch_f6_out(const GemmParams& p, hipStream_t s) {
  if (p.grouped) {
    const int64_t tiles = ((p.M + 127) / 128) * (p.N / 128);
    if (p.act == ACT_U4) hipLaunchKernelGGL((gemm_f6_grp_kernel<OUT, true>), dim3((unsigned)tiles), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_f6_grp_kernel<OUT, false>), dim3((unsigned)tiles), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  if (p.M <= 64) {
    const dim3 grid((unsigned)(p.N / 16));
    switch ((p.M + 15) / 16) {
      case 1: hipLaunchKernelGGL((gemm_f6_skinny_kernel<1, OUT>), grid, dim3(F6_SK_WAVES * 64), 0, s, p); break;
      case 2: hipLaunchKernelGGL((gemm_f6_skinny_kernel<2, OUT>), grid, dim3(F6_SK_WAVES * 64), 0, s, p); break;
      case 3: hipLaunchKernelGGL((gemm_f6_skinny_kernel<3, OUT>), grid, dim3(F6_SK_WAVES * 64), 0, s, p); break;
      default: hipLaunchKernelGGL((gemm_f6_skinny_kernel<4, OUT>), grid, dim3(F6_SK_WAVES * 64), 0, s, p); break;
    }
    return hipGetLastError();
  }
  // 256 x 256 blocks (16 waves, 147 KB of stages) for wide outputs with at
  // least three rounds of tiles on the 256 CUs (8192 x 12288: 1536; 8192 x
  // 6144: 768, measured 103 against 111-113 us with 256 x 192 blocks): a
  // sixth less operand traffic per output than 256 x 192; 256 x 192 blocks (one per CU, 12
  // waves) when they fill the chip: a third less operand traffic per output
  // than 128 x 128 (measured on MI355X at 4096 x 3072 x 3072: 30.4 against
  // 32.9 us); otherwise 128 x 128 blocks, three per CU, or 64 x 64 blocks
  // for mid-size M
  if (p.N % 256 == 0 && ((p.M + 255) / 256) * (p.N / 256) >= 768) {
    const int64_t tiles = ((p.M + 255) / 256) * (p.N / 256);
    hipLaunchKernelGGL((gemm_f6_kernel<256, 256, 2, 2, 2, 3, 1, OUT>), dim3((unsigned)tiles), dim3(1024), 0, s, p);
    return hipGetLastError();
  }
  if (p.N % 192 == 0 && ((p.M + 255) / 256) * (p.N / 192) >= 256) {
    const int64_t tiles = ((p.M + 255) / 256) * (p.N / 192);
    hipLaunchKernelGGL((gemm_f6_kernel<256, 192, 2, 2, 2, 3, 1, OUT>), dim3((unsigned)tiles), dim3(768), 0, s, p);
    return hipGetLastError();
  }
  const int64_t tiles = ((p.M + 127) / 128) * (p.N / 128);
  if (tiles < 256) {
    // mid-size M (e.g. 512 text tokens): 128 x 128 blocks leave most CUs
    // idle, so 64 x 64 blocks of four 32 x 32 waves, three stages
    const int64_t t64 = ((p.M + 63) / 64) * (p.N / 64);
    hipLaunchKernelGGL((gemm_f6_kernel<64, 64, 1, 1, 2, 3, 4, OUT>), dim3((unsigned)t64), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_f6_kernel<128, 128, 2, 2, 2, 2, 3, OUT>), dim3((unsigned)tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_f6(const GemmParams& p, hipStream_t s) {
  switch (p.out_type) {
    case CR_OUT_BF16: return launch_f6_out<CR_OUT_BF16>(p, s);
    case CR_OUT_F32: return launch_f6_out<CR_OUT_F32>(p, s);
    default: return launch_f6_out<CR_OUT_I32_RAW>(p, s);
  }
}

}  // namespace cr
