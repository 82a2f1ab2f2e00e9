// W4A4 GEMM (gfx950): int4 activations x tile-packed int4 weights on the
// int8 matrix cores, with the fused epilogue (tensor / row / 64-group
// scales, unsigned-shift correction, low-rank up-projection, bias).
//
// "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4" page, Measurements: a fused
// INT4 matrix multiply with a rank-one (s_a x s_w) rescale. "Qwen-Image-Edit-
// 2511 INT4 (ComfyUI Optimized)", Key Technical Optimizations (tile-packed
// weights, fused LoRA-up) and Kernel Engineering (multi-stage global->shared
// pipeline, scales staged in shared memory, unsigned +0.171875 activations).
//
// gfx950 has no int4 matrix instruction: a signed nibble q is widened
// exactly to the byte 16*q with one mask (no shift), so
// v_mfma_i32_16x16x64_i8 accumulates 256 * sum(qa*qw) (16 * sum for unsigned
// activation bytes) and an exact arithmetic shift recovers the integer.
//
// Operand roles: MFMA A = weights (16 output channels), B = activations (16
// tokens); a lane of the 16x16 result holds one token and four consecutive
// channels (one 8-byte bf16 store).
//
// Data movement per stage (BK = 128, two 64-deep k-tiles): the activation
// codes come in the tiled layout [M/16][K/64][512 B] (or natural rows) and
// the weights in [N/128][K/64][8][512 B]; each 512-byte run is one operand
// fragment, so global loads are 16-byte contiguous pieces, LDS stores and
// fragment reads are linear (bank-conflict free). Two register sets keep
// the loads two stages ahead of the matrix cores; LDS is double-buffered.

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace cr {

typedef float v2f_w __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_w __attribute__((ext_vector_type(2)));

template <int ACT>
CR_DEV v4i widen_a4(u32x2 x) {
  return ACT == ACT_S4 ? widen_s4x16(x) : widen_u4(x);
}

template <int BM, int BN, int WM, int WN, int MINB, int ACT, bool A_TILED, bool GROUPED, int OUT>
__global__ __launch_bounds__(WM * WN * 64, MINB) void gemm_w4a4_kernel(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int A_ST = BM * 64;            // bytes per stage: BM rows x 128 k x 4 bit
  constexpr int W_ST = BN * 64;
  constexpr bool GRP = GROUPED && OUT != CR_OUT_I32_RAW;
  constexpr int S_ST = GRP ? 2 * (BM + BN) * 4 : 0;
  constexpr int STAGE = A_ST + W_ST + S_ST;
  constexpr int SH = (ACT == ACT_S4) ? 8 : 4;
  constexpr int PA = A_ST / 16 / NT;       // 16-byte pieces per thread per stage
  constexpr int PW = W_ST / 16 / NT;
  constexpr int PS = GRP ? (2 * (BM + BN) + NT - 1) / NT : 0;
  static_assert(A_ST % (16 * NT) == 0 && W_ST % (16 * NT) == 0, "tile / thread mismatch");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // block -> tile: consecutive block ids land on different XCDs, so each XCD
  // gets a contiguous range of tiles, walked in bands of 8 tile rows column
  // by column (neighbouring tiles share operands in that XCD's L2).
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
  const int64_t KT = K / 64;
  const int nkb = (int)(K / 128);
  const int64_t MB = (p.M + 15) / 16;

  // per-thread global byte offsets at stage 0 (+ stage * stride later)
  uint32_t offa[PA], offw[PW];
#pragma unroll
  for (int j = 0; j < PA; ++j) {
    const int pc = tid + j * NT;
    if constexpr (A_TILED) {
      const int mb = pc >> 6;                                    // 1 KB = 64 pieces per 16-row block
      const int64_t b = imin64(m0 / 16 + mb, MB - 1);
      offa[j] = (uint32_t)(b * KT * 512 + (pc & 63) * 16);
    } else {
      const int row = pc >> 2, part = pc & 3;                    // 4 x 16 B per row per stage
      const int64_t m = imin64(m0 + row, p.M - 1);
      offa[j] = (uint32_t)(m * (K / 2) + part * 16);
    }
  }
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    const int pc = tid + j * NT;
    const int nb = pc >> 6, w = pc & 63;                         // 16-col block, piece inside its 1 KB
    const int64_t n16 = n0 / 16 + nb;
    offw[j] = (uint32_t)(((n16 >> 3) * KT + (w >> 5)) * 4096 + (n16 & 7) * 512 + (w & 31) * 16);
  }
  const uint32_t a_stride = A_TILED ? 1024u : 64u;               // bytes per stage
  const uint32_t w_stride = 8192u;

  auto gload = [&](int kb, u32x4 (&ra)[PA], u32x4 (&rw)[PW], float (&rs)[PS > 0 ? PS : 1]) {
#pragma unroll
    for (int j = 0; j < PA; ++j) ra[j] = *reinterpret_cast<const u32x4*>(p.a + offa[j] + (uint32_t)kb * a_stride);
#pragma unroll
    for (int j = 0; j < PW; ++j) rw[j] = *reinterpret_cast<const u32x4*>(p.w + offw[j] + (uint32_t)kb * w_stride);
    if constexpr (GRP) {
      const int64_t G = KT;
#pragma unroll
      for (int j = 0; j < PS; ++j) {
        const int idx = tid + j * NT;
        if (idx < 2 * BM) {
          const int kt = idx / BM, r = idx % BM;
          const int64_t m = imin64(m0 + r, p.M - 1);
          rs[j] = p.a_scales[m * G + kb * 2 + kt];
        } else if (idx < 2 * (BM + BN)) {
          const int q = idx - 2 * BM;
          const int kt = q / BN, c = q % BN;
          const int64_t n = n0 + c;
          rs[j] = p.w_scales[((n >> 7) * G + kb * 2 + kt) * 128 + (n & 127)];
        }
      }
    }
  };
  auto lstore = [&](int buf, const u32x4 (&ra)[PA], const u32x4 (&rw)[PW], const float (&rs)[PS > 0 ? PS : 1]) {
    uint8_t* As = smem + buf * STAGE;
    uint8_t* Ws = As + A_ST;
#pragma unroll
    for (int j = 0; j < PA; ++j) {
      const int pc = tid + j * NT;
      if constexpr (A_TILED) {
        *reinterpret_cast<u32x4*>(As + pc * 16) = ra[j];
      } else {
        const int row = pc >> 2, part = pc & 3;
        const int kt = part >> 1, c = (part & 1) * 2;
        uint8_t* base = As + ((row >> 4) * 2 + kt) * 512;
        *reinterpret_cast<u32x2*>(base + (c * 16 + (row & 15)) * 8) = u32x2{ra[j][0], ra[j][1]};
        *reinterpret_cast<u32x2*>(base + ((c + 1) * 16 + (row & 15)) * 8) = u32x2{ra[j][2], ra[j][3]};
      }
    }
#pragma unroll
    for (int j = 0; j < PW; ++j) *reinterpret_cast<u32x4*>(Ws + (tid + j * NT) * 16) = rw[j];
    if constexpr (GRP) {
      float* Ss = reinterpret_cast<float*>(Ws + W_ST);
#pragma unroll
      for (int j = 0; j < PS; ++j) {
        const int idx = tid + j * NT;
        if (idx < 2 * (BM + BN)) Ss[idx] = rs[j];
      }
    }
  };

  v4i acc[FM][FN];
  float yacc[GRP ? FM : 1][GRP ? FN : 1][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  if constexpr (GRP) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) yacc[i][j][e] = 0.f;
  }

  auto compute = [&](int buf) {
    const uint8_t* As = smem + buf * STAGE;
    const uint8_t* Ws = As + A_ST;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      v4i wv[FN], av[FM];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        wv[j] = widen_s4x16(*reinterpret_cast<const u32x2*>(Ws + ((wn * FN + j) * 2 + kt) * 512 + l * 8));
#pragma unroll
      for (int i = 0; i < FM; ++i)
        av[i] = widen_a4<ACT>(*reinterpret_cast<const u32x2*>(As + ((wm * FM + i) * 2 + kt) * 512 + l * 8));
      if constexpr (GRP) {
        const float* Ss = reinterpret_cast<const float*>(Ws + W_ST);
        float sa[FM];
        v4f sw[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = Ss[kt * BM + (wm * FM + i) * 16 + (l & 15)];
#pragma unroll
        for (int j = 0; j < FN; ++j)
          sw[j] = *reinterpret_cast<const v4f*>(Ss + 2 * BM + kt * BN + (wn * FN + j) * 16 + (l >> 4) * 4);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            v4i pp = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[j], av[i], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              yacc[i][j][e] = __builtin_fmaf((float)(pp[e] >> SH) * sw[j][e], sa[i], yacc[i][j][e]);
          }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[j], av[i], acc[i][j], 0, 0, 0);
      }
    }
  };

  // two register sets: set (kb & 1) holds stage kb until it is stored to LDS
  u32x4 ra0[PA], rw0[PW], ra1[PA], rw1[PW];
  float rs0[PS > 0 ? PS : 1], rs1[PS > 0 ? PS : 1];
  gload(0, ra0, rw0, rs0);
  if (nkb > 1) gload(1, ra1, rw1, rs1);
  lstore(0, ra0, rw0, rs0);
  __syncthreads();
  for (int kb = 0; kb < nkb; kb += 2) {
    // even stage kb: LDS buffer 0; set 0 is free, set 1 holds stage kb+1
    if (kb + 2 < nkb) gload(kb + 2, ra0, rw0, rs0);
    compute(0);
    if (kb + 1 < nkb) lstore(1, ra1, rw1, rs1);
    __syncthreads();
    if (kb + 1 >= nkb) break;
    // odd stage kb+1: LDS buffer 1; set 1 is free, set 0 holds stage kb+2
    if (kb + 3 < nkb) gload(kb + 3, ra1, rw1, rs1);
    compute(1);
    if (kb + 2 < nkb) lstore(0, ra0, rw0, rs0);
    __syncthreads();
  }

  // ---- epilogue ----
  const float sa_t = (!GRP && p.a_gran == CR_GRAN_TENSOR) ? p.a_scales[0] : 0.f;
  const float sw_t = (!GRP && p.w_gran == CR_GRAN_TENSOR) ? p.w_scales[0] : 0.f;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t mb = m0 + (wm * FM + i) * 16;
    const int64_t m = mb + (l & 15);
    const int64_t mc = m < p.M ? m : p.M - 1;
    float sa = 0.f;
    if constexpr (!GRP && OUT != CR_OUT_I32_RAW) sa = (p.a_gran == CR_GRAN_TENSOR) ? sa_t : p.a_scales[mc];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + (wn * FN + j) * 16 + (l >> 4) * 4;
      float y[4];
      int raw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[e] = acc[i][j][e] >> SH;
      if constexpr (GRP) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = yacc[i][j][e];
      } else if constexpr (OUT != CR_OUT_I32_RAW) {
        v4f sw;
        if (p.w_gran == CR_GRAN_TENSOR) sw = v4f{sw_t, sw_t, sw_t, sw_t};
        else sw = *reinterpret_cast<const v4f*>(p.w_scales + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (float)raw[e] * (sa * sw[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = 0.f;
      }
      finish_block<OUT>(p, m, n, mb, l, y, raw);
    }
  }
}

// ---------------------------------------------------------------------------
// Main kernel for tile-ordered activation codes with tensor or row scales:
// operands go straight from global memory into LDS (global_load_lds_dwordx4:
// each wave instruction moves 64 arbitrary 16-byte pieces into 1 KB of
// contiguous LDS, no staging registers), through a ring of LDS_S stages of
// two 64-deep k-tiles (LDS_S - 1 stages in flight). One barrier per stage:
// each wave waits for its own loads of the stage (vmcnt: the loads of later
// stages stay in flight) and its own LDS reads (lgkmcnt), then s_barrier
// makes the stage visible to every wave and frees the slot the next loads
// go into. The fence that __syncthreads() adds would also wait for the
// loads of later stages, so the barrier is issued bare.
// Block 128 x 128, 2 x 2 waves of 64 x 64, three blocks per CU (measured on
// MI355X at M=4096, N=K=3072: 42.5 us against 49.6 us for the register-
// staged kernel). Three stages (48 KB per block) measured slower: 46 us at
// that shape, 270 against 234 us at 8192 x 12288 x 3072.
// ---------------------------------------------------------------------------
typedef const void __attribute__((address_space(1)))* gas_ptr;
typedef void __attribute__((address_space(3)))* las_ptr;

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] in bits 3:0,
// vmcnt[5:4] in bits 15:14, expcnt in bits 6:4 left at its maximum).
template <int N>
CR_DEV void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Wait until at most AHEAD_MAX stages' loads of this wave (L each) remain in
// flight, for `ahead` later stages already issued (0 <= ahead <= 2).
template <int L>
CR_DEV void wait_stage(int ahead) {
  if (ahead >= 2) wait_vmcnt_lgkm0<2 * L>();
  else if (ahead == 1) wait_vmcnt_lgkm0<L>();
  else wait_vmcnt_lgkm0<0>();
}

#ifndef CR_W4A4_LDS_S
#define CR_W4A4_LDS_S 2
#endif
#ifndef CR_W4A4_LDS_BKT
#define CR_W4A4_LDS_BKT 2
#endif
constexpr int LDS_BM = 128, LDS_BN = 128, LDS_BKT = CR_W4A4_LDS_BKT, LDS_S = CR_W4A4_LDS_S;

// GRP: 64-group scales (the float epilogue runs per k-tile). A stage then
// also holds the scales of its two k-tiles: activation scales [2][BM] (4-byte
// pieces from the row-major [M, K/64] array) and weight scales [2][BN] (one
// 1 KB piece of the tile-packed [N/128][K/64][128] array).
template <int ACT, int OUT, bool GRP>
__global__ __launch_bounds__(256, GRP ? 2 : 3) void gemm_w4a4_lds_kernel(GemmParams p) {
  constexpr int BM = LDS_BM, BN = LDS_BN, BKT = LDS_BKT, S = LDS_S;
  constexpr int WN = 2, NW = 4;
  constexpr int FM = BM / 2 / 16, FN = BN / WN / 16;
  constexpr int A_ST = BM * 32 * BKT, W_ST = BN * 32 * BKT;
  constexpr int SA_ST = GRP ? BKT * BM * 4 : 0, SW_ST = GRP ? BKT * BN * 4 : 0;
  constexpr int STAGE = A_ST + W_ST + SA_ST + SW_ST;
  constexpr int NA = A_ST / 1024, NWL = W_ST / 1024;   // 1 KB wave-loads per stage
  static_assert(NA % NW == 0 && NWL % NW == 0, "wave-loads split evenly over the waves");
  static_assert(SW_ST == 0 || SW_ST == 1024, "weight scales of a stage are one wave-load");
  constexpr int LA = NA / NW, LW = NWL / NW;
  constexpr int LSA = SA_ST / 256 / NW;                // 256-byte (4 B per lane) wave-loads per wave
  static_assert(SA_ST % (256 * NW) == 0, "activation scales split evenly over the waves");
  constexpr int SH = (ACT == ACT_S4) ? 8 : 4;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;

  // block -> tile, as in the register-staged kernel (XCD-aware, bands of 8 tile rows)
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
  const int64_t MB = (p.M + 15) / 16;

  // LDS stage: A [BM/16][BKT][512 B], W [BN/16][BKT][512 B]; wave-load wl
  // fills bytes [wl * 1 KB, +1 KB) of its part. Lane offsets at stage 0:
  uint32_t offa[LA], offw[LW];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int pc = (wave + NW * j) * 64 + l;            // 16-byte piece of the A part
    const int mb = pc / (BKT * 32), w = pc % (BKT * 32);
    const int64_t b = imin64(m0 / 16 + mb, MB - 1);     // rows past M: the last block, never stored
    offa[j] = (uint32_t)(b * KT * 512 + w * 16);
  }
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    const int pc = (wave + NW * j) * 64 + l;
    const int nb = pc / (BKT * 32), w = pc % (BKT * 32), kt = w / 32, r = w % 32;
    const int64_t n16 = n0 / 16 + nb;
    offw[j] = (uint32_t)(((n16 >> 3) * KT + kt) * 4096 + (n16 & 7) * 512 + r * 16);
  }
  // scales (GRP): activation-scale entry e = kt * BM + r of a stage is
  // a_scales[(m0 + r) * K/64 + BKT * kb + kt]; the weight scales of a stage
  // are the 1 KB run ((n0 / 128) * K/64 + BKT * kb) * 512 of the packed array
  int64_t offsa[GRP ? LSA : 1];
  if constexpr (GRP) {
#pragma unroll
    for (int j = 0; j < LSA; ++j) {
      const int e = (wave + NW * j) * 64 + l;
      const int kt = e / BM, r = e % BM;
      offsa[j] = imin64(m0 + r, p.M - 1) * KT + kt;
    }
  }
  auto issue = [&](int kb) {
    uint8_t* st = smem + (kb % S) * STAGE;
    const uint8_t* ga = p.a + (size_t)kb * (BKT * 512);
    const uint8_t* gw = p.w + (size_t)kb * (BKT * 4096);
#pragma unroll
    for (int j = 0; j < LA; ++j)
      __builtin_amdgcn_global_load_lds((gas_ptr)(ga + offa[j]), (las_ptr)(st + (wave + NW * j) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < LW; ++j)
      __builtin_amdgcn_global_load_lds((gas_ptr)(gw + offw[j]), (las_ptr)(st + A_ST + (wave + NW * j) * 1024), 16, 0,
                                       0);
    if constexpr (GRP) {
      uint8_t* ss = st + A_ST + W_ST;
#pragma unroll
      for (int j = 0; j < LSA; ++j)
        __builtin_amdgcn_global_load_lds((gas_ptr)(p.a_scales + offsa[j] + (int64_t)kb * BKT),
                                         (las_ptr)(ss + (wave + NW * j) * 256), 4, 0, 0);
      if (wave == 0)
        __builtin_amdgcn_global_load_lds(
            (gas_ptr)(reinterpret_cast<const uint8_t*>(p.w_scales) + ((n0 >> 7) * KT + (int64_t)kb * BKT) * 512 + l * 16),
            (las_ptr)(ss + SA_ST), 16, 0, 0);
    }
  };

  v4i acc[GRP ? 1 : FM][GRP ? 1 : FN];
  float yacc[GRP ? FM : 1][GRP ? FN : 1][4];
#pragma unroll
  for (int i = 0; i < (GRP ? 1 : FM); ++i)
#pragma unroll
    for (int j = 0; j < (GRP ? 1 : FN); ++j) acc[i][j] = v4i{0, 0, 0, 0};
  if constexpr (GRP) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) yacc[i][j][e] = 0.f;
  }

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nkb) issue(s);

  static_assert(S >= 2 && S <= 4, "stages in flight behind the current one: 0 to 2");
  constexpr int LST = LA + LW + (GRP ? LSA : 0);        // loads per stage of a wave (+1 for wave 0 with GRP)
  for (int kb = 0; kb < nkb; ++kb) {
    const int ahead = min(S - 2, nkb - 1 - kb);         // later stages already issued
    if (GRP && wave == 0) wait_stage<LST + 1>(ahead);
    else wait_stage<LST>(ahead);
    __builtin_amdgcn_s_barrier();
    if (kb + S - 1 < nkb) issue(kb + S - 1);
    const uint8_t* As = smem + (kb % S) * STAGE;
    const uint8_t* Ws = As + A_ST;
    u32x2 ra[2][FM], rw[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) ra[0][i] = *reinterpret_cast<const u32x2*>(As + ((wm * FM + i) * BKT) * 512 + l * 8);
#pragma unroll
    for (int j = 0; j < FN; ++j) rw[0][j] = *reinterpret_cast<const u32x2*>(Ws + ((wn * FN + j) * BKT) * 512 + l * 8);
#pragma unroll
    for (int kt = 0; kt < BKT; ++kt) {
      const int cb = kt & 1;
      if (kt + 1 < BKT) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          ra[cb ^ 1][i] = *reinterpret_cast<const u32x2*>(As + ((wm * FM + i) * BKT + kt + 1) * 512 + l * 8);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          rw[cb ^ 1][j] = *reinterpret_cast<const u32x2*>(Ws + ((wn * FN + j) * BKT + kt + 1) * 512 + l * 8);
      }
      v4i wv[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) wv[j] = widen_s4x16(rw[cb][j]);
      if constexpr (GRP) {
        // y += P * a_s * w_s for this 64-deep group; the widening factor
        // 2^SH is folded into the weight scale (exact: a power of two)
        const float* Ss = reinterpret_cast<const float*>(Ws + W_ST);
        float sa[FM];
        v4f sw[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = Ss[kt * BM + (wm * FM + i) * 16 + (l & 15)];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          sw[j] = *reinterpret_cast<const v4f*>(Ss + BKT * BM + kt * BN + (wn * FN + j) * 16 + (l >> 4) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) sw[j][e] *= 1.0f / (float)(1 << SH);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const v4i av = widen_a4<ACT>(ra[cb][i]);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const v4i pp = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[j], av, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) yacc[i][j][e] = __builtin_fmaf((float)pp[e] * sw[j][e], sa[i], yacc[i][j][e]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const v4i av = widen_a4<ACT>(ra[cb][i]);
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[j], av, acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  if constexpr (OUT == CR_OUT_BF16) {
    // all values first (scales, shift correction, low-rank branch, bias), then
    // bf16 through LDS in two halves of 32 token rows per wave, so that every
    // store writes whole 128-byte output rows (the 16 x 16 fragment layout
    // would write 32-byte pieces of 16 rows per instruction)
    float yv[FM][FN][4];
    const float sa_t = GRP ? 0.f : ((p.a_gran == CR_GRAN_TENSOR) ? p.a_scales[0] : 0.f);
    const float sw_t = GRP ? 0.f : ((p.w_gran == CR_GRAN_TENSOR) ? p.w_scales[0] : 0.f);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t mb = m0 + (wm * FM + i) * 16;
      const int64_t mc = imin64(mb + (l & 15), p.M - 1);
      float sa = 0.f;
      if constexpr (!GRP) sa = (p.a_gran == CR_GRAN_TENSOR) ? sa_t : p.a_scales[mc];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + (wn * FN + j) * 16 + (l >> 4) * 4;
        if constexpr (GRP) {
#pragma unroll
          for (int e = 0; e < 4; ++e) yv[i][j][e] = yacc[i][j][e];
        } else {
          v4f sw;
          if (p.w_gran == CR_GRAN_TENSOR) sw = v4f{sw_t, sw_t, sw_t, sw_t};
          else sw = *reinterpret_cast<const v4f*>(p.w_scales + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) yv[i][j][e] = (float)(acc[i][j][e] >> SH) * (sa * sw[e]);
        }
        finish_values<OUT>(p, n, mb, l, yv[i][j]);
      }
    }
    constexpr int RS = 144;                            // LDS row stride of a 32 x 64 half tile
    static_assert(4 * 32 * RS <= S * STAGE, "half tiles fit the stage buffers");
    __syncthreads();                                   // every wave is done with the stage buffers
    uint8_t* tile = smem + wave * (32 * RS);
#pragma unroll
    for (int hh = 0; hh < FM / 2; ++hh) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float* y = yv[2 * hh + ii][j];
          const v2bf_w lo = __builtin_convertvector((v2f_w){y[0], y[1]}, v2bf_w);
          const v2bf_w hi = __builtin_convertvector((v2f_w){y[2], y[3]}, v2bf_w);
          *reinterpret_cast<u32x2*>(tile + (ii * 16 + (l & 15)) * RS + (j * 16 + (l >> 4) * 4) * 2) =
              u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0): this wave's half tile is written
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int r = (l >> 3) + 8 * qq;
        const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * RS + (l & 7) * 16);
        const int64_t m = m0 + wm * FM * 16 + hh * 32 + r;
        if (m < p.M)
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldc + n0 + wn * FN * 16 + (l & 7) * 8) =
              v;
      }
    }
    return;
  }

  if constexpr (GRP) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t mb = m0 + (wm * FM + i) * 16;
      const int64_t m = mb + (l & 15);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + (wn * FN + j) * 16 + (l >> 4) * 4;
        const int raw[4] = {0, 0, 0, 0};
        finish_block<OUT>(p, m, n, mb, l, yacc[i][j], raw);
      }
    }
    return;
  }

  // ---- epilogue (tensor or row scales) ----
  if constexpr (!GRP) {
  const float sa_t = (p.a_gran == CR_GRAN_TENSOR) ? p.a_scales[0] : 0.f;
  const float sw_t = (p.w_gran == CR_GRAN_TENSOR) ? p.w_scales[0] : 0.f;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t mb = m0 + (wm * FM + i) * 16;
    const int64_t m = mb + (l & 15);
    const int64_t mc = m < p.M ? m : p.M - 1;
    float sa = 0.f;
    if constexpr (OUT != CR_OUT_I32_RAW) sa = (p.a_gran == CR_GRAN_TENSOR) ? sa_t : p.a_scales[mc];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + (wn * FN + j) * 16 + (l >> 4) * 4;
      float y[4];
      int raw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[e] = acc[i][j][e] >> SH;
      if constexpr (OUT != CR_OUT_I32_RAW) {
        v4f sw;
        if (p.w_gran == CR_GRAN_TENSOR) sw = v4f{sw_t, sw_t, sw_t, sw_t};
        else sw = *reinterpret_cast<const v4f*>(p.w_scales + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (float)raw[e] * (sa * sw[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = 0.f;
      }
      finish_block<OUT>(p, m, n, mb, l, y, raw);
    }
  }
  }
}

// ---------------------------------------------------------------------------
// Small-M kernel (M <= 64): weight streaming, bound by the weight bytes.
// A block owns 16 output channels; its SK_WAVES waves take the 64-deep
// k-tiles round robin, each issuing the loads of up to 4 k-tiles before
// its first matrix op (at K = 3072 one round of loads covers the whole K);
// every fragment is a contiguous 512-byte run read straight from global
// memory; partial sums are reduced through LDS in a fixed order.
// ---------------------------------------------------------------------------
constexpr int SK_WAVES = 16;

template <int FM, int ACT, bool A_TILED, bool GROUPED, int OUT>
__global__ __launch_bounds__(SK_WAVES * 64) void gemm_w4a4_skinny_kernel(GemmParams p) {
  constexpr bool GRP = GROUPED && OUT != CR_OUT_I32_RAW;
  constexpr int SH = (ACT == ACT_S4) ? 8 : 4;
  constexpr int U = (GRP && FM == 4) ? 3 : 4;   // k-tiles in flight per wave (register budget of 1024 threads)
  constexpr int NW = SK_WAVES;
  __shared__ __attribute__((aligned(16))) int red[NW][FM][64][4];
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t K = p.K;
  const int nkt = (int)(K / 64);
  const int64_t G = K / 64;

  int64_t mrow[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) mrow[i] = imin64((int64_t)(i * 16 + (l & 15)), p.M - 1);

  v4i acc[FM];
  float yacc[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    acc[i] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) yacc[i][e] = 0.f;
  }
  const uint8_t* wbase = p.w + (n0 >> 7) * G * 4096 + ((n0 & 127) >> 4) * 512 + l * 8;

  for (int kt0 = wave * U; kt0 < nkt; kt0 += NW * U) {
    u32x2 wr[U], ar[U][FM];
    float sa[U][FM];
    v4f sw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = kt0 + u;
      if (kt >= nkt) break;
      wr[u] = *reinterpret_cast<const u32x2*>(wbase + (int64_t)kt * 4096);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (A_TILED)
          ar[u][i] = *reinterpret_cast<const u32x2*>(p.a + ((int64_t)i * G + kt) * 512 + l * 8);
        else
          ar[u][i] = *reinterpret_cast<const u32x2*>(p.a + mrow[i] * (K / 2) + kt * 32 + (l >> 4) * 8);
        if constexpr (GRP) sa[u][i] = p.a_scales[mrow[i] * G + kt];
      }
      if constexpr (GRP) {
        const int64_t n = n0 + (l >> 4) * 4;
        sw[u] = *reinterpret_cast<const v4f*>(p.w_scales + ((n >> 7) * G + kt) * 128 + (n & 127));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = kt0 + u;
      if (kt >= nkt) break;
      const v4i wv = widen_s4x16(wr[u]);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const v4i av = widen_a4<ACT>(ar[u][i]);
        if constexpr (GRP) {
          v4i pp = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv, av, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            yacc[i][e] = __builtin_fmaf((float)(pp[e] >> SH) * sw[u][e], sa[u][i], yacc[i][e]);
        } else {
          acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv, av, acc[i], 0, 0, 0);
        }
      }
    }
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][i][l][e] = GRP ? __float_as_int(yacc[i][e]) : acc[i][e];
  __syncthreads();
  if (wave < FM) {
    const int i = wave;
    float y[4];
    int raw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (GRP) {
        float t = __int_as_float(red[0][i][l][e]);
#pragma unroll
        for (int w = 1; w < NW; ++w) t += __int_as_float(red[w][i][l][e]);
        y[e] = t;
        raw[e] = 0;
      } else {
        int t = red[0][i][l][e];
#pragma unroll
        for (int w = 1; w < NW; ++w) t += red[w][i][l][e];
        raw[e] = t >> SH;
      }
    }
    const int64_t mb = i * 16;
    const int64_t m = mb + (l & 15);
    const int64_t n = n0 + (l >> 4) * 4;
    if constexpr (!GRP && OUT != CR_OUT_I32_RAW) {
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
      for (int e = 0; e < 4; ++e) y[e] = (float)raw[e] * (sa * sw[e]);
    } else if constexpr (!GRP) {
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = 0.f;
    }
    finish_block<OUT>(p, m, n, mb, l, y, raw);
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <int ACT, bool AT, bool GROUPED, int OUT>
static hipError_t launch_w4a4_kind(const GemmParams& p, hipStream_t s) {
  if (p.M <= 64) {
    const int fm = (int)((p.M + 15) / 16);
    const dim3 grid((unsigned)(p.N / 16));
    switch (fm) {
      case 1: hipLaunchKernelGGL((gemm_w4a4_skinny_kernel<1, ACT, AT, GROUPED, OUT>), grid, dim3(SK_WAVES * 64), 0, s, p); break;
      case 2: hipLaunchKernelGGL((gemm_w4a4_skinny_kernel<2, ACT, AT, GROUPED, OUT>), grid, dim3(SK_WAVES * 64), 0, s, p); break;
      case 3: hipLaunchKernelGGL((gemm_w4a4_skinny_kernel<3, ACT, AT, GROUPED, OUT>), grid, dim3(SK_WAVES * 64), 0, s, p); break;
      default: hipLaunchKernelGGL((gemm_w4a4_skinny_kernel<4, ACT, AT, GROUPED, OUT>), grid, dim3(SK_WAVES * 64), 0, s, p); break;
    }
    return hipGetLastError();
  }
  if constexpr (AT) {
    constexpr bool GRPK = GROUPED && OUT != CR_OUT_I32_RAW;
    const int64_t tiles = ((p.M + LDS_BM - 1) / LDS_BM) * (p.N / LDS_BN);
    hipLaunchKernelGGL((gemm_w4a4_lds_kernel<ACT, OUT, GRPK>), dim3((unsigned)tiles), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  // 128 x 128 tiles, two blocks per CU (measured on MI355X at M=4096,
  // N=K=3072: 128 x 192 at one block per CU is 25% slower). The 64-group
  // epilogue keeps a float accumulator beside the integer one and would
  // spill within the two-block register budget, so it runs one block per CU.
  constexpr bool GRP = GROUPED && OUT != CR_OUT_I32_RAW;
  constexpr int MINB = GRP ? 1 : 2;
  const int64_t t128 = ((p.M + 127) / 128) * (p.N / 128);
  hipLaunchKernelGGL((gemm_w4a4_kernel<128, 128, 2, 2, MINB, ACT, AT, GROUPED, OUT>), dim3((unsigned)t128), dim3(256),
                     0, s, p);
  return hipGetLastError();
}

template <int ACT, bool AT, bool GROUPED>
static hipError_t launch_w4a4_out(const GemmParams& p, hipStream_t s) {
  switch (p.out_type) {
    case CR_OUT_BF16: return launch_w4a4_kind<ACT, AT, GROUPED, CR_OUT_BF16>(p, s);
    case CR_OUT_F32: return launch_w4a4_kind<ACT, AT, GROUPED, CR_OUT_F32>(p, s);
    default: return launch_w4a4_kind<ACT, AT, GROUPED, CR_OUT_I32_RAW>(p, s);
  }
}

template <int ACT, bool AT>
static hipError_t launch_w4a4_grp(const GemmParams& p, hipStream_t s) {
  return p.grouped ? launch_w4a4_out<ACT, AT, true>(p, s) : launch_w4a4_out<ACT, AT, false>(p, s);
}

hipError_t launch_gemm_w4a4(const GemmParams& p, hipStream_t s) {
  if (p.act == ACT_U4) return p.a_tiled ? launch_w4a4_grp<ACT_U4, true>(p, s) : launch_w4a4_grp<ACT_U4, false>(p, s);
  return p.a_tiled ? launch_w4a4_grp<ACT_S4, true>(p, s) : launch_w4a4_grp<ACT_S4, false>(p, s);
}

}  // namespace cr
