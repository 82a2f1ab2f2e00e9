// INT8 x INT8 tensorwise GEMM of the ConvRot low-bit linear (gfx950): int8
// activations x natural int8 weights. The kernel templates are generic over
// the operand kinds; only the INT8 instantiation is dispatched (the W4A4
// kernels live in gemm_w4a4.hip).
//
// "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4" page, Measurements: a fused
// INT4 matmul with a rank-one (s_a x s_w) rescale; intro: INT8 tensorwise
// layers in the same model. "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)",
// Key Technical Optimizations and Kernel Engineering: tile-packed weights,
// LoRA-up fused into the epilogue, scales staged in shared memory, unsigned
// post-GELU activations with a +0.171875 shift.
//
// gfx950 has no int4 matrix instruction, so int4 codes are widened exactly to
// int8 in registers: a signed nibble q becomes the byte 16*q (a mask, no
// shift), so one v_mfma_i32_16x16x64_i8 accumulates 256 * sum(qa*qw) (or
// 16 * sum for unsigned activation bytes), and the true integer is recovered
// by an exact arithmetic right shift.
//
// Operand roles: the MFMA A operand is the weight (16 output channels n),
// the B operand the activation (16 tokens m). Each lane of the 16x16 result
// then holds one token and four consecutive output channels, so a bf16
// result leaves as one 8-byte store.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace cr {

typedef float v2f_i __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_i __attribute__((ext_vector_type(2)));

template <int ACT>
CR_DEV v4i widen_act(const uint8_t* lds) {
  if constexpr (ACT == ACT_I8) {
    return *reinterpret_cast<const v4i*>(lds);
  } else {
    u32x2 x = *reinterpret_cast<const u32x2*>(lds);
    return ACT == ACT_S4 ? widen_s4x16(x) : widen_u4(x);
  }
}
// The int4 widening above emits a lane's 16 k-values in the order (even k of
// the first 8, odd k of the first 8, even of the second 8, odd of the second
// 8). Int8 activation codes that meet such weights are put in the same order
// (a dot product does not depend on the order of its terms).
CR_DEV v4i i8_in_s4_order(v4i a) {
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm((uint32_t)a[1], (uint32_t)a[0], 0x06040200u);
  r[1] = (int)__builtin_amdgcn_perm((uint32_t)a[1], (uint32_t)a[0], 0x07050301u);
  r[2] = (int)__builtin_amdgcn_perm((uint32_t)a[3], (uint32_t)a[2], 0x06040200u);
  r[3] = (int)__builtin_amdgcn_perm((uint32_t)a[3], (uint32_t)a[2], 0x07050301u);
  return r;
}
template <int ACT, int WGT>
CR_DEV v4i act_operand(const uint8_t* lds) {
  const v4i a = widen_act<ACT>(lds);
  if constexpr (ACT == ACT_I8 && WGT == WGT_S4T) return i8_in_s4_order(a);
  else return a;
}

template <int WGT>
CR_DEV v4i widen_wgt(const uint8_t* lds) {
  if constexpr (WGT == WGT_I8N) {
    return *reinterpret_cast<const v4i*>(lds);
  } else {
    return widen_s4x16(*reinterpret_cast<const u32x2*>(lds));
  }
}
// right shift that recovers sum(qa*qw) from the widened accumulation
template <int ACT, int WGT>
constexpr int acc_shift() {
  return (ACT == ACT_S4 ? 4 : 0) + (WGT == WGT_S4T ? 4 : 0);
}

CR_DEV v4i mfma_i8(v4i a, v4i b, v4i c) { return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0); }

// ---------------------------------------------------------------------------
// Large-M kernel: BM x BN block tile, WM x WN waves, BK = 128 per stage
// (two 64-deep k-tiles), double-buffered LDS. LDS operand layout per stage:
// [k-tile][16-row block][64 lanes][frag bytes], i.e. fragment order, so every
// fragment read is 64 consecutive 8/16-byte words.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int ACT, int WGT, bool GROUPED, int OUT>
__global__ __launch_bounds__(WM * WN * 64) void gemm_big_kernel(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int AFB = (ACT == ACT_I8) ? 16 : 8;
  constexpr int WFB = (WGT == WGT_I8N) ? 16 : 8;
  constexpr int A_ST = 2 * (BM / 16) * 64 * AFB;
  constexpr int W_ST = 2 * (BN / 16) * 64 * WFB;
  constexpr bool GRP = GROUPED && OUT != CR_OUT_I32_RAW;
  constexpr int S_ST = GRP ? 2 * (BM + BN) * 4 : 0;
  constexpr int STAGE = A_ST + W_ST + S_ST;
  constexpr int SH = acc_shift<ACT, WGT>();
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // block -> tile, XCD-aware: consecutive block ids land on different XCDs,
  // so give each XCD a contiguous range of tiles, ordered in bands of 8 tile
  // rows walked column by column (neighbouring tiles share operands in L2).
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

  // ---- global -> register prefetch descriptors ----
  constexpr int A_PIECES = (ACT == ACT_I8) ? BM * 8 : BM * 4;    // 16-byte pieces per stage
  constexpr int W_PIECES = (WGT == WGT_I8N) ? BN * 8 : BN * 4;
  constexpr int PA = (A_PIECES + NT - 1) / NT;
  constexpr int PW = (W_PIECES + NT - 1) / NT;
  u32x4 ra[PA], rw[PW];
  float rs[GRP ? (2 * (BM + BN) + NT - 1) / NT : 1];

  auto gload = [&](int kb) {
    const int64_t k0 = (int64_t)kb * 128;
#pragma unroll
    for (int j = 0; j < PA; ++j) {
      int pc = tid + j * NT;
      if (pc < A_PIECES) {
        if constexpr (ACT == ACT_I8) {
          int row = pc >> 3, part = pc & 7;
          int64_t m = imin64(m0 + row, p.M - 1);
          ra[j] = *reinterpret_cast<const u32x4*>(p.a + m * K + k0 + part * 16);
        } else {
          int row = pc >> 2, part = pc & 3;
          int64_t m = imin64(m0 + row, p.M - 1);
          ra[j] = *reinterpret_cast<const u32x4*>(p.a + m * (K / 2) + k0 / 2 + part * 16);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      int pc = tid + j * NT;
      if (pc < W_PIECES) {
        if constexpr (WGT == WGT_I8N) {
          int row = pc >> 3, part = pc & 7;
          rw[j] = *reinterpret_cast<const u32x4*>(p.w + (n0 + row) * K + k0 + part * 16);
        } else {
          int chunk = pc >> 5, off = (pc & 31) * 16;
          int kt = chunk / (BN / 16), nb = chunk % (BN / 16);
          int64_t n = n0 + 16 * nb;
          rw[j] = *reinterpret_cast<const u32x4*>(p.w + ((n >> 7) * (K / 64) + k0 / 64 + kt) * 4096 +
                                                  ((n & 127) >> 4) * 512 + off);
        }
      }
    }
    if constexpr (GRP) {
      const int64_t G = K / 64;
#pragma unroll
      for (int j = 0; j < (int)(sizeof(rs) / sizeof(float)); ++j) {
        int idx = tid + j * NT;
        if (idx < 2 * BM) {
          int kt = idx / BM, r = idx % BM;
          int64_t m = imin64(m0 + r, p.M - 1);
          rs[j] = p.a_scales[m * G + kb * 2 + kt];
        } else if (idx < 2 * (BM + BN)) {
          int q = idx - 2 * BM;
          int kt = q / BN, c = q % BN;
          int64_t n = n0 + c;
          rs[j] = p.w_scales[((n >> 7) * G + kb * 2 + kt) * 128 + (n & 127)];
        }
      }
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* As = smem + buf * STAGE;
    uint8_t* Ws = As + A_ST;
#pragma unroll
    for (int j = 0; j < PA; ++j) {
      int pc = tid + j * NT;
      if (pc < A_PIECES) {
        if constexpr (ACT == ACT_I8) {
          int row = pc >> 3, part = pc & 7;
          int kt = part >> 2, c = part & 3;
          *reinterpret_cast<u32x4*>(As + ((kt * (BM / 16) + (row >> 4)) * 64 + c * 16 + (row & 15)) * 16) = ra[j];
        } else {
          int row = pc >> 2, part = pc & 3;
          int kt = part >> 1, c = (part & 1) * 2;
          uint8_t* base = As + (kt * (BM / 16) + (row >> 4)) * 512;
          *reinterpret_cast<u32x2*>(base + (c * 16 + (row & 15)) * 8) = u32x2{ra[j][0], ra[j][1]};
          *reinterpret_cast<u32x2*>(base + ((c + 1) * 16 + (row & 15)) * 8) = u32x2{ra[j][2], ra[j][3]};
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      int pc = tid + j * NT;
      if (pc < W_PIECES) {
        if constexpr (WGT == WGT_I8N) {
          int row = pc >> 3, part = pc & 7;
          int kt = part >> 2, c = part & 3;
          *reinterpret_cast<u32x4*>(Ws + ((kt * (BN / 16) + (row >> 4)) * 64 + c * 16 + (row & 15)) * 16) = rw[j];
        } else {
          *reinterpret_cast<u32x4*>(Ws + pc * 16) = rw[j];
        }
      }
    }
    if constexpr (GRP) {
      float* Ss = reinterpret_cast<float*>(Ws + W_ST);
#pragma unroll
      for (int j = 0; j < (int)(sizeof(rs) / sizeof(float)); ++j) {
        int idx = tid + j * NT;
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

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
    const uint8_t* As = smem + buf * STAGE;
    const uint8_t* Ws = As + A_ST;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      v4i wv[FN], av[FM];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        wv[j] = widen_wgt<WGT>(Ws + ((kt * (BN / 16) + wn * FN + j) * 64 + l) * WFB);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        av[i] = act_operand<ACT, WGT>(As + ((kt * (BM / 16) + wm * FM + i) * 64 + l) * AFB);
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
            v4i pp = mfma_i8(wv[j], av[i], v4i{0, 0, 0, 0});
#pragma unroll
            for (int e = 0; e < 4; ++e)
              yacc[i][j][e] = __builtin_fmaf((float)(pp[e] >> SH) * sw[j][e], sa[i], yacc[i][j][e]);
          }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma_i8(wv[j], av[i], acc[i][j]);
      }
    }
    if (kb + 1 < nkb) lstore(buf ^ 1);
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
// Small-M kernel (M <= 64): weight streaming. A block owns 16 output channels;
// its 4 waves split the 64-deep k-tiles round robin, fragments come straight
// from global memory (the tile-packed weight fragment is 512 contiguous
// bytes), partial sums are reduced through LDS in a fixed order.
// ---------------------------------------------------------------------------
template <int FM, int ACT, int WGT, bool GROUPED, int OUT>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmParams p) {
  constexpr bool GRP = GROUPED && OUT != CR_OUT_I32_RAW;
  constexpr int SH = acc_shift<ACT, WGT>();
  constexpr int U = 4;
  __shared__ __attribute__((aligned(16))) int red[4][FM][64][4];
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

  for (int kt0 = wave * U; kt0 < nkt; kt0 += 4 * U) {
    u32x4 wr[U], ar[U][FM];
    float sa[U][FM];
    v4f sw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = kt0 + u;
      if (kt >= nkt) break;
      if constexpr (WGT == WGT_I8N) {
        wr[u] = *reinterpret_cast<const u32x4*>(p.w + (n0 + (l & 15)) * K + kt * 64 + (l >> 4) * 16);
      } else {
        u32x2 t = *reinterpret_cast<const u32x2*>(p.w + ((n0 >> 7) * (K / 64) + kt) * 4096 +
                                                  ((n0 & 127) >> 4) * 512 + l * 8);
        wr[u] = u32x4{t[0], t[1], 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (ACT == ACT_I8) {
          ar[u][i] = *reinterpret_cast<const u32x4*>(p.a + mrow[i] * K + kt * 64 + (l >> 4) * 16);
        } else {
          u32x2 t = *reinterpret_cast<const u32x2*>(p.a + mrow[i] * (K / 2) + kt * 32 + (l >> 4) * 8);
          ar[u][i] = u32x4{t[0], t[1], 0u, 0u};
        }
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
      v4i wv;
      if constexpr (WGT == WGT_I8N) wv = __builtin_bit_cast(v4i, wr[u]);
      else wv = widen_s4x16(u32x2{wr[u][0], wr[u][1]});
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        v4i av;
        if constexpr (ACT == ACT_I8 && WGT == WGT_S4T) av = i8_in_s4_order(__builtin_bit_cast(v4i, ar[u][i]));
        else if constexpr (ACT == ACT_I8) av = __builtin_bit_cast(v4i, ar[u][i]);
        else if constexpr (ACT == ACT_S4) av = widen_s4x16(u32x2{ar[u][i][0], ar[u][i][1]});
        else av = widen_u4(u32x2{ar[u][i][0], ar[u][i][1]});
        if constexpr (GRP) {
          v4i pp = mfma_i8(wv, av, v4i{0, 0, 0, 0});
#pragma unroll
          for (int e = 0; e < 4; ++e)
            yacc[i][e] = __builtin_fmaf((float)(pp[e] >> SH) * sw[u][e], sa[u][i], yacc[i][e]);
        } else {
          acc[i] = mfma_i8(wv, av, acc[i]);
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
        y[e] = ((__int_as_float(red[0][i][l][e]) + __int_as_float(red[1][i][l][e])) +
                __int_as_float(red[2][i][l][e])) + __int_as_float(red[3][i][l][e]);
        raw[e] = 0;
      } else {
        int s = red[0][i][l][e] + red[1][i][l][e] + red[2][i][l][e] + red[3][i][l][e];
        raw[e] = s >> SH;
      }
    }
    const int64_t mb = i * 16;
    const int64_t m = mb + (l & 15);
    const int64_t n = n0 + (l >> 4) * 4;
    if constexpr (!GRP && OUT != CR_OUT_I32_RAW) {
      const int64_t mc = m < p.M ? m : p.M - 1;
      float sa = (p.a_gran == CR_GRAN_TENSOR) ? p.a_scales[0] : p.a_scales[mc];
      v4f sw;
      if (p.w_gran == CR_GRAN_TENSOR) {
        float t = p.w_scales[0];
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
// INT8 main kernel (M > 64): v_mfma_i32_32x32x32_i8, whose operand is 16
// consecutive k-bytes of one row per lane (lanes 0-31 k 0..15, lanes 32-63
// k 16..31 of the 32-deep step), so both operands keep their natural
// row-major int8 layout all the way into the matrix cores.
// Block BM tokens x BN channels of waves with TM x TN blocks of 32 x 32
// (int32 accumulators in VGPRs): 256 x 128 of 4 waves of 128 x 64, two
// blocks per CU with a 3-stage ring or three with a 2-stage ring, or, for
// mid-size M, 64 x 64 of 4 waves of 32 x 32 (see launch_int8_lds). Each
// 64-deep k-tile is one stage of the LDS ring filled by 16-byte
// global_load_lds pieces (1 KB wave-loads of 16 rows): BM activation rows
// and BN weight rows of 64 bytes, the four 16-byte slots of a row
// XOR-swizzled by the row index so that the 32 rows of a fragment read land
// on distinct banks. Each wave waits (vmcnt) only for the stage it is about
// to use, then one bare s_barrier per stage.
// Operand roles: A = weights (32 channels), B = activations (32 tokens), so a
// lane ends with one token and 4 consecutive channels per 8 accumulators:
// one activation scale and one 8-byte bf16 (16-byte int32 / float) store.
// ---------------------------------------------------------------------------
typedef const void __attribute__((address_space(1)))* gas_ptr_i8;
typedef void __attribute__((address_space(3)))* las_ptr_i8;

template <int N>
CR_DEV void wait_vmcnt_i8() {   // s_waitcnt vmcnt(N), other counters untouched
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16-byte slot of k-chunk c (0..3) in row r of a 64-byte stage row
CR_DEV int i8_slot(int r, int c) { return c ^ (((r >> 1) ^ (r >> 3)) & 3); }

// TW: per-tensor weight scale and no bias (the epilogue keeps one scalar
// instead of per-channel scale and bias vectors)
template <int OUT, int NS, int MINB, bool TW, int BM = 256, int BN = 128, int TM = 4, int TN = 2>
__global__ __launch_bounds__((BM / (32 * TM)) * (BN / (32 * TN)) * 64, MINB) void gemm_int8_lds_kernel(GemmParams p) {
  static_assert(NS == 2 || NS == 3, "two or three stages");
  static_assert(BM % (32 * TM) == 0 && BN % (32 * TN) == 0, "whole wave tiles");
  constexpr int WN = BN / (32 * TN);                 // waves along the channels
  constexpr int NW = (BM / (32 * TM)) * WN;
  constexpr int A_ST = BM * 64, W_ST = BN * 64, STAGE = A_ST + W_ST;
  constexpr int NA = BM / 16, NL = (BM + BN) / 16;   // 1 KB wave-loads per stage (activation part first)
  constexpr int LPW = (NL + NW - 1) / NW;            // wave-loads of the busiest waves
  constexpr int NHI = NL - (LPW - 1) * NW;           // waves 0 .. NHI-1 take LPW, the others LPW - 1
  // whole-row bf16 stores through LDS for the 256 x 128 block (pairs of
  // 32-row blocks, 64 channels per wave); other shapes store 8-byte pieces
  constexpr bool LDS_EPI = (TM % 2 == 0) && TN == 2;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem_i8[];
  uint8_t* smem = smem_i8;

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

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
  const int nst = (int)(K / 64);

  // wave-load idx = wave + NW j fills stage bytes [idx KB, +1 KB): rows
  // 16 idx + l / 4 of the activation part (idx < NA), else of the weight
  // part, slot l % 4
  const uint8_t* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int idx = min(wave + NW * j, NL - 1);
    if (idx < NA) {
      const int r = 16 * idx + (l >> 2);
      src[j] = p.a + imin64(m0 + r, p.M - 1) * K + 16 * i8_slot(r, l & 3);   // rows past M: never stored
    } else {
      const int r = 16 * (idx - NA) + (l >> 2);
      src[j] = p.w + (n0 + r) * K + 16 * i8_slot(r, l & 3);
    }
  }
  auto issue = [&](int s) {
    uint8_t* st = smem + (s % NS) * STAGE;
    const int64_t k0 = (int64_t)s * 64;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      if (j < LPW - 1 || wave < NHI)
        __builtin_amdgcn_global_load_lds((gas_ptr_i8)(src[j] + k0), (las_ptr_i8)(st + (wave + NW * j) * 1024), 16,
                                         0, 0);
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  // fragment rows: activations wm*32*TM + 32 i + l % 32, weights wn*32*TN + 32 j + l % 32
  const int lr = l & 31, h = l >> 5;
  const int fl = ((lr >> 1) ^ (lr >> 3)) & 3;
  int abase[2], wbase[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c = 2 * ks + h;                       // 16-byte k-chunk of this lane in step ks
    abase[ks] = (wm * 32 * TM + lr) * 64 + 16 * (c ^ fl);
    wbase[ks] = A_ST + (wn * 32 * TN + lr) * 64 + 16 * (c ^ fl);
  }

  issue(0);
  if (NS == 3 && nst > 1) issue(1);
  for (int s = 0; s < nst; ++s) {
    if (NS == 3 && s + 1 < nst) {                    // stage s + 1 may stay in flight
      if (wave < NHI) wait_vmcnt_i8<LPW>();
      else wait_vmcnt_i8<LPW - 1>();
    } else {
      wait_vmcnt_i8<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (s + NS - 1 < nst) issue(s + NS - 1);
    const uint8_t* st = smem + (s % NS) * STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i fa[TM], fw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = *reinterpret_cast<const v4i*>(st + abase[ks] + i * 2048);
#pragma unroll
      for (int j = 0; j < TN; ++j) fw[j] = *reinterpret_cast<const v4i*>(st + wbase[ks] + j * 2048);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[j], fa[i], acc[i][j], 0, 0, 0);
    }
  }

  // lane owns token m = l % 32 of each 32 x 32 block and channels 8 (r / 4) + 4 h + r % 4.
  // Every epilogue input is loaded before the first store (a load between
  // stores would make each later store wait for the earlier ones).
  float sa[TM];
  v4f sw[TN][4];
  u32x2 bw[TN][4];
  if constexpr (OUT != CR_OUT_I32_RAW) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = imin64(m0 + wm * 32 * TM + i * 32 + lr, p.M - 1);
      sa[i] = p.a_scales[p.a_gran == CR_GRAN_TENSOR ? 0 : m];
    }
    const bool wrow = p.w_gran != CR_GRAN_TENSOR;
    const float sw_t = p.w_scales[0];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (TW) {
          sw[j][q] = v4f{sw_t, sw_t, sw_t, sw_t};
          bw[j][q] = u32x2{0u, 0u};
        } else {
          const int64_t n = n0 + (wn * TN + j) * 32 + 8 * q + 4 * h;
          sw[j][q] = wrow ? *reinterpret_cast<const v4f*>(p.w_scales + n) : v4f{sw_t, sw_t, sw_t, sw_t};
          bw[j][q] = p.bias ? *reinterpret_cast<const u32x2*>(p.bias + n) : u32x2{0u, 0u};
        }
      }
  }
  if constexpr (OUT == CR_OUT_BF16 && LDS_EPI) {
    // bf16 (v_cvt_pk_bf16_f32, half to even) through LDS in pieces of 64
    // token rows per wave, so that every store writes whole 128-byte output
    // rows instead of 8-byte pieces spread over 32 rows
    constexpr int RS = 144;                          // LDS row stride of a half tile, 16-byte aligned
    static_assert(NW * 64 * RS <= NS * STAGE, "half tiles fit the stage buffers");
    __syncthreads();                                 // every wave is done with the stage buffers
    uint8_t* tile = smem + wave * (64 * RS);
#pragma unroll
    for (int hh = 0; hh < TM / 2; ++hh) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = 2 * hh + ii;
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              y[e] = (float)acc[i][j][4 * q + e] * (sa[i] * sw[j][q][e]) +
                     ((e & 1) ? bf16_hi(bw[j][q][e >> 1]) : bf16_lo(bw[j][q][e >> 1]));
            const v2bf_i lo = __builtin_convertvector((v2f_i){y[0], y[1]}, v2bf_i);
            const v2bf_i hi = __builtin_convertvector((v2f_i){y[2], y[3]}, v2bf_i);
            *reinterpret_cast<u32x2*>(tile + (ii * 32 + lr) * RS + (j * 32 + 8 * q + 4 * h) * 2) =
                u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          }
      __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0): this wave's half tile is written
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) {
        const int r = (l >> 3) + 8 * qq;
        const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * RS + (l & 7) * 16);
        const int64_t m = m0 + wm * 32 * TM + hh * 64 + r;
        if (m < p.M)
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldc + n0 + wn * 64 + (l & 7) * 8) = v;
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = n0 + (wn * TN + j) * 32 + 8 * q + 4 * h;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * 32 * TM + i * 32 + lr;
        if (m >= p.M) continue;
        if constexpr (OUT == CR_OUT_I32_RAW) {
          *reinterpret_cast<v4i*>(reinterpret_cast<int32_t*>(p.out) + m * p.ldc + n) =
              v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        } else {
          const float b[4] = {bf16_lo(bw[j][q][0]), bf16_hi(bw[j][q][0]), bf16_lo(bw[j][q][1]), bf16_hi(bw[j][q][1])};
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = (float)acc[i][j][4 * q + e] * (sa[i] * sw[j][q][e]) + b[e];
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
}

template <int OUT, int NS, int MINB, bool TW, int BM = 256, int BN = 128, int TM = 4, int TN = 2>
static hipError_t launch_int8_lds_cfg(const GemmParams& p, int64_t tiles, hipStream_t s) {
  constexpr int lds = NS * (BM + BN) * 64;
  constexpr int threads = (BM / (32 * TM)) * (BN / (32 * TN)) * 64;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)gemm_int8_lds_kernel<OUT, NS, MINB, TW, BM, BN, TM, TN>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemm_int8_lds_kernel<OUT, NS, MINB, TW, BM, BN, TM, TN>), dim3((unsigned)tiles),
                     dim3(threads), lds, s, p);
  return hipGetLastError();
}

// Three-stage ring and two blocks per CU; when the tiles number more than
// two but at most three per CU (8192 x 3072: 768 tiles), a two-stage ring and
// three blocks per CU, so that every tile runs in the first round (two
// blocks per CU leave the second round of 256 tiles on half the slots).
template <int OUT>
static hipError_t launch_int8_lds(const GemmParams& p, hipStream_t s) {
  const int64_t tiles = ((p.M + 255) / 256) * (p.N / 128);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  // mid-size M (e.g. 512 text tokens x 3072: 48 blocks of 256 x 128): 64 x 64
  // blocks of four 32 x 32 waves fill the chip instead
  if (cus > 0 && tiles < cus) {
    const int64_t t64 = ((p.M + 63) / 64) * (p.N / 64);
    return launch_int8_lds_cfg<OUT, 3, 4, false, 64, 64, 1, 1>(p, t64, s);
  }
  // per-channel weight scales or a bias keep more epilogue registers: those
  // stay at two blocks per CU (three would spill)
  const bool tw = OUT == CR_OUT_I32_RAW || (p.w_gran == CR_GRAN_TENSOR && !p.bias);
  if (!tw) return launch_int8_lds_cfg<OUT, 3, 2, false>(p, tiles, s);
  if (cus > 0 && tiles > 2 * cus && tiles <= 3 * cus) return launch_int8_lds_cfg<OUT, 2, 3, true>(p, tiles, s);
  return launch_int8_lds_cfg<OUT, 3, 2, true>(p, tiles, s);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <int ACT, int WGT, bool GROUPED, int OUT>
static hipError_t launch_kind(const GemmParams& p, hipStream_t s) {
  if (p.M <= 64) {
    const int fm = (int)((p.M + 15) / 16);
    dim3 grid((unsigned)(p.N / 16));
    switch (fm) {
      case 1: hipLaunchKernelGGL((gemm_skinny_kernel<1, ACT, WGT, GROUPED, OUT>), grid, dim3(256), 0, s, p); break;
      case 2: hipLaunchKernelGGL((gemm_skinny_kernel<2, ACT, WGT, GROUPED, OUT>), grid, dim3(256), 0, s, p); break;
      case 3: hipLaunchKernelGGL((gemm_skinny_kernel<3, ACT, WGT, GROUPED, OUT>), grid, dim3(256), 0, s, p); break;
      default: hipLaunchKernelGGL((gemm_skinny_kernel<4, ACT, WGT, GROUPED, OUT>), grid, dim3(256), 0, s, p); break;
    }
    return hipGetLastError();
  }
  if constexpr (ACT == ACT_I8 && WGT == WGT_I8N && !GROUPED) {
    return launch_int8_lds<OUT>(p, s);
  } else {
    constexpr int BM = 128, BN = 128;
    const int64_t tiles = ((p.M + BM - 1) / BM) * (p.N / BN);
    hipLaunchKernelGGL((gemm_big_kernel<BM, BN, 2, 2, ACT, WGT, GROUPED, OUT>), dim3((unsigned)tiles), dim3(256), 0,
                       s, p);
    return hipGetLastError();
  }
}

template <int ACT, int WGT, bool GROUPED>
static hipError_t launch_out(const GemmParams& p, hipStream_t s) {
  switch (p.out_type) {
    case CR_OUT_BF16: return launch_kind<ACT, WGT, GROUPED, CR_OUT_BF16>(p, s);
    case CR_OUT_F32: return launch_kind<ACT, WGT, GROUPED, CR_OUT_F32>(p, s);
    default: return launch_kind<ACT, WGT, GROUPED, CR_OUT_I32_RAW>(p, s);
  }
}

hipError_t launch_gemm_int(const GemmParams& p, hipStream_t s) {
  return launch_out<ACT_I8, WGT_I8N, false>(p, s);
}

// 8-bit activations x W4A4-format weights: the int4 weights widen to 16 q
// as in the W4A4 GEMM, the activation codes enter the matrix cores as they
// are, and an arithmetic shift by 4 returns the exact sum (the generic
// weight-streaming kernel for M <= 64, the register-staged one above).
hipError_t launch_gemm_a8w4(const GemmParams& p, hipStream_t s) {
  return launch_out<ACT_I8, WGT_S4T, false>(p, s);
}

}  // namespace cr
