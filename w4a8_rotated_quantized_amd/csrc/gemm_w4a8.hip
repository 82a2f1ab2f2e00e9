// W4A8 GEMM (gfx950): per-token int8 activations x asymmetric uint4 weights
// with a float16 scale and a uint4 zero point per 16 input channels.
//
// "Qwen-Image-Edit-2511-W4A8-ConvRot" card, build table and file layout
// (asym_w4a8_int8, group_size 16, convrot_groupsize 256, 8-bit activations).
//
// Exact group partials on the fp16 matrix cores. Every 16-deep group is one
// v_mfma_f32_32x32x16_f16 whose operands are small integers held exactly in
// fp16: the activation codes a (|a| <= 127) and the weight codes minus their
// zero point, q - z (|q - z| <= 15). Each product and each partial sum of a
// group is an integer of magnitude <= 16 * 127 * 15 = 30480 < 2^24, so the
// float32 result is the group partial P[m, n, g] = sum_{k in g} a (q - z)
// exactly, whatever order the matrix core adds in. The outputs follow:
//   float:  acc[m, n] += s_w[n, g] * P   (one float32 FMA per output and
//           group, groups in increasing k), y = s_a[m] * acc (+ low rank)
//           (+ bias);
//   int32:  acc[m, n] += P as an integer (the exact sum_k a (q - z)).
// Both come from the same partials, so the exact int32 output checks the
// products that the float outputs scale.
//
// Operand roles: MFMA A = activations (32 tokens x 16 k), B = weights (16 k x
// 32 channels). Lane l of a 32 x 32 result holds channel l % 32 and, in
// register r, token 8 (r / 4) + 4 (l / 32) + r % 4: the group scale s_w[n, g]
// is one value per lane.
//
// Activation codes arrive either as int8 [M, K] (each lane turns its 8 bytes
// into fp16 in registers: a ^ 0x80 is the byte a + 128, 0x64 placed above it
// is the fp16 value 1024 + (a + 128), and one packed subtraction of 1152 is
// exact) or as the fp16 values of the same codes ([M, K], CR_LAYOUT_F16,
// written by the quantizer), which the kernel uses as they are.
// Weights (tile-packed, 4096-byte tiles of 128 channels x 64 k): a lane's
// word holds the 8 nibbles of its k-half; 0x64 above a nibble is the fp16
// value 1024 + q and one packed subtraction of 1024 + z gives q - z exactly.
//
// Block 256 x 128 outputs, 4 waves. A stage is one 64-deep k-tile of the
// block's activation rows (16-byte slots XOR-swizzled per row so that reads
// of consecutive rows hit distinct LDS banks), its weight tile, fp16 scales
// and zero points, loaded straight into LDS by 16-byte global_load_lds.
#include "common.h"
#include "kernels.h"

namespace cr {

typedef _Float16 v8h_ __attribute__((ext_vector_type(8)));
typedef _Float16 v2h_ __attribute__((ext_vector_type(2)));
typedef float v2f_ __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef const void __attribute__((address_space(1)))* gas_ptr_w8;
typedef void __attribute__((address_space(3)))* las_ptr_w8;

CR_DEV uint32_t h2_sub(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h_, a) - __builtin_bit_cast(v2h_, b));
}

template <int N>
CR_DEV void w8_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// int8 activation stage, rows of 64 bytes (4 slots of 16): slot of group g in row r
CR_DEV int w8_slot(int r, int g) { return g ^ (((r >> 1) ^ (r >> 3)) & 3); }

// at most `ahead` later stages (L loads each) of this wave left in flight
template <int L>
CR_DEV void w8_wait_stage(int ahead) {
  if (ahead >= 2) w8_wait_vm<2 * L>();
  else if (ahead == 1) w8_wait_vm<L>();
  else w8_wait_vm<0>();
}

// 8 int8 codes (two words, k order) -> 8 exact fp16 values
CR_DEV v8h_ a8_to_h(uint32_t x0, uint32_t x1) {
  const uint32_t u0 = x0 ^ 0x80808080u, u1 = x1 ^ 0x80808080u;
  const uint32_t off = 0x64806480u;                     // fp16 pair (1152, 1152)
  return __builtin_bit_cast(v8h_, u32x4{h2_sub(__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u), off),
                                        h2_sub(__builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u), off),
                                        h2_sub(__builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u), off),
                                        h2_sub(__builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u), off)});
}

// one lane's weight word (byte i = q[i] | q[4 + i] << 4) and zero point -> 8 exact fp16 values q - z
CR_DEV v8h_ w4_to_h(uint32_t x, uint32_t z) {
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
  const uint32_t zz = 0x64006400u | z | (z << 16);      // fp16 pair (1024 + z, 1024 + z)
  return __builtin_bit_cast(v8h_, u32x4{h2_sub(__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u), zz),
                                        h2_sub(__builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u), zz),
                                        h2_sub(__builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u), zz),
                                        h2_sub(__builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u), zz)});
}

// TM x TN 32 x 32 blocks per wave, WN = 4 / WM waves along the channels.
template <int TM, int TN, bool A16, int OUT>
__global__ __launch_bounds__(256, 2) void gemm_w4a8_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 128, NW = 4;
  constexpr int WN = BN / (32 * TN), WM = NW / WN;
  static_assert(WM * WN == NW && WM * TM * 32 == BM, "wave tiles cover the block");
  constexpr int AROW = A16 ? 128 : 64;                  // bytes of one activation row per stage
  constexpr int A_ST = BM * AROW;
  constexpr int W_ST = 4096, S_ST = 1024, Z_ST = 1024;  // weights, fp16 scales, zero points (+512 B copy)
  constexpr int STAGE = A_ST + W_ST + S_ST + Z_ST;
  constexpr int NS = A16 ? 2 : 3;
  constexpr int AL = A_ST / 1024 / NW;                  // activation wave-loads per wave and stage
  constexpr bool RAW = OUT == CR_OUT_I32_RAW;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem_w8[];
  uint8_t* smem = smem_w8;

  const int tid = threadIdx.x;
  const int l = tid & 63, lr = l & 31, h = l >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // block -> tile: consecutive blocks round robin over the 8 XCDs, then bands
  // of 4 tile rows walked column by column
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
  // k-tiles [k_lo, k_hi) of this launch (the whole K unless the int32 output is split)
  const int kt0 = p.k_hi > 0 ? p.k_lo : 0;
  const int nst = (p.k_hi > 0 ? p.k_hi : (int)KT) - kt0;
  const int64_t wt0 = (int64_t)tn * KT + kt0;          // first packed k-tile of this channel block

  // activation wave-load j of this wave fills stage bytes [(wave + 4 j) KB, +1 KB):
  // fp16 rows of 128 B (8 rows, slot = lane % 8 holds k-slot slot ^ (row % 8)),
  // or int8 rows of 64 B (16 rows, slot = lane % 4 holds group w8_slot(row, slot))
  // (byte offsets from the block's first row; rows past M read the last row, never stored)
  uint32_t aoff[AL];
#pragma unroll
  for (int j = 0; j < AL; ++j) {
    const int idx = wave + NW * j;
    if constexpr (A16) {
      const int r = 8 * idx + (l >> 3);
      aoff[j] = (uint32_t)((imin64(m0 + r, p.M - 1) - m0) * K * 2) + 16 * ((l & 7) ^ (r & 7));
    } else {
      const int r = 16 * idx + (l >> 2);
      aoff[j] = (uint32_t)((imin64(m0 + r, p.M - 1) - m0) * K) + 16 * w8_slot(r, l & 3);
    }
  }

  auto issue = [&](int s) {
    uint8_t* st = smem + (s % NS) * STAGE;
    const uint8_t* ga = p.a + m0 * K * (A16 ? 2 : 1) + (int64_t)(kt0 + s) * AROW;
#pragma unroll
    for (int j = 0; j < AL; ++j)
      __builtin_amdgcn_global_load_lds((gas_ptr_w8)(ga + aoff[j]), (las_ptr_w8)(st + (wave + NW * j) * 1024), 16, 0, 0);
    const int64_t tile = wt0 + s;
    __builtin_amdgcn_global_load_lds((gas_ptr_w8)(p.w + tile * 4096 + wave * 1024 + l * 16),
                                     (las_ptr_w8)(st + A_ST + wave * 1024), 16, 0, 0);
    if constexpr (!RAW) {
      if (wave == 0)
        __builtin_amdgcn_global_load_lds(
            (gas_ptr_w8)(reinterpret_cast<const uint8_t*>(p.w_scales16) + tile * 1024 + l * 16),
            (las_ptr_w8)(st + A_ST + W_ST), 16, 0, 0);
    }
    if (wave == 1)
      __builtin_amdgcn_global_load_lds((gas_ptr_w8)(p.w_zeros + tile * 512 + (l & 31) * 16),
                                       (las_ptr_w8)(st + A_ST + W_ST + S_ST), 16, 0, 0);
  };
  // loads per stage of this wave: AL + 1, plus the scales (wave 0) or zero points (wave 1)
  auto wait_stage = [&](int ahead) {
    if (wave == 1 || (!RAW && wave == 0)) w8_wait_stage<AL + 2>(ahead);
    else w8_wait_stage<AL + 1>(ahead);
  };

  // float outputs: sum_g s_w[n, g] P (one FMA per group); int32 output: the
  // partials chained through the matrix op's accumulator, exact because at
  // most 512 groups (|sum| <= 512 * 30480 < 2^24) are summed per launch
  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};

  // lane-constant parts of the fragment addresses (row % 32 = lr in every 32-row block)
  const int arow0 = (wm * TM * 32 + lr) * AROW;
  const int asw8 = ((lr >> 1) ^ (lr >> 3)) & 3;
  const int wcol0 = wn * TN;                            // first 32-channel block of this wave

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nst) issue(s);
  for (int s = 0; s < nst; ++s) {
    wait_stage(min(NS - 2, nst - 1 - s));             // this wave's loads of stage s have landed
    __builtin_amdgcn_s_barrier();                      // ... and every wave's; stage s - 1 is consumed
    if (s + NS - 1 < nst) issue(s + NS - 1);
    const uint8_t* st = smem + (s % NS) * STAGE;
    const uint8_t* Ws = st + A_ST;
    const uint16_t* Ss = reinterpret_cast<const uint16_t*>(st + A_ST + W_ST);
    const uint8_t* Zs = st + A_ST + W_ST + S_ST;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      v8h_ wf[TN];
      float sc[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int nb = wcol0 + j;
        const uint32_t x = *reinterpret_cast<const uint32_t*>(Ws + g * 1024 + nb * 256 + l * 4);
        wf[j] = w4_to_h(x, Zs[g * 128 + nb * 32 + lr]);
        if constexpr (!RAW) {
          // the scale as a float32 register: the 16 FMAs then run as plain
          // v_fmac_f32 instead of mixed-precision FMAs
          float f;
          asm("v_cvt_f32_f16 %0, %1" : "=v"(f) : "v"((uint32_t)Ss[g * 128 + nb * 32 + lr]));
          sc[j] = f;
        }
      }
      v8h_ af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (A16) {
          af[i] = __builtin_bit_cast(
              v8h_, *reinterpret_cast<const u32x4*>(st + arow0 + i * 32 * AROW + 16 * ((2 * g + h) ^ (lr & 7))));
        } else {
          const u32x2 x = *reinterpret_cast<const u32x2*>(st + arow0 + i * 32 * AROW + 16 * (g ^ asw8) + 8 * h);
          af[i] = a8_to_h(x[0], x[1]);
        }
      }
      if constexpr (RAW) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], wf[j], acc[i][j], 0, 0, 0);
      } else {
        // software pipeline over the TM x TN blocks: the matrix op of block
        // t + 1 is issued before the vector work on block t's partial, so two
        // partials are live at a time and the op's latency is hidden
        constexpr int T = TM * TN;
        v16f Pc = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[0], wf[0], v16f{}, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          v16f Pn;
          if (t + 1 < T) Pn = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[(t + 1) / TN], wf[(t + 1) % TN], v16f{}, 0, 0, 0);
          const int i = t / TN, j = t % TN;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(Pc[r], sc[j], acc[i][j][r]);
          __builtin_amdgcn_sched_barrier(0x104);        // only LDS reads and scalar work may cross
          if (t + 1 < T) Pc = Pn;
        }
      }
    }
  }

  // ---- epilogue: lane holds channel n of block j and tokens 8 q + 4 h + e of block i ----
  const int64_t mw = m0 + wm * TM * 32;                 // first token of the wave
  const int64_t nw0 = n0 + wcol0 * 32;                  // first channel of the wave
  if constexpr (!RAW) {
    // y = s_a[m] acc + bias[n], then the low-rank branch onto the finished values
    const bool tensor = p.a_gran == CR_GRAN_TENSOR;
    const float sa_t = tensor ? p.a_scales[0] : 0.f;
    float bj[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) bj[j] = p.bias ? bf16_lo(p.bias[nw0 + j * 32 + lr]) : 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      v4f sa[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t mq = mw + i * 32 + 8 * q + 4 * h;
        if (tensor) {
          sa[q] = v4f{sa_t, sa_t, sa_t, sa_t};
        } else if (mq + 3 < p.M) {
          sa[q] = *reinterpret_cast<const v4f*>(p.a_scales + mq);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) sa[q][e] = p.a_scales[imin64(mq + e, p.M - 1)];
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(acc[i][j][r], sa[r >> 2][r & 3], bj[j]);
    }
    if (p.lora_act) {
      // y += sum_r la[m, r] L1[n, r]: A = la (tokens), B = L1 (channels)
      const int R = p.R;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = nw0 + j * 32 + lr;   // L1 in the tiled layout [N/128][R][128]
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int64_t mr = imin64(mw + i * 32 + lr, p.M - 1);
          if (!p.lora_f32) {
            const uint16_t* la = reinterpret_cast<const uint16_t*>(p.lora_act) + mr * R;
            for (int r0 = 0; r0 < R; r0 += 16)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(la + r0 + 8 * h)),
                  lora_up8(p.lora_up, R, n, r0 + 8 * h), acc[i][j], 0, 0, 0);
          } else {
            const float* la = reinterpret_cast<const float*>(p.lora_act) + mr * R;
            for (int r0 = 0; r0 < R; r0 += 2)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(la[r0 + h], lora_up1(p.lora_up, R, n, r0 + h),
                                                               acc[i][j], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);            // one block's operands live at a time
        }
      }
    }
  }
  // Stores through LDS, 32 token rows of the wave at a time: the lane writes
  // its column of each row, then whole 16-byte pieces of the rows go out
  // (bf16 rounded half to even; int32 and float32 as they are).
  constexpr int ES = (OUT == CR_OUT_BF16) ? 2 : 4;      // bytes per output element
  constexpr int CS = TN * 32 * ES + 16;                 // LDS row stride of a 32-row chunk
  constexpr int PR = TN * 32 * ES / 16;                 // 16-byte pieces per row
  static_assert(NW * 32 * CS <= NS * STAGE, "store chunks fit the stage buffers");
  __syncthreads();                                      // every wave is done with the stage buffers
  uint8_t* chunk = smem + wave * (32 * CS);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        uint8_t* d = chunk + (8 * (r >> 2) + 4 * h + (r & 3)) * CS + (j * 32 + lr) * ES;   // rows r, r + 1
        if constexpr (OUT == CR_OUT_BF16) {
          const uint32_t pk =
              __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_){acc[i][j][r], acc[i][j][r + 1]}, v2bf));
          *reinterpret_cast<uint16_t*>(d) = (uint16_t)pk;
          *reinterpret_cast<uint16_t*>(d + CS) = (uint16_t)(pk >> 16);
        } else if constexpr (RAW) {
          *reinterpret_cast<int32_t*>(d) = (int)acc[i][j][r];
          *reinterpret_cast<int32_t*>(d + CS) = (int)acc[i][j][r + 1];
        } else {
          *reinterpret_cast<float*>(d) = acc[i][j][r];
          *reinterpret_cast<float*>(d + CS) = acc[i][j][r + 1];
        }
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0): the chunk is in LDS (a wave's LDS ops stay in order)
#pragma unroll
    for (int q = 0; q < 32 * PR / 64; ++q) {
      const int pc = q * 64 + l;
      const int row = pc / PR, c = pc % PR;
      u32x4 v = *reinterpret_cast<const u32x4*>(chunk + row * CS + c * 16);
      const int64_t m = mw + i * 32 + row;
      if (m < p.M) {
        u32x4* o = reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(p.out) + (m * p.ldc + nw0) * ES + c * 16);
        if (RAW && p.k_lo > 0) v += *o;                 // a later K chunk: add to the earlier chunks' sum
        *o = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                 // reads done before the next chunk overwrites
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int TM, int TN, bool A16, int OUT>
static hipError_t launch_w4a8_t(const GemmParams& p, hipStream_t s) {
  constexpr int stage = 256 * (A16 ? 128 : 64) + 4096 + 1024 + 1024;
  constexpr int lds = (A16 ? 2 : 3) * stage;
  static const hipError_t attr = hipFuncSetAttribute((const void*)gemm_w4a8_kernel<TM, TN, A16, OUT>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = ((p.M + 255) / 256) * (p.N / 128);
  hipLaunchKernelGGL((gemm_w4a8_kernel<TM, TN, A16, OUT>), dim3((unsigned)tiles), dim3(256), lds, s, p);
  return hipGetLastError();
}

// 2 x 2 waves of 128 x 64 outputs (int8 codes: each activation fragment is
// converted once per two channel blocks)
template <int OUT>
static hipError_t launch_w4a8_out(const GemmParams& p, hipStream_t s) {
  if (p.a_f16) return launch_w4a8_t<4, 2, true, OUT>(p, s);
  return launch_w4a8_t<4, 2, false, OUT>(p, s);
}

hipError_t launch_gemm_w4a8(const GemmParams& p, hipStream_t s) {
  switch (p.out_type) {
    case CR_OUT_BF16: return launch_w4a8_out<CR_OUT_BF16>(p, s);
    case CR_OUT_F32: return launch_w4a8_out<CR_OUT_F32>(p, s);
    default: {
      // the int32 output in K chunks of at most 8192 (128 k-tiles), each exact
      // in float32 and added in int32 by the next launch
      const int KT = (int)(p.K / 64);
      for (int k0 = 0; k0 < KT; k0 += 128) {
        GemmParams q = p;
        q.k_lo = k0;
        q.k_hi = k0 + 128 < KT ? k0 + 128 : KT;
        const hipError_t e = launch_w4a8_out<CR_OUT_I32_RAW>(q, s);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
}

}  // namespace cr
