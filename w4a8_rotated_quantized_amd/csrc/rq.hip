// Rotate + quantize kernels (gfx950).
//
// ConvRot rotation: "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4" page, intro
// (group-256 regular Hadamard on weights offline and on activations online,
// followed by dynamic quantization). Unsigned post-GELU path and the shared
// LoRA-down: "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Key Technical
// Optimizations and Kernel Engineering. Asymmetric g16 weights:
// "Qwen-Image-Edit-2511-W4A8-ConvRot" card, file layout.
//
// Rotation layout. A 256-element group is held by the 16 lanes of one DPP
// row, 16 fp32 values per lane. Element index bits b0 b1 b6 b7 live in the
// register index e = b0 + 2 b1 + 4 b6 + 8 b7; bits b2..b5 live in the lane.
// The lane <-> bits map uses the XOR patterns a single DPP move provides
// inside a row (lane^1, lane^2, lane^7, lane^8):
//     L = b2*1 ^ b3*2 ^ b4*7 ^ b5*8.
// Each lane loads 4 x 8 contiguous bytes (elements b0,b1 for each b6,b7), so
// one load instruction of a row covers 128 contiguous bytes.
//
// Butterfly order is h = 1, 2, 4, ..., 128 (bits b0..b7), each a float32
// add/sub, matching the reference definition exactly. Cross-lane stages use
// one fused multiply-add with a DPP operand, x += c * partner(x), c = +-1
// (an exact product, so the single rounding equals that of x +- partner).
// The lane then holds sigma * (true value) with sigma = +-1 a per-lane
// constant; the digit-sign vector D splits into a per-register part (digits
// b0b1 and b6b7, applied as compile-time negations) and a per-lane part
// (digits b2b3 and b4b5, folded into sigma). All of it is undone exactly by
// the sign of the quantization multiplier (fl(s*v*r) = s*fl(v*r)).
#include "common.h"
#include "kernels.h"

namespace cr {

// f(d) of the digit-sign vector: -1 for a zero base-4 digit.
CR_DEV float fdig(int d) { return d == 0 ? -1.f : 1.f; }
constexpr float fdig_c(int d) { return d == 0 ? -1.f : 1.f; }
// per-register part of D: digits (b1 b0) and (b7 b6) of e = b0 + 2b1 + 4b6 + 8b7
constexpr bool dreg_neg(int e) { return fdig_c(e & 3) * fdig_c(e >> 2) < 0; }

struct LaneRot {
  int gL;          // element bits b2..b5 of this lane, packed (b2 + 2b3 + 4b4 + 8b5)
  float c[4];      // cross-lane butterfly multipliers for bits b2..b5
  float tau;       // final per-lane sign
};

CR_DEV LaneRot lane_rot(int L) {
  LaneRot r;
  const int b2 = (L ^ (L >> 2)) & 1;
  const int b3 = ((L >> 1) ^ (L >> 2)) & 1;
  const int b4 = (L >> 2) & 1;
  const int b5 = (L >> 3) & 1;
  r.gL = b2 | (b3 << 1) | (b4 << 2) | (b5 << 3);
  const int bits[4] = {b2, b3, b4, b5};
  // stage s flips element bit b_{2+s}; digit of that bit is (b3 b2) for s<2, (b5 b4) for s>=2
  for (int s = 0; s < 4; ++s) {
    int lo = (s < 2) ? 0 : 2;
    int d = bits[lo] + 2 * bits[lo + 1];
    int dp = d ^ (1 << (s - lo));
    float sign = bits[s] ? -1.f : 1.f;
    r.c[s] = sign * fdig(d) * fdig(dp);
  }
  r.tau = (__popc(r.gL) & 1) ? -1.f : 1.f;
  return r;
}

// In-register butterflies over register bit `rb` (1, 2, 4, 8).
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

// Loads one 256-group of bf16 (row pointer p at the group start) and rotates it.
// Returns stored values (sigma * H x per element, before the final signs).
CR_DEV void load_group(const uint16_t* __restrict__ p, int gL, u32x2 (&w)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = *reinterpret_cast<const u32x2*>(p + q * 64 + gL * 4);
}

CR_DEV void rotate_group(const u32x2 (&w)[4], const LaneRot& lr, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float t0 = bf16_lo(w[q][0]), t1 = bf16_hi(w[q][0]);
    float t2 = bf16_lo(w[q][1]), t3 = bf16_hi(w[q][1]);
    v[4 * q + 0] = dreg_neg(4 * q + 0) ? -t0 : t0;
    v[4 * q + 1] = dreg_neg(4 * q + 1) ? -t1 : t1;
    v[4 * q + 2] = dreg_neg(4 * q + 2) ? -t2 : t2;
    v[4 * q + 3] = dreg_neg(4 * q + 3) ? -t3 : t3;
  }
  bfly_reg<1>(v);                      // h = 1   (b0)
  bfly_reg<2>(v);                      // h = 2   (b1)
  bfly_lane_x1(v, lr.c[0]);            // h = 4   (b2): partner lane ^ 1
  bfly_lane_x2(v, lr.c[1]);            // h = 8   (b3): partner lane ^ 2
  bfly_lane_x7(v, lr.c[2]);            // h = 16  (b4): partner lane ^ 7
  bfly_lane_x8(v, lr.c[3]);            // h = 32  (b5): partner lane ^ 8
  bfly_reg<4>(v);                      // h = 64  (b6)
  bfly_reg<8>(v);                      // h = 128 (b7)
}

// code bits: fl(fl(v * r) + 1.5*2^23); low bits are the rounded integer
CR_DEV uint32_t qbits(float v, float r) {
  return __float_as_uint(__fadd_rn(__fmul_rn(v, r), CR_MAGIC_RNE));
}

// Store the 16 codes of a rotated group for symmetric INT4 / INT8.
// rsgn = tau * r (per-lane signed multiplier); per-register sign from D.
template <int QT>
CR_DEV void quant_store_sym(const float (&v)[16], float rsgn, uint8_t* __restrict__ dst_group, int gL) {
  uint32_t b[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) b[e] = qbits(v[e], dreg_neg(e) ? -rsgn : rsgn);
  if (QT == CR_Q_SYM_INT4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h = (b[4 * q] & 0xF) | ((b[4 * q + 1] & 0xF) << 4) | ((b[4 * q + 2] & 0xF) << 8) |
                   ((b[4 * q + 3] & 0xF) << 12);
      *reinterpret_cast<uint16_t*>(dst_group + q * 32 + gL * 2) = (uint16_t)h;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h = (b[4 * q] & 0xFF) | ((b[4 * q + 1] & 0xFF) << 8) | ((b[4 * q + 2] & 0xFF) << 16) |
                   ((b[4 * q + 3] & 0xFF) << 24);
      *reinterpret_cast<uint32_t*>(dst_group + q * 64 + gL * 4) = h;
    }
  }
}

// ---------------------------------------------------------------------------
// rq_rot: rotation on. GR: 0 = TENSOR pass 1 (block max), 1 = TENSOR pass 2,
// 2 = ROW, 3 = ROW_GROUP(64), 4 = ASYM ROW_GROUP(16).
// Work: each block owns 16*GPS group slots; slot (i, seg) -> i*16 + seg.
// ROW: a block owns rpb whole rows (slots past rpb*G idle).
// ---------------------------------------------------------------------------
enum { RG_T1 = 0, RG_T2 = 1, RG_ROW = 2, RG_G64 = 3, RG_ASYM = 4 };

template <int QT, int GR, int GPS>
__global__ __launch_bounds__(256) void rq_rot_kernel(RQParams a) {
  __shared__ float red[16];
  __shared__ unsigned rowmax[16 * 8];
  const int tid = threadIdx.x;
  const int seg = tid >> 4;
  const int L = tid & 15;
  const LaneRot lr = lane_rot(L);
  const int G = a.G;
  const float qmax = (QT == CR_Q_SYM_INT8) ? 127.f : 7.f;

  int64_t row[GPS];
  int grp[GPS];
  bool ok[GPS];
#pragma unroll
  for (int i = 0; i < GPS; ++i) {
    if (GR == RG_ROW) {
      int local = i * 16 + seg;
      int rl = local / G;
      row[i] = (int64_t)blockIdx.x * a.rpb + rl;
      grp[i] = local - rl * G;
      ok[i] = (rl < a.rpb) && (row[i] < a.rows);
    } else {
      int64_t gi = (int64_t)blockIdx.x * (16 * GPS) + i * 16 + seg;
      ok[i] = gi < a.total_groups;
      row[i] = ok[i] ? gi / G : 0;
      grp[i] = ok[i] ? (int)(gi - row[i] * G) : 0;
    }
  }

  u32x2 w[GPS][4];
#pragma unroll
  for (int i = 0; i < GPS; ++i) {
    if (ok[i]) {
      load_group(a.x + row[i] * a.ldx + (int64_t)grp[i] * 256, lr.gL, w[i]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) w[i][q] = u32x2{0u, 0u};
    }
  }

  float v[GPS][16];
#pragma unroll
  for (int i = 0; i < GPS; ++i) rotate_group(w[i], lr, v[i]);

  if (GR == RG_T1 || GR == RG_T2 || GR == RG_ROW) {
    // ---------------- max over the scale group ----------------
    float gm[GPS];
#pragma unroll
    for (int i = 0; i < GPS; ++i) {
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[i][e]));
      gm[i] = row16_max(m);
    }
    float A;
    if (GR == RG_ROW) {
      if (tid < 16 * 8) rowmax[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < GPS; ++i)
        if (ok[i] && L == 0) atomicMax(&rowmax[(i * 16 + seg) / G], __float_as_uint(gm[i]));
      __syncthreads();
    } else {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < GPS; ++i) m = fmaxf(m, gm[i]);
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      if ((tid & 63) == 0) red[tid >> 6] = m;
      __syncthreads();
      float bm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      if (GR == RG_T1) {
        if (tid == 0) a.ws[blockIdx.x] = bm;
        return;
      }
      // pass 2: global max over the pass-1 block maxima
      float t = 0.f;
      for (int j = tid; j < a.nblk; j += 256) t = fmaxf(t, a.ws[j]);
      t = wave_max(t);
      __syncthreads();
      if ((tid & 63) == 0) red[4 + (tid >> 6)] = t;
      __syncthreads();
      A = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
      if (blockIdx.x == 0 && tid == 0) {
        float s = (A > 0.f) ? __fmul_rn(div_rn(A, qmax), 0.0625f) : 0.f;
        reinterpret_cast<float*>(a.scales)[0] = s;
      }
    }
#pragma unroll
    for (int i = 0; i < GPS; ++i) {
      if (!ok[i]) continue;
      float Ai = A;
      if (GR == RG_ROW) {
        int rl = (i * 16 + seg) / G;
        Ai = __uint_as_float(rowmax[rl]);
        if (L == 0 && grp[i] == 0) {
          float s = (Ai > 0.f) ? __fmul_rn(div_rn(Ai, qmax), 0.0625f) : 0.f;
          reinterpret_cast<float*>(a.scales)[row[i]] = s;
        }
      }
      float r = (Ai > 0.f) ? div_rn(qmax, Ai) : 0.f;
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.codes) +
                     row[i] * (QT == CR_Q_SYM_INT4 ? a.K / 2 : a.K) +
                     (int64_t)grp[i] * (QT == CR_Q_SYM_INT4 ? 128 : 256);
      quant_store_sym<QT>(v[i], lr.tau * r, dst, lr.gL);
    }
  } else if (GR == RG_G64) {
    // 64-groups inside a 256-group: elements with fixed (b6, b7) = registers 4q..4q+3
#pragma unroll
    for (int i = 0; i < GPS; ++i) {
      float rq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float m = amax3(fabsf(v[i][4 * q]), fabsf(v[i][4 * q + 1]),
                        fmaxf(fabsf(v[i][4 * q + 2]), fabsf(v[i][4 * q + 3])));
        m = row16_max(m);
        rq[q] = (m > 0.f) ? div_rn(qmax, m) : 0.f;
        if (ok[i] && L == 0) {
          float s = (m > 0.f) ? __fmul_rn(div_rn(m, qmax), 0.0625f) : 0.f;
          reinterpret_cast<float*>(a.scales)[row[i] * (a.K / 64) + grp[i] * 4 + q] = s;
        }
      }
      if (!ok[i]) continue;
      uint32_t b[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float rs = lr.tau * rq[e >> 2];
        b[e] = qbits(v[i][e], dreg_neg(e) ? -rs : rs);
      }
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.codes) +
                     row[i] * (QT == CR_Q_SYM_INT4 ? a.K / 2 : a.K) +
                     (int64_t)grp[i] * (QT == CR_Q_SYM_INT4 ? 128 : 256);
      if (QT == CR_Q_SYM_INT4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t h = (b[4 * q] & 0xF) | ((b[4 * q + 1] & 0xF) << 4) | ((b[4 * q + 2] & 0xF) << 8) |
                       ((b[4 * q + 3] & 0xF) << 12);
          *reinterpret_cast<uint16_t*>(dst + q * 32 + lr.gL * 2) = (uint16_t)h;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t h = (b[4 * q] & 0xFF) | ((b[4 * q + 1] & 0xFF) << 8) |
                       ((b[4 * q + 2] & 0xFF) << 16) | ((b[4 * q + 3] & 0xFF) << 24);
          *reinterpret_cast<uint32_t*>(dst + q * 64 + lr.gL * 4) = h;
        }
      }
    }
  } else {  // RG_ASYM: asymmetric uint4 per 16 consecutive rotated channels
    // 16-group = bits b0..b3: registers 4q..4q+3 of the quad of lanes sharing L>>2.
#pragma unroll
    for (int i = 0; i < GPS; ++i) {
      float t[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float s = dreg_neg(e) ? -lr.tau : lr.tau;
        t[e] = __fmul_rn(__fmul_rn(v[i][e], s), 0.0625f);
      }
      uint32_t hw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float mn = fminf(fminf(t[4 * q], t[4 * q + 1]), fminf(t[4 * q + 2], t[4 * q + 3]));
        float mx = fmaxf(fmaxf(t[4 * q], t[4 * q + 1]), fmaxf(t[4 * q + 2], t[4 * q + 3]));
        float lo = fminf(0.f, quad_min(mn));
        float hi = fmaxf(0.f, quad_max(mx));
        _Float16 s16 = (_Float16)div_rn(__fsub_rn(hi, lo), 15.f);
        bool cst = (hi == lo) || (s16 == (_Float16)0.f);
        if (cst) s16 = (_Float16)1.f;
        float sf = (float)s16;
        float z = cst ? 0.f : fminf(fmaxf(rintf(div_rn(-lo, sf)), 0.f), 15.f);
        uint32_t h = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float qq = cst ? 0.f : fminf(fmaxf(rintf(div_rn(t[4 * q + j], sf)) + z, 0.f), 15.f);
          h |= ((uint32_t)qq) << (4 * j);
        }
        hw[q] = h;
        // group index inside the 256-group: b4 + 2 b5 + 4 q = (L >> 2) + 4 q
        int gq = (L >> 2) + 4 * q;
        uint32_t zi = (uint32_t)z;
        uint32_t zn = __shfl_down(zi, 4, 16);       // partner quad (gq + 1)
        if (ok[i] && (L & 3) == 0) {
          reinterpret_cast<_Float16*>(a.scales)[row[i] * (a.K / 16) + grp[i] * 16 + gq] = s16;
          if (((L >> 2) & 1) == 0) {
            reinterpret_cast<uint8_t*>(a.zeros)[row[i] * (a.K / 32) + (grp[i] * 16 + gq) / 2] =
                (uint8_t)(zi | (zn << 4));
          }
        }
      }
      if (!ok[i]) continue;
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.codes) + row[i] * (a.K / 2) + (int64_t)grp[i] * 128;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint16_t*>(dst + q * 32 + lr.gL * 2) = (uint16_t)hw[q];
    }
  }
}

// ---------------------------------------------------------------------------
// rq_plain: no rotation, ROW_GROUP(64) scales, signed INT4 or unsigned
// shifted INT4, optional fused LoRA-down (bf16 matrix cores, fp32 accumulate).
// Block = 4 waves over the same 16 rows, wave w takes every 4th 64-column
// slice. Lane l: row l%16, 8-element chunk l/16 of each 32-column half; this
// is also the A-operand layout of the 16x16x32 bf16 MFMA used for LoRA-down.
// ---------------------------------------------------------------------------
template <bool UNSIGNED, bool LORA>
__global__ __launch_bounds__(256) void rq_plain_kernel(RQParams a) {
  __shared__ float lred[4][16][32];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = tid & 63;
  const int rl = l & 15;
  const int c = l >> 4;
  const int64_t row = (int64_t)blockIdx.x * 16 + rl;
  const bool rok = row < a.rows;
  const int64_t rowc = rok ? row : (a.rows - 1);
  const uint16_t* xr = a.x + rowc * a.ldx;
  const int nsl = (int)(a.K / 64);
  const float sh = a.shift;
  const float qmax = UNSIGNED ? 15.f : 7.f;
  v4f acc[2] = {v4f{0, 0, 0, 0}, v4f{0, 0, 0, 0}};

  for (int t = wave; t < nsl; t += 4) {
    u32x4 w0 = *reinterpret_cast<const u32x4*>(xr + t * 64 + c * 8);
    u32x4 w1 = *reinterpret_cast<const u32x4*>(xr + t * 64 + 32 + c * 8);
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_lo(w0[j]);
      v[2 * j + 1] = bf16_hi(w0[j]);
      v[8 + 2 * j] = bf16_lo(w1[j]);
      v[8 + 2 * j + 1] = bf16_hi(w1[j]);
    }
    if (LORA) {
      // la += X[16 rows, 64 cols] @ L2^T[64 cols, 32 ranks]
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 xa = h ? w1 : w0;
        v8bf afr = __builtin_bit_cast(v8bf, xa);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const uint16_t* lp = a.lora_down + (int64_t)(rb * 16 + rl) * a.K + t * 64 + h * 32 + c * 8;
          u32x4 lb = *reinterpret_cast<const u32x4*>(lp);
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, __builtin_bit_cast(v8bf, lb), acc[rb], 0, 0, 0);
        }
      }
    }
    float m = 0.f;
    if (UNSIGNED) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        v[e] = __fadd_rn(v[e], sh);
        m = fmaxf(m, v[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
    }
    // max over the 4 lanes of this row (l, l^16, l^32, l^48)
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    const float r = (m > 0.f) ? div_rn(qmax, m) : 0.f;
    if (rok && c == 0) {
      float s = (m > 0.f) ? div_rn(m, qmax) : 0.f;
      reinterpret_cast<float*>(a.scales)[row * nsl + t] = s;
    }
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      uint32_t b;
      if (UNSIGNED) {
        float p = rintf(__fmul_rn(v[e], r));
        p = fminf(fmaxf(p, 0.f), 15.f);
        b = (uint32_t)p;
      } else {
        b = qbits(v[e], r) & 0xF;
      }
      out[e >> 3] |= b << (4 * (e & 7));
    }
    if (rok) {
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.codes) + row * (a.K / 2) + t * 32;
      *reinterpret_cast<uint32_t*>(dst + c * 4) = out[0];
      *reinterpret_cast<uint32_t*>(dst + 16 + c * 4) = out[1];
    }
  }
  if (LORA) {
    // output fragment: lane l holds rank rb*16 + l%16, rows 4*(l/16) + j
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j) lred[wave][4 * c + j][rb * 16 + rl] = acc[rb][j];
    __syncthreads();
    for (int idx = tid; idx < 16 * 32; idx += 256) {
      int rr = idx >> 5, rk = idx & 31;
      int64_t orow = (int64_t)blockIdx.x * 16 + rr;
      if (orow >= a.rows) continue;
      float s = ((lred[0][rr][rk] + lred[1][rr][rk]) + lred[2][rr][rk]) + lred[3][rr][rk];
      if (a.lora_f32)
        reinterpret_cast<float*>(a.lora_act)[orow * 32 + rk] = s;
      else
        reinterpret_cast<uint16_t*>(a.lora_act)[orow * 32 + rk] = (uint16_t)f32_to_bf16_bits(s);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int QT, int GR, int GPS>
static hipError_t launch_rot(const RQParams& p, int nblk, hipStream_t s) {
  hipLaunchKernelGGL((rq_rot_kernel<QT, GR, GPS>), dim3(nblk), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int QT, int GR>
static hipError_t launch_rot_gps(const RQParams& p, int gps, int nblk, hipStream_t s) {
  switch (gps) {
    case 1: return launch_rot<QT, GR, 1>(p, nblk, s);
    case 2: return launch_rot<QT, GR, 2>(p, nblk, s);
    case 3: return launch_rot<QT, GR, 3>(p, nblk, s);
    case 4: return launch_rot<QT, GR, 4>(p, nblk, s);
    default: return launch_rot<QT, GR, 8>(p, nblk, s);
  }
}

// Block geometry shared by the host-side workspace sizing and the launch.
RQGeometry rq_geometry(int64_t rows, int64_t K, int gran_kind) {
  RQGeometry g{};
  const int64_t G = K / 256;
  if (gran_kind == RG_ROW) {
    // whole rows per block: pick the slot count (1, 2, 3, 4 or 8 groups per
    // 16-lane segment) that leaves the fewest idle slots
    const int cand[5] = {1, 2, 3, 4, 8};
    double best = -1.0;
    for (int i = 0; i < 5; ++i) {
      int64_t slots = 16 * cand[i];
      if (slots < G) continue;
      int64_t rpb = slots / G;
      if (rpb > 128) rpb = 128;
      double util = (double)(rpb * G) / (double)slots;
      if (util > best + 1e-9) {
        best = util;
        g.gps = cand[i];
        g.rpb = (int)rpb;
      }
    }
    g.nblk = g.rpb ? (rows + g.rpb - 1) / g.rpb : 0;
  } else {
    g.gps = 3;
    g.rpb = 0;
    int64_t tot = rows * G;
    g.nblk = (tot + 16 * g.gps - 1) / (16 * g.gps);
  }
  return g;
}

hipError_t launch_rotate_quantize(RQParams p, hipStream_t s) {
  if (p.rot_group == 0) {
    const int nblk = (int)((p.rows + 15) / 16);
    const bool lora = p.lora_down != nullptr;
    if (p.qtype == CR_Q_UNSIGNED_INT4_SHIFT) {
      if (lora) hipLaunchKernelGGL((rq_plain_kernel<true, true>), dim3(nblk), dim3(256), 0, s, p);
      else hipLaunchKernelGGL((rq_plain_kernel<true, false>), dim3(nblk), dim3(256), 0, s, p);
    } else {
      if (lora) hipLaunchKernelGGL((rq_plain_kernel<false, true>), dim3(nblk), dim3(256), 0, s, p);
      else hipLaunchKernelGGL((rq_plain_kernel<false, false>), dim3(nblk), dim3(256), 0, s, p);
    }
    return hipGetLastError();
  }
  p.G = (int)(p.K / 256);
  p.total_groups = p.rows * p.G;
  if (p.qtype == CR_Q_ASYM_UINT4) {
    RQGeometry g = rq_geometry(p.rows, p.K, RG_ASYM);
    return launch_rot<CR_Q_ASYM_UINT4, RG_ASYM, 3>(p, (int)g.nblk, s);
  }
  if (p.gran == CR_GRAN_TENSOR) {
    RQGeometry g = rq_geometry(p.rows, p.K, RG_T1);
    p.nblk = (int)g.nblk;
    hipError_t e;
    if (p.qtype == CR_Q_SYM_INT4) {
      e = launch_rot<CR_Q_SYM_INT4, RG_T1, 3>(p, p.nblk, s);
      if (e != hipSuccess) return e;
      return launch_rot<CR_Q_SYM_INT4, RG_T2, 3>(p, p.nblk, s);
    }
    e = launch_rot<CR_Q_SYM_INT8, RG_T1, 3>(p, p.nblk, s);
    if (e != hipSuccess) return e;
    return launch_rot<CR_Q_SYM_INT8, RG_T2, 3>(p, p.nblk, s);
  }
  if (p.gran == CR_GRAN_ROW) {
    RQGeometry g = rq_geometry(p.rows, p.K, RG_ROW);
    p.rpb = g.rpb;
    if (p.qtype == CR_Q_SYM_INT4) return launch_rot_gps<CR_Q_SYM_INT4, RG_ROW>(p, g.gps, (int)g.nblk, s);
    return launch_rot_gps<CR_Q_SYM_INT8, RG_ROW>(p, g.gps, (int)g.nblk, s);
  }
  RQGeometry g = rq_geometry(p.rows, p.K, RG_G64);
  if (p.qtype == CR_Q_SYM_INT4) return launch_rot<CR_Q_SYM_INT4, RG_G64, 3>(p, (int)g.nblk, s);
  return launch_rot<CR_Q_SYM_INT8, RG_G64, 3>(p, (int)g.nblk, s);
}

}  // namespace cr
