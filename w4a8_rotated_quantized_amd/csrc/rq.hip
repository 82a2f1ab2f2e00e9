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
// row, 16 fp32 values per lane. Element index bits b0..b3 are the register
// index e (each lane owns 16 contiguous elements: two 16-byte loads, one
// 8-byte (int4) or 16-byte (int8) code store); bits b4..b7 live in the lane,
// with the lane <-> bits map chosen so that every cross-lane partner is one
// DPP move inside a row (lane^1, lane^2, lane^7, lane^8):
//     L = b4*1 ^ b5*2 ^ b6*7 ^ b7*8.
//
// Butterfly order is h = 1, 2, 4, ..., 128 (bits b0..b7), each a float32
// add/sub, matching the reference definition exactly. Cross-lane stages use
// one fused multiply-add with a DPP operand, x += c * partner(x), c = +-1
// (an exact product, so the single rounding equals that of x +- partner).
// The lane then holds sigma * (true value) with sigma = +-1 a per-lane
// constant; the digit-sign vector D splits into a per-register part (digits
// b1b0 and b3b2, applied as compile-time negations) and a per-lane part
// (digits b5b4 and b7b6, folded into sigma). All of it is undone exactly by
// the sign of the quantization multiplier (fl(s*v*r) = s*fl(v*r)).
//
// Scale granularities: per tensor (small inputs: one block; inputs whose grid
// fits one block per CU: one launch whose blocks keep their rotated values in
// registers and exchange their maxima through the workspace; larger inputs:
// a first launch writes one maximum per block, a second recomputes the
// rotation and quantizes with the maximum of those), per row (blocks own
// whole rows), per 64-group (a quad of lanes), asymmetric per 16-group (one
// lane).
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "rotate.h"

namespace cr {

// Workspace of the per-tensor passes (block maxima, the one-launch exchange)
// for convrot_rotate_quantize_noalloc: a fixed array in device memory (one copy per GPU, kept until the process
// ends) used in place of a caller workspace. Host code never passes the
// array's name to a kernel: rq_noalloc_scratch() returns its device address,
// looked up once per device with that device current.
static __device__ __align__(256) float scratch[kNoallocScratchFloats];

// per-tensor scale: inputs of at most TINY_UNITS 256-groups take one block
// (rq_tiny_kernel); larger ones take one launch (rq_onepass_kernel) while its
// grid fits one block per CU, else two launches
constexpr int TINY_UNITS = 64;

hipError_t rq_noalloc_scratch(float** out) {
  static std::mutex mu;
  static float* ptr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<float*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

// code bits: fl(fl(v * r) + 1.5*2^23); the low byte is the rounded integer
CR_DEV uint32_t qbits(float v, float r) {
  return __float_as_uint(__fadd_rn(__fmul_rn(v, r), CR_MAGIC_RNE));
}

// low bytes of four words -> one word (v_perm_b32 x3)
CR_DEV uint32_t gather4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint32_t t = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
  uint32_t u = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
  return __builtin_amdgcn_perm(u, t, 0x05040100u);
}

// Quantize and store the 16 codes of one lane (elements 16*gL .. 16*gL+15 of
// the group) at dst (16 bytes for INT8, 8 bytes for INT4).
// rs = tau * r; the per-register sign of D is applied as a negated multiplier.
template <int QT>
CR_DEV void quant_store(const float (&v)[16], float rs, uint8_t* __restrict__ dst) {
  uint32_t b[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) b[e] = qbits(v[e], dreg_neg(e) ? -rs : rs);
  if constexpr (QT == CR_Q_SYM_INT8) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = gather4(b[4 * j], b[4 * j + 1], b[4 * j + 2], b[4 * j + 3]);
    *reinterpret_cast<u32x4*>(dst) = o;
  } else {
    u32x2 o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 8 * h;
      uint32_t ev = gather4(b[e], b[e + 2], b[e + 4], b[e + 6]);
      uint32_t od = gather4(b[e + 1], b[e + 3], b[e + 5], b[e + 7]);
      o[h] = (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
    }
    *reinterpret_cast<u32x2*>(dst) = o;
  }
}

// Address of one lane's codes: natural rows, or (INT4 only) the tiled
// fragment layout [rows/16][K/64][64 lanes x 8 B] where the lane's 16
// elements (k = 256 grp + 16 gL ...) are chunk gL%4 of k-tile 4 grp + gL/4.
template <int QT>
CR_DEV uint8_t* code_dst(const RQParams& a, int64_t row, int grp, int gL) {
  if constexpr (QT == CR_Q_SYM_INT8) {
    return reinterpret_cast<uint8_t*>(a.codes) + row * a.K + grp * 256 + gL * 16;
  } else {
    if (a.tiled)
      return reinterpret_cast<uint8_t*>(a.codes) + ((row >> 4) * (a.K / 64) + grp * 4 + (gL >> 2)) * 512 +
             ((gL & 3) * 16 + (row & 15)) * 8;
    return reinterpret_cast<uint8_t*>(a.codes) + row * (a.K / 2) + grp * 128 + gL * 8;
  }
}

// fp6 E2M3 fragment layout (INT4 codes for the fp6 matrix-core GEMM): the
// lane's 16 codes (k = 256 grp + 16 gL + e) are half gL & 1 of fragment lane
// 32 ((gL >> 1) & 1) + row % 32 in the 1536-byte fragment of row block
// row / 32 and k-tile 4 grp + gL / 4; that lane's bytes 0..15 sit at
// lane * 16 and bytes 16..23 at 1024 + lane * 8, so half 0 is three words at
// lane * 16 and half 1 one word at lane * 16 + 12 and two at 1024 + lane * 8.
// Each code is the rounded integer as a float (adding and removing
// 1.5 * 2^23 rounds half to even and turns -0 into +0), converted exactly;
// the conversion interleaves its two sources (field 2i from the first,
// 2i + 1 from the second).
CR_DEV float f6_qval(float v, float r) {   // the rounded integer code as a float (+0 for zero)
  return __fsub_rn(__fadd_rn(__fmul_rn(v, r), CR_MAGIC_RNE), CR_MAGIC_RNE);
}

// codes of two groups' 16 values (the second may be a copy of the first):
// words 0..2 hold the first group's 16 six-bit fields, words 3..5 the second's
CR_DEV u32x4 f6_pack2(const float (&v0)[16], float rs0, const float (&v1)[16], float rs1, uint32_t (&w45)[2]) {
  v16f s0, s1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s0[i] = f6_qval(v0[2 * i], dreg_neg(2 * i) ? -rs0 : rs0);
    s1[i] = f6_qval(v0[2 * i + 1], dreg_neg(2 * i + 1) ? -rs0 : rs0);
    s0[8 + i] = f6_qval(v1[2 * i], dreg_neg(2 * i) ? -rs1 : rs1);
    s1[8 + i] = f6_qval(v1[2 * i + 1], dreg_neg(2 * i + 1) ? -rs1 : rs1);
  }
  const auto o = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(s0, s1, 1.0f);
  w45[0] = o[4];
  w45[1] = o[5];
  return u32x4{o[0], o[1], o[2], o[3]};
}

CR_DEV uint8_t* f6_frag(const RQParams& a, int64_t row, int grp, int gL) {
  return reinterpret_cast<uint8_t*>(a.codes) + ((row >> 5) * (a.K / 64) + grp * 4 + (gL >> 2)) * 1536;
}

// the three words of one lane's half (any lane activity: plain word stores)
CR_DEV void f6_store_words(uint32_t c0, uint32_t c1, uint32_t c2, const RQParams& a, int64_t row, int grp, int gL) {
  uint8_t* frag = f6_frag(a, row, grp, gL);
  const int lm = ((gL >> 1) & 1) * 32 + (int)(row & 31);
  const bool h = gL & 1;
  uint32_t* w0 = reinterpret_cast<uint32_t*>(frag + lm * 16 + (h ? 12 : 0));
  uint32_t* w1 = h ? reinterpret_cast<uint32_t*>(frag + 1024 + lm * 8) : w0 + 1;
  w0[0] = c0;
  w1[0] = c1;
  w1[1] = c2;
}

// the same with all 16 lanes of the DPP row active: the two halves of a
// fragment lane sit in lanes L and L ^ 1 (gL and gL ^ 1), so half 0 takes its
// partner's first word and stores the lane's bytes 0..15 at once, and half 1
// stores bytes 16..23
CR_DEV void f6_store_pair(uint32_t c0, uint32_t c1, uint32_t c2, const RQParams& a, int64_t row, int grp, int gL) {
  const uint32_t p0 = (uint32_t)dpp_i<DPP_QUAD_1032>((int)c0);
  uint8_t* frag = f6_frag(a, row, grp, gL);
  const int lm = ((gL >> 1) & 1) * 32 + (int)(row & 31);
  if ((gL & 1) == 0) *reinterpret_cast<u32x4*>(frag + lm * 16) = u32x4{c0, c1, c2, p0};
  else *reinterpret_cast<u32x2*>(frag + 1024 + lm * 8) = u32x2{c1, c2};
}

CR_DEV void quant_store_f6(const float (&v)[16], float rs, const RQParams& a, int64_t row, int grp, int gL) {
  uint32_t w45[2];
  const u32x4 o = f6_pack2(v, rs, v, rs, w45);
  f6_store_words(o[0], o[1], o[2], a, row, grp, gL);
}

// INT8 codes as fp16 values ([rows, K], the activation operand of the fp16
// matrix-core W4A8 GEMM): the rounded integer as a float (as f6_qval), then
// converted exactly (|code| <= 127), 32 bytes per lane
CR_DEV void quant_store_h16(const float (&v)[16], float rs, uint8_t* __restrict__ dst) {
  uint32_t o[8];
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    const float q0 = f6_qval(v[e], dreg_neg(e) ? -rs : rs);
    const float q1 = f6_qval(v[e + 1], dreg_neg(e + 1) ? -rs : rs);
    o[e >> 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(q0, q1));
  }
  *reinterpret_cast<u32x4*>(dst) = u32x4{o[0], o[1], o[2], o[3]};
  *reinterpret_cast<u32x4*>(dst + 16) = u32x4{o[4], o[5], o[6], o[7]};
}

// codes of one lane in the layout the parameters ask for
template <int QT>
CR_DEV void store_codes(const float (&v)[16], float rs, const RQParams& a, int64_t row, int grp, int gL) {
  if (QT == CR_Q_SYM_INT4 && a.tiled == 2) quant_store_f6(v, rs, a, row, grp, gL);
  else if (QT == CR_Q_SYM_INT8 && a.tiled == 3)
    quant_store_h16(v, rs, reinterpret_cast<uint8_t*>(a.codes) + (row * a.K + grp * 256 + gL * 16) * 2);
  else quant_store<QT>(v, rs, code_dst<QT>(a, row, grp, gL));
}

// ---------------------------------------------------------------------------
// rq_rot: rotation on, one launch: per-row scales (RG_ROW), per-64-group
// scales (RG_G64) and asymmetric 16-group weights (RG_ASYM).
// Work: segment s of block (bx, by) owns row bx*rpb + (s >> lg_spr) and the
// groups by*spr*GPS + (s & (spr-1)) + spr*i, i < GPS (spr = 2^lg_spr).
// ---------------------------------------------------------------------------
enum { RG_ROW = 2, RG_G64 = 3, RG_ASYM = 4 };

template <int QT, int GR, int GPS, int NR, bool SM = false>
__global__ __launch_bounds__(256) void rq_rot_kernel(RQParams a) {
  static_assert(GR != RG_ASYM || NR == 256, "asymmetric g16 weights use the 256 rotation");
  static_assert(!SM || NR != 1024, "smoothing with the 1024 rotation is not built");
  static_assert(NR != 1024 || GPS % 4 == 0, "a 1024-group is four chunks of one segment");
  __shared__ unsigned rowmax[16];
  const int tid = threadIdx.x;
  const int seg = tid >> 4;
  const int L = tid & 15;
  const LaneRot lr = lane_rot<NR>(L);
  constexpr float post = RotSize<NR>::inv_sqrt;
  const float qmax = (QT == CR_Q_SYM_INT8) ? 127.f : 7.f;
  const int lg = a.lg_spr;
  const int spr = 1 << lg;
  const int rl = seg >> lg;
  const int64_t row = (int64_t)blockIdx.x * a.rpb + rl;
  const bool row_ok = rl < a.rpb && row < a.rows;
  // chunk i of the segment: groups interleaved over the segments of a row,
  // or (NR = 1024) GPS consecutive chunks, whole 1024-groups
  const int g0 = (NR == 1024) ? (int)blockIdx.y * (spr * GPS) + (seg & (spr - 1)) * GPS
                              : (int)blockIdx.y * (spr * GPS) + (seg & (spr - 1));
  const int gstep = (NR == 1024) ? 1 : spr;
  const uint16_t* xr = a.x + (row_ok ? row : 0) * a.ldx + lr.gL * 16;

  bool ok[GPS];
  u32x4 w[GPS][2];
#pragma unroll
  for (int i = 0; i < GPS; ++i) {
    const int grp = g0 + gstep * i;
    ok[i] = row_ok && grp < a.G;
    if (ok[i]) {
      w[i][0] = *reinterpret_cast<const u32x4*>(xr + grp * 256);
      w[i][1] = *reinterpret_cast<const u32x4*>(xr + grp * 256 + 8);
    } else {
      w[i][0] = u32x4{0u, 0u, 0u, 0u};
      w[i][1] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  float v[GPS][16];
#pragma unroll
  for (int i = 0; i < GPS; ++i) {
    if constexpr (SM) {
      const int grp = min(g0 + gstep * i, a.G - 1);
      rotate_group<NR, false, true>(w[i], lr, v[i], a.smooth + grp * 256 + lr.gL * 16);
    } else if (NR == 1024 && chunk_neg(i)) {
      rotate_group<NR, true>(w[i], lr, v[i]);
    } else {
      rotate_group<NR>(w[i], lr, v[i]);
    }
  }
  if constexpr (NR == 1024) bfly_chunks<GPS>(v);
  // quantization multiplier sign of chunk i (lane sign, and D's chunk digit for 1024)
  float csg[GPS];
#pragma unroll
  for (int i = 0; i < GPS; ++i) csg[i] = (NR == 1024 && chunk_neg(i)) ? -lr.tau : lr.tau;

  const int64_t crow_i = row_ok ? row : 0;

  if constexpr (GR == RG_ROW) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < GPS; ++i)
#pragma unroll
      for (int e = 0; e < 16; e += 2) m = amax3(m, fabsf(v[i][e]), fabsf(v[i][e + 1]));
    m = row16_max(m);
    if (tid < 16) rowmax[tid] = 0u;
    __syncthreads();
    if (L == 0 && row_ok) atomicMax(&rowmax[rl], __float_as_uint(m));
    __syncthreads();
    const float A = __uint_as_float(rowmax[rl]);
    if (row_ok && (seg & (spr - 1)) == 0 && L == 0) {
      float sc = (A > 0.f) ? __fmul_rn(div_rn(A, qmax), post) : 0.f;
      reinterpret_cast<float*>(a.scales)[row] = sc;
    }
    const float r = (A > 0.f) ? div_rn(qmax, A) : 0.f;
#pragma unroll
    for (int i = 0; i < GPS; ++i)
      if (ok[i]) store_codes<QT>(v[i], csg[i] * r, a, crow_i, g0 + gstep * i, lr.gL);
  } else if constexpr (GR == RG_G64) {
    // 64-group = bits b0..b5: the quad of lanes sharing (b6, b7) = (L2, L3)
#pragma unroll
    for (int i = 0; i < GPS; ++i) {
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) m = amax3(m, fabsf(v[i][e]), fabsf(v[i][e + 1]));
      m = quad_max(m);
      const int grp = g0 + gstep * i;
      if (ok[i] && (L & 3) == 0) {
        float s = (m > 0.f) ? __fmul_rn(div_rn(m, qmax), post) : 0.f;
        reinterpret_cast<float*>(a.scales)[row * (a.K / 64) + grp * 4 + (L >> 2)] = s;
      }
      const float r = (m > 0.f) ? div_rn(qmax, m) : 0.f;
      if (ok[i]) store_codes<QT>(v[i], csg[i] * r, a, crow_i, grp, lr.gL);
    }
  } else {  // RG_ASYM: asymmetric uint4 per 16 consecutive rotated channels = one lane
#pragma unroll
    for (int i = 0; i < GPS; ++i) {
      float t[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float s = dreg_neg(e) ? -lr.tau : lr.tau;
        t[e] = __fmul_rn(__fmul_rn(v[i][e], s), post);
      }
      float mn = t[0], mx = t[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) {
        mn = fminf(mn, t[e]);
        mx = fmaxf(mx, t[e]);
      }
      const float lo = fminf(0.f, mn), hi = fmaxf(0.f, mx);
      _Float16 s16 = (_Float16)div_rn(__fsub_rn(hi, lo), 15.f);
      const bool cst = (hi == lo) || (s16 == (_Float16)0.f);
      if (cst) s16 = (_Float16)1.f;
      const float sf = (float)s16;
      const float z = cst ? 0.f : fminf(fmaxf(rintf(div_rn(-lo, sf)), 0.f), 15.f);
      u32x2 o = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float qq = cst ? 0.f : fminf(fmaxf(rintf(div_rn(t[e], sf)) + z, 0.f), 15.f);
        o[e >> 3] |= ((uint32_t)qq) << (4 * (e & 7));
      }
      const uint32_t zi = (uint32_t)z;
      const uint32_t zp = (uint32_t)dpp_i<DPP_QUAD_1032>((int)zi);   // group gL ^ 1
      const int grp = g0 + gstep * i;
      if (ok[i]) {
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(a.codes) + crow_i * (a.K / 2) + grp * 128 + 8 * lr.gL) = o;
        reinterpret_cast<_Float16*>(a.scales)[row * (a.K / 16) + grp * 16 + lr.gL] = s16;
        if ((lr.gL & 1) == 0)
          reinterpret_cast<uint8_t*>(a.zeros)[row * (a.K / 32) + grp * 8 + lr.gL / 2] = (uint8_t)(zi | (zp << 4));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// rq_tensor: per-tensor scale with rotation on, two launches over the same
// block -> data map, the second walking it backwards within each XCD (pass
// 1 then re-reads X from the L2 of the XCD that read it in pass 0, or from
// the last-level cache, most recently read data first).
// Block b owns 16 rows, row block b / GC, and J consecutive 256-groups
// starting at group (b % GC) * J (GC = ceil(G / J)); segment seg (16 lanes)
// takes row seg. A segment reads J * 512 contiguous bytes of its row, and a
// block writes whole J * 2 KB runs of the tiled code layout from one CU
// (spreading the 16 rows of a run over blocks on different XCDs turns the
// code stores into 8-byte partial-line writes from several L2s).
//   PASS 0: max |H x| of the block -> ws[blockIdx.x].
//   PASS 1: A = max over ws[0 .. gridDim.x), rotation recomputed, codes.
//   PASS 2: as PASS 1, writing the INT4 codes (codes, scales) and the INT8
//           codes of the same rotated values (codes8, scales8).
// All J loads are issued first and each group is rotated as soon as its
// data is in. Rows past the end are clamped to the last row and groups past
// the end to the last group, which keeps every load and store free of
// branches (a conditional memory operation makes the compiler wait for all
// loads in flight before any arithmetic), leaves the maximum unchanged and
// rewrites identical code bytes.
// ---------------------------------------------------------------------------
template <int QT, int PASS, int J, int NWS, int NR>
__global__ __launch_bounds__(256) void rq_tensor_kernel(RQParams a) {
  static_assert(NR != 1024 || J % 4 == 0, "a 1024-group is four chunks of one segment");
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int seg = tid >> 4;
  const LaneRot lr = lane_rot<NR>(tid & 15);
  const float qmax = (QT == CR_Q_SYM_INT8) ? 127.f : 7.f;
  const int G = a.G;
  const int GC = (G + J - 1) / J;
  // passes 1 and 2 walk the blocks of pass 0 backwards within each XCD
  // (blocks go round robin over the 8 XCDs): the data pass 0 read last,
  // most likely still in that XCD's L2 or in the last-level cache, is read
  // again first
  const unsigned nb = gridDim.x;
  unsigned b = blockIdx.x;
  if (PASS >= 1) b = (nb % 8 == 0) ? (nb / 8 - 1 - b / 8) * 8 + b % 8 : nb - 1 - b;
  const int64_t row = imin64((int64_t)(b / (unsigned)GC) * 16 + seg, a.rows - 1);
  const int g0 = (int)(b % (unsigned)GC) * J;
  const uint16_t* xr = a.x + row * a.ldx + lr.gL * 16;

  // PASS 1: the block maxima of pass 0 are loaded before the rows (up to
  // 256 * NWS of them, unconditional loads with clamped indices; for NWS >= 4
  // 16-byte loads of four maxima, the workspace being 16-byte aligned, and
  // the last three one by one), so that waiting for them leaves the row
  // loads in flight; NWS = 0 is the loop for grids beyond 256 * 32 blocks.
  float t = 0.f;
  if constexpr (PASS >= 1) {
    const int gd = (int)gridDim.x;
    if constexpr (NWS >= 4) {
      const v4f* w4 = reinterpret_cast<const v4f*>(a.ws);
      const int n4 = gd >> 2;   // whole groups of four (gd > 256 here)
#pragma unroll
      for (int i = 0; i < NWS / 4; ++i) {
        const v4f q = w4[min(tid + 256 * i, n4 - 1)];
        t = fmaxf(t, fmaxf(fmaxf(q[0], q[1]), fmaxf(q[2], q[3])));
      }
      t = fmaxf(t, fmaxf(a.ws[gd - 1], fmaxf(a.ws[gd - 2], a.ws[gd - 3])));
    } else if constexpr (NWS > 0) {
#pragma unroll
      for (int i = 0; i < NWS; ++i) t = fmaxf(t, a.ws[min(tid + 256 * i, gd - 1)]);
    } else {
      for (int i = tid; i < gd; i += 256) t = fmaxf(t, a.ws[i]);
    }
  }

  int grp[J];
  u32x4 w[J][2];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    grp[j] = min(g0 + j, G - 1);
    const uint16_t* px = xr + grp[j] * 256;
    w[j][0] = *reinterpret_cast<const u32x4*>(px);
    w[j][1] = *reinterpret_cast<const u32x4*>(px + 8);
  }
  __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use

  // NR = 1024: all J chunks stay in registers for the two cross-chunk stages
  float vall[NR == 1024 ? J : 1][16];
  if constexpr (NR == 1024) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (chunk_neg(j)) rotate_group<NR, true>(w[j], lr, vall[j]);
      else rotate_group<NR>(w[j], lr, vall[j]);
    }
    bfly_chunks<J>(vall);
  }

  if constexpr (PASS == 0) {
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      float v[16];
      if constexpr (NR == 1024) {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = vall[j][e];
      } else {
        rotate_group<NR>(w[j], lr, v);
      }
#pragma unroll
      for (int e = 0; e < 16; e += 2) m = amax3(m, fabsf(v[e]), fabsf(v[e + 1]));
    }
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) a.ws[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  } else {
    t = wave_max(t);
    if ((tid & 63) == 0) red[tid >> 6] = t;
    __syncthreads();
    const float A = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (blockIdx.x == 0 && tid == 0) {
      const float sc = (A > 0.f) ? __fmul_rn(div_rn(A, qmax), RotSize<NR>::inv_sqrt) : 0.f;
      reinterpret_cast<float*>(a.scales)[0] = sc;
      if constexpr (PASS == 2) {
        const float sc8 = (A > 0.f) ? __fmul_rn(div_rn(A, 127.f), RotSize<NR>::inv_sqrt) : 0.f;
        reinterpret_cast<float*>(a.scales8)[0] = sc8;
      }
    }
    const float rq = lr.tau * ((A > 0.f) ? div_rn(qmax, A) : 0.f);
    const float rq8 = lr.tau * ((A > 0.f) ? div_rn(127.f, A) : 0.f);   // PASS 2 only
    RQParams a8 = a;
    a8.codes = a.codes8;
    if (QT == CR_Q_SYM_INT4 && a.tiled == 2) {
      // fp6 fragments: two groups per conversion, every lane of the row active
#pragma unroll
      for (int j = 0; j < J; j += 2) {
        const int j1 = (j + 1 < J) ? j + 1 : j;
        float v0[16], v1[16];
        if constexpr (NR == 1024) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            v0[e] = vall[j][e];
            v1[e] = vall[j1][e];
          }
        } else {
          rotate_group<NR>(w[j], lr, v0);
          rotate_group<NR>(w[j1], lr, v1);
        }
        const float sg0 = (NR == 1024 && chunk_neg(j)) ? -1.f : 1.f;
        const float sg1 = (NR == 1024 && chunk_neg(j1)) ? -1.f : 1.f;
        uint32_t w45[2];
        const u32x4 o = f6_pack2(v0, sg0 * rq, v1, sg1 * rq, w45);
        f6_store_pair(o[0], o[1], o[2], a, row, grp[j], lr.gL);
        if (j + 1 < J) f6_store_pair(o[3], w45[0], w45[1], a, row, grp[j1], lr.gL);
        if constexpr (PASS == 2) {
          quant_store<CR_Q_SYM_INT8>(v0, sg0 * rq8, code_dst<CR_Q_SYM_INT8>(a8, row, grp[j], lr.gL));
          if (j + 1 < J) quant_store<CR_Q_SYM_INT8>(v1, sg1 * rq8, code_dst<CR_Q_SYM_INT8>(a8, row, grp[j1], lr.gL));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float v[16];
        if constexpr (NR == 1024) {
#pragma unroll
          for (int e = 0; e < 16; ++e) v[e] = vall[j][e];
        } else {
          rotate_group<NR>(w[j], lr, v);
        }
        const float sg = (NR == 1024 && chunk_neg(j)) ? -1.f : 1.f;
        store_codes<QT>(v, sg * rq, a, row, grp[j], lr.gL);
        if constexpr (PASS == 2) quant_store<CR_Q_SYM_INT8>(v, sg * rq8, code_dst<CR_Q_SYM_INT8>(a8, row, grp[j], lr.gL));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// rq_plain: no rotation, ROW_GROUP(64) scales, signed INT4 or unsigned
// shifted INT4, optional fused LoRA-down (bf16 matrix cores, fp32 accumulate).
// Block = RPB rows (16 or 32) and NWV = 4 RPB / 16 waves; wave w takes the
// 64-column slices t = w, w + NWV, ... of all RPB rows, as Q = RPB / 16
// tiles of 16 rows. Lane l: row l%16 of each tile, 8-element chunk l/16 of
// each 32-column half; this is also the A-operand layout of the 16x16x32
// bf16 MFMA of the LoRA-down, whose B fragments (read from L2 per slice) then
// serve Q tiles.
// Streaming: the next two slices of a wave are in flight while it quantizes
// one (rounds of three name-rotated buffers; a round's surplus phases redo
// the wave's last slice: identical stores, no low-rank accumulation), and no
// load or code store in the loop is conditional: rows past the end are
// clamped to the last row (their stores rewrite that row's identical bytes).
// Code stores go through a wave-private LDS image of the slice's output
// (LAY 1: the Q tiles of 512 bytes; LAY 2: the fp6 fragment rows of these
// tiles), written back as whole 16-byte pieces of contiguous runs.
// LAY: code layout (0 natural, 1 tiled int8-core fragments, 2 fp6 fragments).
// ---------------------------------------------------------------------------
template <int RPB, int R>
struct PlainSmem {
  static constexpr int NWV = 4 * RPB / 16;
  static constexpr int STAGE = 1536;                  // bytes per wave
  static constexpr int LRED = NWV * RPB * R * 4;      // low-rank partial sums per wave
  static constexpr int BYTES = (LRED > NWV * STAGE) ? LRED : NWV * STAGE;
};

template <bool UNSIGNED, bool LORA, int R = 32, bool QUANT = true, bool SM = false, int LAY = 0, int RPB = 16>
__global__ __launch_bounds__(4 * RPB / 16 * 64) void rq_plain_kernel(RQParams a) {
  static_assert(R == 32 || R == 64, "low-rank branch of rank 32 or 64");
  static_assert(QUANT || LORA, "nothing to do");
  static_assert(RPB == 16 || RPB == 32, "16 or 32 rows per block");
  constexpr int RB = R / 16;
  constexpr int Q = RPB / 16;
  constexpr int NWV = PlainSmem<RPB, R>::NWV;
  __shared__ __attribute__((aligned(16))) uint8_t smem[PlainSmem<RPB, (LORA ? R : 1)>::BYTES];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = tid & 63;
  const int rl = l & 15;
  const int c = l >> 4;
  int64_t rowc[Q];
  const uint16_t* xr[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int64_t row = (int64_t)blockIdx.x * RPB + 16 * q + rl;
    rowc[q] = (row < a.rows) ? row : (a.rows - 1);
    xr[q] = a.x + rowc[q] * a.ldx + c * 8;
  }
  const int nsl = (int)(a.K / 64);
  const float sh = a.shift;
  const float qmax = UNSIGNED ? 15.f : 7.f;
  uint8_t* stage = smem + wave * PlainSmem<RPB, R>::STAGE;
  v4f acc[Q][RB];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[q][rb] = v4f{0, 0, 0, 0};

  const int nw = (nsl - wave + NWV - 1) / NWV;
  const int tlast = wave + NWV * (nw - 1);
  auto tof = [&](int i) { return min(wave + NWV * i, tlast); };
  auto ld = [&](int t, u32x4 (&w)[Q][2]) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      w[q][0] = *reinterpret_cast<const u32x4*>(xr[q] + t * 64);
      w[q][1] = *reinterpret_cast<const u32x4*>(xr[q] + t * 64 + 32);
    }
  };
  auto step = [&](int i, const u32x4 (&cur)[Q][2], u32x4 (&nxt)[Q][2]) {
    const int t = tof(i);
    const bool valid = i < nw;
    // low-rank fragments of this slice (L2 hits), issued before the prefetch
    // of slice i + 2 so that waiting for them (in-order counter) leaves that
    // prefetch in flight; consumed after the quantization
    u32x4 lb[LORA ? 2 : 1][LORA ? RB : 1];
    if constexpr (LORA) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          lb[h][rb] = *reinterpret_cast<const u32x4*>(a.lora_down + (int64_t)(rb * 16 + rl) * a.K + t * 64 + h * 32 + c * 8);
    }
    ld(tof(i + 2), nxt);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (QUANT) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const u32x4 w0 = cur[q][0], w1 = cur[q][1];
        float v[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = bf16_lo(w0[j]);
          v[2 * j + 1] = bf16_hi(w0[j]);
          v[8 + 2 * j] = bf16_lo(w1[j]);
          v[8 + 2 * j + 1] = bf16_hi(w1[j]);
        }
        if constexpr (SM) {   // elements t*64 + c*8 + 0..7 and t*64 + 32 + c*8 + 0..7
          const v4f* m0 = reinterpret_cast<const v4f*>(a.smooth + t * 64 + c * 8);
          const v4f* m1 = reinterpret_cast<const v4f*>(a.smooth + t * 64 + 32 + c * 8);
          const v4f ma = m0[0], mb = m0[1], mc = m1[0], md = m1[1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = __fmul_rn(v[e], ma[e]);
            v[4 + e] = __fmul_rn(v[4 + e], mb[e]);
            v[8 + e] = __fmul_rn(v[8 + e], mc[e]);
            v[12 + e] = __fmul_rn(v[12 + e], md[e]);
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
        reinterpret_cast<float*>(a.scales)[rowc[q] * nsl + t] = (m > 0.f) ? div_rn(m, qmax) : 0.f;
        if constexpr (LAY == 2) {
          // fp6: signed codes as themselves, unsigned codes u as the E2M3
          // value u/2 (exact; the GEMM doubles the product). Run h of this
          // lane (elements 32h + 8c ..) is quarter c (6 bytes at 6c of 24) of
          // fragment lane 32h + row % 32; bytes 0..15 of a fragment lane sit
          // at lane * 16, bytes 16..23 at 1024 + lane * 8.
          v16f s0 = {}, s1 = {};
#pragma unroll
          for (int i2 = 0; i2 < 8; ++i2) {
            const int e0 = (i2 < 4) ? 2 * i2 : 8 + 2 * (i2 - 4);
            float q0, q1;
            if (UNSIGNED) {
              q0 = 0.5f * fminf(fmaxf(rintf(__fmul_rn(v[e0], r)), 0.f), 15.f);
              q1 = 0.5f * fminf(fmaxf(rintf(__fmul_rn(v[e0 + 1], r)), 0.f), 15.f);
            } else {
              q0 = __fsub_rn(__fadd_rn(__fmul_rn(v[e0], r), CR_MAGIC_RNE), CR_MAGIC_RNE);
              q1 = __fsub_rn(__fadd_rn(__fmul_rn(v[e0 + 1], r), CR_MAGIC_RNE), CR_MAGIC_RNE);
            }
            s0[i2] = q0;
            s1[i2] = q1;
          }
          const auto o = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(s0, s1, 1.0f);
          // run 0: bits 0..47 of o; run 1: bits 48..95
          const uint32_t r0a = o[0], r0b = o[1] & 0xFFFFu;
          const uint32_t r1a = (o[1] >> 16) | (o[2] << 16), r1b = o[2] >> 16;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t pa = h ? r1a : r0a, pb = h ? r1b : r0b;   // 48 bits: pa (32) then pb (16)
            const int lm = 32 * h + (int)(rowc[q] & 31);
            uint8_t* f = stage + lm * 16;
            uint8_t* g = stage + 1024 + lm * 8;
            if (c == 0) {            // bytes 0..5
              *reinterpret_cast<uint32_t*>(f) = pa;
              *reinterpret_cast<uint16_t*>(f + 4) = (uint16_t)pb;
            } else if (c == 1) {     // bytes 6..11
              *reinterpret_cast<uint16_t*>(f + 6) = (uint16_t)pa;
              *reinterpret_cast<uint32_t*>(f + 8) = (pa >> 16) | (pb << 16);
            } else if (c == 2) {     // bytes 12..17
              *reinterpret_cast<uint32_t*>(f + 12) = pa;
              *reinterpret_cast<uint16_t*>(g) = (uint16_t)pb;
            } else {                 // bytes 18..23
              *reinterpret_cast<uint16_t*>(g + 2) = (uint16_t)pa;
              *reinterpret_cast<uint32_t*>(g + 4) = (pa >> 16) | (pb << 16);
            }
          }
        } else {
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
          if constexpr (LAY == 1) {
            // elements 64t + 32h + 8c .. +8 are half (c&1) of chunk 2h + c/2 of k-tile t
            uint8_t* dst = stage + q * 512 + (int)(rowc[q] & 15) * 8 + (c & 1) * 4;
            *reinterpret_cast<uint32_t*>(dst + (c >> 1) * 128) = out[0];
            *reinterpret_cast<uint32_t*>(dst + (2 + (c >> 1)) * 128) = out[1];
          } else {
            uint8_t* dst = reinterpret_cast<uint8_t*>(a.codes) + rowc[q] * (a.K / 2) + t * 32;
            *reinterpret_cast<uint32_t*>(dst + c * 4) = out[0];
            *reinterpret_cast<uint32_t*>(dst + 16 + c * 4) = out[1];
          }
        }
      }
      // the staged image back to global memory in 16-byte pieces (LDS
      // accesses of one wave complete in order: no wait between)
      if constexpr (LAY == 2) {
        const int64_t fb = (int64_t)blockIdx.x * RPB / 32;               // 32-row fragment block
        uint8_t* frag = reinterpret_cast<uint8_t*>(a.codes) + (fb * (a.K / 64) + t) * 1536;
        const bool mine = (Q == 2) || (((l >> 4) & 1) == (int)(((int64_t)blockIdx.x * RPB / 16) & 1));
        const u32x4 va = *reinterpret_cast<const u32x4*>(stage + l * 16);
        const u32x2 vb = *reinterpret_cast<const u32x2*>(stage + 1024 + l * 8);
        if (mine) {
          *reinterpret_cast<u32x4*>(frag + l * 16) = va;
          *reinterpret_cast<u32x2*>(frag + 1024 + l * 8) = vb;
        }
      } else if constexpr (LAY == 1) {
        const int q = l >> 5;                                               // lanes 0..31: tile 0, 32..63: tile 1
        const int64_t tb = (int64_t)blockIdx.x * Q + q;                     // 16-row tile
        const u32x4 va = *reinterpret_cast<const u32x4*>(stage + l * 16);
        if (q < Q && tb * 16 < a.rows)
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(a.codes) + (tb * (a.K / 64) + t) * 512 + (l & 31) * 16) = va;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (LORA && valid) {
      // la += X[16 rows, 64 cols] @ L2^T[64 cols, R ranks], per 16-row tile
#pragma unroll
      for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v8bf afr = __builtin_bit_cast(v8bf, cur[q][h]);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[q][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, __builtin_bit_cast(v8bf, lb[h][rb]), acc[q][rb], 0, 0, 0);
        }
    }
  };
  if (nw > 0) {
    u32x4 b0[Q][2], b1[Q][2], b2[Q][2];
    ld(tof(0), b0);
    ld(tof(1), b1);
    for (int i = 0; i < nw; i += 3) {
      step(i, b0, b2);
      step(i + 1, b1, b0);
      step(i + 2, b2, b1);
    }
  }
  if constexpr (LORA) {
    // output fragment: lane l holds rank rb*16 + l%16, rows 4*(l/16) + j of each tile
    __syncthreads();                                   // the stage buffers become the reduction array
    float* lred = reinterpret_cast<float*>(smem);      // [NWV][RPB][R]
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j) lred[(wave * RPB + 16 * q + 4 * c + j) * R + rb * 16 + rl] = acc[q][rb][j];
    __syncthreads();
    for (int idx = tid; idx < RPB * R; idx += NWV * 64) {
      const int rr = idx / R, rk = idx % R;
      const int64_t orow = (int64_t)blockIdx.x * RPB + rr;
      if (orow >= a.rows) continue;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) s += lred[(w * RPB + rr) * R + rk];
      if (a.lora_f32)
        reinterpret_cast<float*>(a.lora_act)[orow * R + rk] = s;
      else
        reinterpret_cast<uint16_t*>(a.lora_act)[orow * R + rk] = (uint16_t)f32_to_bf16_bits(s);
    }
  }
}

// ---------------------------------------------------------------------------
// Per-tensor scale in ONE launch. Both kernels rotate every 256-group once,
// keep the rotated values in registers until the maximum of the whole tensor
// is known, then quantize them (no second read of X, no second rotation).
//
// rq_tiny: inputs of at most 64 groups (e.g. two rows of 3072). One block,
// one group per 16-lane segment (segments past the end redo the last group:
// same maximum, identical code bytes), maximum reduced in LDS.
//
// rq_onepass: the two-pass kernel's block -> data map (block b: 16 rows,
// U consecutive groups) with a grid of at most one block per CU, so that the
// whole grid is resident at once, and U of 1 or 2 (1 for the 16 and 64
// rotations). Measured against the two launches: 512 x 3072 with U = 2
// (192 blocks) 8.0 against 9.3 us, 32 x 3072 6.0 against 7.4 us; more
// groups per lane lose (a single wave per SIMD rotates them one after the
// other: 512 x 12288 with U = 6, 256 blocks, 13.5 against 11.0 us; two
// blocks per CU with U = 4, 13.1 us). The block maxima meet in the workspace:
//   bytes 0..7        epoch E (any initial value)
//   bytes 16..31      result {tag, maximum}
//   bytes 32 + 16 b   slot of block b {tag, maximum}
// Every block reads E first, then writes its maximum and then the tag
// mix(E + 1 + b 2^40) to its slot; block 0 waits for all tags, publishes the
// maximum with the tag mix(E + 1 + (2^20 - 1) 2^40) and moves E on by one;
// the other blocks wait for that tag. Every exchanged word is an agent-scope
// atomic (coherent across XCDs by itself), and a tag is stored only after
// the store of its maximum has completed (s_waitcnt): the order a release
// gives these stores, without the L2 write-back a release adds for ordinary
// stores, and without an L2 invalidation on the reading side (a release per
// block and an acquire per slot measured 14-22 us at 384-512 blocks, against
// 8-15 us). mix is a bijection
// of 64-bit words, so a slot left by an earlier call (a smaller epoch) never
// carries the expected tag, and any other leftover content does so with
// probability 2^-64: the workspace needs no clearing, also under graph replay
// (E lives in the workspace). Block 0 moves E on only after every block has
// written its slot, i.e. after every block has read E. One workspace serves
// one call at a time. Waits are bounded (about a second); a wait that runs out
// (a grid that could not be resident at once) yields NaN scales.
// ---------------------------------------------------------------------------

CR_DEV uint64_t mix64(uint64_t z) {   // SplitMix64 output function (a bijection)
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
CR_DEV uint64_t xtag(uint64_t e1, uint64_t id) { return mix64(e1 + (id << 40)); }
constexpr uint64_t XRESULT = 0xFFFFFull;
constexpr int XSPIN = 1 << 20;
// the stores before it have completed (and the compiler keeps them there)
CR_DEV void xstore_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
}
// loads after it are issued after the loads before it have returned
CR_DEV void xload_order() {
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}
struct XSlot {
  uint64_t tag;
  float m;
  uint32_t pad;
};

// scales and quantization multipliers of the per-tensor path from the maximum
// A of the rotated tensor (NaN: the exchange ran out of time)
template <int QT, bool DUAL, int NR>
CR_DEV void write_tensor_scales(const RQParams& a, float A) {
  const float qmax = (QT == CR_Q_SYM_INT8) ? 127.f : 7.f;
  const bool lost = !(A >= 0.f);
  const float sc = lost ? __int_as_float(0x7fc00000) : (A > 0.f) ? __fmul_rn(div_rn(A, qmax), RotSize<NR>::inv_sqrt) : 0.f;
  reinterpret_cast<float*>(a.scales)[0] = sc;
  if constexpr (DUAL) {
    const float sc8 = lost ? __int_as_float(0x7fc00000) : (A > 0.f) ? __fmul_rn(div_rn(A, 127.f), RotSize<NR>::inv_sqrt) : 0.f;
    reinterpret_cast<float*>(a.scales8)[0] = sc8;
  }
}

template <int QT, bool DUAL, int NR>
__global__ __launch_bounds__(1024) void rq_tiny_kernel(RQParams a) {
  static_assert(NR != 1024, "the 1024 rotation spans four groups of a segment");
  __shared__ float red[16];
  const int tid = threadIdx.x;
  const int seg = tid >> 4;
  const LaneRot lr = lane_rot<NR>(tid & 15);
  const float qmax = (QT == CR_Q_SYM_INT8) ? 127.f : 7.f;
  const int G = a.G;
  const int u = min(seg, (int)(a.rows * G) - 1);
  const int64_t row = u / G;
  const int grp = u % G;
  const uint16_t* px = a.x + row * a.ldx + grp * 256 + lr.gL * 16;
  u32x4 w[2];
  w[0] = *reinterpret_cast<const u32x4*>(px);
  w[1] = *reinterpret_cast<const u32x4*>(px + 8);
  float v[16];
  rotate_group<NR>(w, lr, v);
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 16; e += 2) m = amax3(m, fabsf(v[e]), fabsf(v[e + 1]));
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  float A = red[0];
  const int nw = (int)(blockDim.x >> 6);
  for (int i = 1; i < nw; ++i) A = fmaxf(A, red[i]);
  if (tid == 0) write_tensor_scales<QT, DUAL, NR>(a, A);
  const float rq = lr.tau * ((A > 0.f) ? div_rn(qmax, A) : 0.f);
  store_codes<QT>(v, rq, a, row, grp, lr.gL);
  if constexpr (DUAL) {
    RQParams a8 = a;
    a8.codes = a.codes8;
    const float rq8 = lr.tau * ((A > 0.f) ? div_rn(127.f, A) : 0.f);
    quant_store<CR_Q_SYM_INT8>(v, rq8, code_dst<CR_Q_SYM_INT8>(a8, row, grp, lr.gL));
  }
}

template <int QT, bool DUAL, int U, int NR>
__global__ __launch_bounds__(256) void rq_onepass_kernel(RQParams a) {
  static_assert(NR != 1024, "the 1024 rotation takes the two-pass kernel");
  __shared__ float red[4];
  __shared__ float gmax;
  __shared__ uint64_t ep;
  const int tid = threadIdx.x;
  const int seg = tid >> 4;
  const LaneRot lr = lane_rot<NR>(tid & 15);
  const float qmax = (QT == CR_Q_SYM_INT8) ? 127.f : 7.f;
  const int G = a.G;
  const int GC = (G + U - 1) / U;
  const int64_t row = imin64((int64_t)(blockIdx.x / (unsigned)GC) * 16 + seg, a.rows - 1);
  const int g0 = (int)(blockIdx.x % (unsigned)GC) * U;
  const uint16_t* xr = a.x + row * a.ldx + lr.gL * 16;
  char* wsb = reinterpret_cast<char*>(a.ws);
  uint64_t* E = reinterpret_cast<uint64_t*>(wsb);
  XSlot* res = reinterpret_cast<XSlot*>(wsb + 16);
  XSlot* slot = reinterpret_cast<XSlot*>(wsb + 32);

  if (tid == 0) ep = __hip_atomic_load(E, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int grp[U];
  u32x4 w[U][2];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    grp[j] = min(g0 + j, G - 1);   // past the end: the last group again
    const uint16_t* px = xr + grp[j] * 256;
    w[j][0] = *reinterpret_cast<const u32x4*>(px);
    w[j][1] = *reinterpret_cast<const u32x4*>(px + 8);
  }
  __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use
  float v[U][16];
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < U; ++j) {
    rotate_group<NR>(w[j], lr, v[j]);
#pragma unroll
    for (int e = 0; e < 16; e += 2) m = amax3(m, fabsf(v[j][e]), fabsf(v[j][e + 1]));
  }
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const uint64_t e1 = ep + 1;
  if (tid == 0) {
    const float bm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __hip_atomic_store(&slot[blockIdx.x].m, bm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    xstore_order();
    __hip_atomic_store(&slot[blockIdx.x].tag, xtag(e1, blockIdx.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (blockIdx.x == 0) {
    float g = 0.f;
    bool ok = true;
    for (int i = tid; i < (int)gridDim.x; i += 256) {
      const uint64_t want = xtag(e1, (uint64_t)i);
      int k = 0;
      while (__hip_atomic_load(&slot[i].tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want && ++k < XSPIN)
        __builtin_amdgcn_s_sleep(2);
      ok = ok && k < XSPIN;
      xload_order();
      g = fmaxf(g, __hip_atomic_load(&slot[i].m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    g = wave_max(g);
    __syncthreads();   // red[] of the block maximum is read
    if ((tid & 63) == 0) red[tid >> 6] = g;
    const int lost = __syncthreads_or(!ok);
    if (tid == 0) {
      float A = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      if (lost) A = __int_as_float(0x7fc00000);
      gmax = A;
      __hip_atomic_store(&res->m, A, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      xstore_order();
      __hip_atomic_store(&res->tag, xtag(e1, XRESULT), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(E, e1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      write_tensor_scales<QT, DUAL, NR>(a, A);
    }
  } else if (tid == 0) {
    const uint64_t want = xtag(e1, XRESULT);
    int k = 0;
    while (__hip_atomic_load(&res->tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want && ++k < XSPIN)
      __builtin_amdgcn_s_sleep(2);
    xload_order();
    gmax = (k < XSPIN) ? __hip_atomic_load(&res->m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : __int_as_float(0x7fc00000);
  }
  __syncthreads();
  const float A = gmax;
  const float rq = lr.tau * ((A > 0.f) ? div_rn(qmax, A) : 0.f);
  const float rq8 = lr.tau * ((A > 0.f) ? div_rn(127.f, A) : 0.f);   // DUAL only
  RQParams a8 = a;
  a8.codes = a.codes8;
  if (QT == CR_Q_SYM_INT4 && a.tiled == 2) {
    // fp6 fragments: two groups per conversion, every lane of the row active
#pragma unroll
    for (int j = 0; j < U; j += 2) {
      const int j1 = (j + 1 < U) ? j + 1 : j;
      uint32_t w45[2];
      const u32x4 o = f6_pack2(v[j], rq, v[j1], rq, w45);
      f6_store_pair(o[0], o[1], o[2], a, row, grp[j], lr.gL);
      if (j + 1 < U) f6_store_pair(o[3], w45[0], w45[1], a, row, grp[j1], lr.gL);
      if constexpr (DUAL) {
        quant_store<CR_Q_SYM_INT8>(v[j], rq8, code_dst<CR_Q_SYM_INT8>(a8, row, grp[j], lr.gL));
        if (j + 1 < U) quant_store<CR_Q_SYM_INT8>(v[j1], rq8, code_dst<CR_Q_SYM_INT8>(a8, row, grp[j1], lr.gL));
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      store_codes<QT>(v[j], rq, a, row, grp[j], lr.gL);
      if constexpr (DUAL) quant_store<CR_Q_SYM_INT8>(v[j], rq8, code_dst<CR_Q_SYM_INT8>(a8, row, grp[j], lr.gL));
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// Block geometry: spr segments per row, gps groups per segment, rpb rows per
// block (16 / spr). ROW granularity needs a whole row per block.
RQGeometry rq_geometry(int64_t rows, int64_t K, int gran_kind, int nr) {
  RQGeometry g{};
  const int64_t G = K / 256;
  // chunks per segment: any for the 256 rotation; 1 or 4 for 16 and 64 (fewer
  // kernel instances); 4 for 1024 (one whole group per segment)
  const int cand_gps[5] = {1, 2, 3, 4, 8};
  double best = -1.0;
  for (int lg = 0; lg <= 4; ++lg) {
    const int spr = 1 << lg;
    for (int c = 0; c < 5; ++c) {
      const int gps = cand_gps[c];
      if (nr == 1024 && gps != 4) continue;
      if ((nr == 16 || nr == 64) && gps != 1 && gps != 4) continue;
      const int64_t slots = (int64_t)spr * gps;
      if (gran_kind == 2 && slots < G) continue;           // ROW: the row must fit
      const int64_t gx = (G + slots - 1) / slots;
      double util = (double)G / (double)(gx * slots);
      // prefer 3-4 groups per segment (loads in flight, fewer blocks) on ties
      double score = util + (gps >= 3 && gps <= 4 ? 1e-3 : 0.0) + (gx == 1 ? 1e-4 : 0.0);
      if (score > best) {
        best = score;
        g.gps = gps;
        g.lg_spr = lg;
        g.gx = gx;
      }
    }
  }
  g.rpb = 16 >> g.lg_spr;
  g.gy = (rows + g.rpb - 1) / g.rpb;
  g.nblk = g.gx * g.gy;
  return g;
}

template <int QT, int GR, int GPS, int NR>
static hipError_t launch_rot(const RQParams& p, const RQGeometry& g, hipStream_t s) {
  hipLaunchKernelGGL((rq_rot_kernel<QT, GR, GPS, NR>), dim3((unsigned)g.gy, (unsigned)g.gx), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int QT, int GR, int NR>
static hipError_t launch_rot_gps(const RQParams& p, const RQGeometry& g, hipStream_t s) {
  if constexpr (NR == 1024) {
    return launch_rot<QT, GR, 4, NR>(p, g, s);
  } else if constexpr (NR != 256) {
    if (g.gps == 4) return launch_rot<QT, GR, 4, NR>(p, g, s);
    return launch_rot<QT, GR, 1, NR>(p, g, s);
  } else {
    switch (g.gps) {
      case 1: return launch_rot<QT, GR, 1, NR>(p, g, s);
      case 2: return launch_rot<QT, GR, 2, NR>(p, g, s);
      case 3: return launch_rot<QT, GR, 3, NR>(p, g, s);
      case 8: return launch_rot<QT, GR, 8, NR>(p, g, s);
      default: return launch_rot<QT, GR, 4, NR>(p, g, s);
    }
  }
}

static int rq_tensor_j(int64_t rows, int64_t K, int nr) {
  const int64_t units = ((rows + 15) / 16) * (K / 256);
  if (nr == 1024) return 4;                       // one whole group per segment
  if (nr != 256) return units >= 2 * 256 ? 4 : 1;
  if (units >= 4 * 512) return 4;
  if (units >= 2 * 256) return 2;
  return 1;
}
// compute units of the current device (cached per device)
static int device_cus() {
  static std::mutex mu;
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(mu);
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

// one-pass groups per segment: the smallest whose grid fits the cap
static int onepass_u(int64_t rb, int64_t G, int nr, int64_t cap) {
  const int umax = (nr == 256) ? 2 : 1;
  for (int u = 1; u <= umax; ++u)
    if (rb * ((G + u - 1) / u) <= cap) return u;
  return 0;
}

TensorPlan rq_tensor_plan(int64_t rows, int64_t K, int nr) {
  const int64_t G = K / 256;
  const int64_t rb = (rows + 15) / 16;
  if (nr != 1024) {
    if (rows * G <= TINY_UNITS) return TensorPlan{RQT_TINY, 1, 1};
    const int64_t cap = std::min<int64_t>((int64_t)device_cus(), kOnepassMaxBlocks);
    const int u = onepass_u(rb, G, nr, cap);
    if (u > 0) return TensorPlan{RQT_ONEPASS, u, (int)(rb * ((G + u - 1) / u))};
  }
  return TensorPlan{RQT_TWOPASS, rq_tensor_j(rows, K, nr), rq_tensor_grid(rows, K, nr)};
}

int rq_tensor_launches(int64_t rows, int64_t K, int nr) {
  return rq_tensor_plan(rows, K, nr).kind == RQT_TWOPASS ? 2 : 1;
}

size_t rq_tensor_ws_bytes(int64_t rows, int64_t K, int nr) {
  const size_t two = (size_t)rq_tensor_grid(rows, K, nr) * sizeof(float);
  if (nr == 1024) return two;
  // any one-pass grid is at most the one of a single group per segment
  const int64_t nb1 = ((rows + 15) / 16) * (K / 256);
  const size_t one = 32 + 16 * (size_t)std::min<int64_t>(nb1, kOnepassMaxBlocks);
  return std::max(two, one);
}

// resident blocks per CU of a one-pass instance (its grid needs one)
template <typename KF>
static int blocks_per_cu(KF kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess) return 0;
  return n;
}

template <int QT, bool DUAL, int U, int NR>
static hipError_t launch_onepass_u(const RQParams& p, int nb, hipStream_t s) {
  static const int occ = blocks_per_cu(rq_onepass_kernel<QT, DUAL, U, NR>);
  if (occ < 1) return hipErrorLaunchOutOfResources;   // the exchange needs the whole grid resident
  hipLaunchKernelGGL((rq_onepass_kernel<QT, DUAL, U, NR>), dim3((unsigned)nb), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int QT, bool DUAL, int NR>
static hipError_t launch_tensor_onepass(const RQParams& p, const TensorPlan& t, hipStream_t s) {
  if constexpr (NR == 256) {
    if (t.u == 2) return launch_onepass_u<QT, DUAL, 2, NR>(p, t.nb, s);
  }
  return launch_onepass_u<QT, DUAL, 1, NR>(p, t.nb, s);
}

template <int QT, bool DUAL, int NR>
static hipError_t launch_tensor_tiny(const RQParams& p, hipStream_t s) {
  const int threads = (int)(((p.rows * p.G * 16) + 63) / 64 * 64);   // 16 lanes per group, whole waves
  hipLaunchKernelGGL((rq_tiny_kernel<QT, DUAL, NR>), dim3(1), dim3((unsigned)threads), 0, s, p);
  return hipGetLastError();
}
int rq_tensor_grid(int64_t rows, int64_t K, int nr) {   // blocks of each pass (one workspace float each)
  const int J = rq_tensor_j(rows, K, nr);
  const int64_t G = K / 256;
  return (int)(((rows + 15) / 16) * ((G + J - 1) / J));
}

template <int QT, int PASS, int J, int NR>
static void launch_tensor_j(const RQParams& p, int gd, hipStream_t s) {
  const int nws = (p.nblk + 255) / 256;
  if (PASS == 0 || nws <= 1) hipLaunchKernelGGL((rq_tensor_kernel<QT, PASS, J, 1, NR>), dim3(gd), dim3(256), 0, s, p);
  else if (nws <= 4) hipLaunchKernelGGL((rq_tensor_kernel<QT, PASS, J, 4, NR>), dim3(gd), dim3(256), 0, s, p);
  else if (nws <= 16) hipLaunchKernelGGL((rq_tensor_kernel<QT, PASS, J, 16, NR>), dim3(gd), dim3(256), 0, s, p);
  else if (nws <= 32) hipLaunchKernelGGL((rq_tensor_kernel<QT, PASS, J, 32, NR>), dim3(gd), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((rq_tensor_kernel<QT, PASS, J, 0, NR>), dim3(gd), dim3(256), 0, s, p);
}

template <int QT, int PASS, int NR>
static hipError_t launch_tensor(const RQParams& p, int gd, int J, hipStream_t s) {
  if constexpr (NR == 1024) {
    launch_tensor_j<QT, PASS, 4, NR>(p, gd, s);
  } else if constexpr (NR != 256) {
    if (J == 4) launch_tensor_j<QT, PASS, 4, NR>(p, gd, s);
    else launch_tensor_j<QT, PASS, 1, NR>(p, gd, s);
  } else {
    switch (J) {
      case 1: launch_tensor_j<QT, PASS, 1, NR>(p, gd, s); break;
      case 2: launch_tensor_j<QT, PASS, 2, NR>(p, gd, s); break;
      case 8: launch_tensor_j<QT, PASS, 8, NR>(p, gd, s); break;
      default: launch_tensor_j<QT, PASS, 4, NR>(p, gd, s); break;
    }
  }
  return hipGetLastError();
}

// rotated paths for one rotation size: per tensor (two launches), per row,
// per 64-group; asymmetric g16 weights only with the 256 rotation
template <int NR>
static hipError_t launch_rotated(RQParams p, hipStream_t s) {
  if constexpr (NR == 256) {
    if (p.qtype == CR_Q_ASYM_UINT4) {
      RQGeometry g = rq_geometry(p.rows, p.K, RG_ASYM, NR);
      p.lg_spr = g.lg_spr;
      p.rpb = g.rpb;
      return launch_rot_gps<CR_Q_ASYM_UINT4, RG_ASYM, NR>(p, g, s);
    }
  }
  if (p.gran == CR_GRAN_TENSOR) {
    if constexpr (NR != 1024) {
      const TensorPlan t = rq_tensor_plan(p.rows, p.K, NR);
      if (t.kind == RQT_TINY) {
        if (p.qtype == CR_Q_SYM_INT4) return launch_tensor_tiny<CR_Q_SYM_INT4, false, NR>(p, s);
        return launch_tensor_tiny<CR_Q_SYM_INT8, false, NR>(p, s);
      }
      if (t.kind == RQT_ONEPASS) {
        if (p.qtype == CR_Q_SYM_INT4) return launch_tensor_onepass<CR_Q_SYM_INT4, false, NR>(p, t, s);
        return launch_tensor_onepass<CR_Q_SYM_INT8, false, NR>(p, t, s);
      }
    }
    const int gd = rq_tensor_grid(p.rows, p.K, NR);
    const int J = rq_tensor_j(p.rows, p.K, NR);
    p.nblk = gd;
    hipError_t e;
    if (p.qtype == CR_Q_SYM_INT4) {
      e = launch_tensor<CR_Q_SYM_INT4, 0, NR>(p, gd, J, s);
      if (e != hipSuccess) return e;
      return launch_tensor<CR_Q_SYM_INT4, 1, NR>(p, gd, J, s);
    }
    e = launch_tensor<CR_Q_SYM_INT8, 0, NR>(p, gd, J, s);
    if (e != hipSuccess) return e;
    return launch_tensor<CR_Q_SYM_INT8, 1, NR>(p, gd, J, s);
  }
  const int kind = (p.gran == CR_GRAN_ROW) ? RG_ROW : RG_G64;
  RQGeometry g = rq_geometry(p.rows, p.K, kind, NR);
  p.lg_spr = g.lg_spr;
  p.rpb = g.rpb;
  if constexpr (NR == 256) {
    if (p.smooth) {   // 1 or 4 chunks per segment (the choice the 16 / 64 rotations make)
      g = rq_geometry(p.rows, p.K, kind, 16);
      p.lg_spr = g.lg_spr;
      p.rpb = g.rpb;
      const dim3 grid((unsigned)g.gy, (unsigned)g.gx);
      if (g.gps == 4) {
        if (kind == RG_ROW) {
          if (p.qtype == CR_Q_SYM_INT4) hipLaunchKernelGGL((rq_rot_kernel<CR_Q_SYM_INT4, RG_ROW, 4, 256, true>), grid, dim3(256), 0, s, p);
          else hipLaunchKernelGGL((rq_rot_kernel<CR_Q_SYM_INT8, RG_ROW, 4, 256, true>), grid, dim3(256), 0, s, p);
        } else {
          if (p.qtype == CR_Q_SYM_INT4) hipLaunchKernelGGL((rq_rot_kernel<CR_Q_SYM_INT4, RG_G64, 4, 256, true>), grid, dim3(256), 0, s, p);
          else hipLaunchKernelGGL((rq_rot_kernel<CR_Q_SYM_INT8, RG_G64, 4, 256, true>), grid, dim3(256), 0, s, p);
        }
      } else {
        if (kind == RG_ROW) {
          if (p.qtype == CR_Q_SYM_INT4) hipLaunchKernelGGL((rq_rot_kernel<CR_Q_SYM_INT4, RG_ROW, 1, 256, true>), grid, dim3(256), 0, s, p);
          else hipLaunchKernelGGL((rq_rot_kernel<CR_Q_SYM_INT8, RG_ROW, 1, 256, true>), grid, dim3(256), 0, s, p);
        } else {
          if (p.qtype == CR_Q_SYM_INT4) hipLaunchKernelGGL((rq_rot_kernel<CR_Q_SYM_INT4, RG_G64, 1, 256, true>), grid, dim3(256), 0, s, p);
          else hipLaunchKernelGGL((rq_rot_kernel<CR_Q_SYM_INT8, RG_G64, 1, 256, true>), grid, dim3(256), 0, s, p);
        }
      }
      return hipGetLastError();
    }
  }
  if (kind == RG_ROW) {
    if (p.qtype == CR_Q_SYM_INT4) return launch_rot_gps<CR_Q_SYM_INT4, RG_ROW, NR>(p, g, s);
    return launch_rot_gps<CR_Q_SYM_INT8, RG_ROW, NR>(p, g, s);
  }
  if (p.qtype == CR_Q_SYM_INT4) return launch_rot_gps<CR_Q_SYM_INT4, RG_G64, NR>(p, g, s);
  return launch_rot_gps<CR_Q_SYM_INT8, RG_G64, NR>(p, g, s);
}

template <int NR>
static hipError_t launch_dual(RQParams p, hipStream_t s) {
  if constexpr (NR != 1024) {
    const TensorPlan t = rq_tensor_plan(p.rows, p.K, NR);
    if (t.kind == RQT_TINY) return launch_tensor_tiny<CR_Q_SYM_INT4, true, NR>(p, s);
    if (t.kind == RQT_ONEPASS) return launch_tensor_onepass<CR_Q_SYM_INT4, true, NR>(p, t, s);
  }
  const int gd = rq_tensor_grid(p.rows, p.K, NR);
  const int J = rq_tensor_j(p.rows, p.K, NR);
  p.nblk = gd;
  hipError_t e = launch_tensor<CR_Q_SYM_INT4, 0, NR>(p, gd, J, s);
  if (e != hipSuccess) return e;
  return launch_tensor<CR_Q_SYM_INT4, 2, NR>(p, gd, J, s);
}

hipError_t launch_rotate_quantize_dual(RQParams p, hipStream_t s) {
  p.G = (int)(p.K / 256);
  switch (p.rot_group) {
    case 16: return launch_dual<16>(p, s);
    case 64: return launch_dual<64>(p, s);
    case 1024: return launch_dual<1024>(p, s);
    default: return launch_dual<256>(p, s);
  }
}

template <bool UNSIGNED, bool SM, int LAY, int RPB>
static hipError_t launch_plain_rpb(const RQParams& p, bool lora, hipStream_t s) {
  const dim3 grid((unsigned)((p.rows + RPB - 1) / RPB)), block(4 * RPB / 16 * 64);
  if (!lora)
    hipLaunchKernelGGL((rq_plain_kernel<UNSIGNED, false, 32, true, SM, LAY, RPB>), grid, block, 0, s, p);
  else if (p.R == 64)
    hipLaunchKernelGGL((rq_plain_kernel<UNSIGNED, true, 64, true, SM, LAY, 16>), dim3((unsigned)((p.rows + 15) / 16)),
                       dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((rq_plain_kernel<UNSIGNED, true, 32, true, SM, LAY, RPB>), grid, block, 0, s, p);
  return hipGetLastError();
}
// 32-row blocks (each low-rank fragment read from L2 serves two 16-row
// tiles) once they still give one block per CU; 16-row blocks otherwise
template <bool UNSIGNED, bool SM, int LAY>
static hipError_t launch_plain_lay(const RQParams& p, bool lora, hipStream_t s) {
  if ((p.rows + 31) / 32 >= 256) return launch_plain_rpb<UNSIGNED, SM, LAY, 32>(p, lora, s);
  return launch_plain_rpb<UNSIGNED, SM, LAY, 16>(p, lora, s);
}
template <bool UNSIGNED, bool SM>
static hipError_t launch_plain(const RQParams& p, int nblk, bool lora, hipStream_t s) {
  (void)nblk;
  if (p.tiled == 2) return launch_plain_lay<UNSIGNED, SM, 2>(p, lora, s);
  if (p.tiled == 1) return launch_plain_lay<UNSIGNED, SM, 1>(p, lora, s);
  return launch_plain_lay<UNSIGNED, SM, 0>(p, lora, s);
}

hipError_t launch_rotate_quantize(RQParams p, hipStream_t s) {
  const int nblk = (int)((p.rows + 15) / 16);
  const bool lora = p.lora_down != nullptr;
  if (p.rot_group == 0) {
    if (p.smooth) {
      if (p.qtype == CR_Q_UNSIGNED_INT4_SHIFT) return launch_plain<true, true>(p, nblk, lora, s);
      return launch_plain<false, true>(p, nblk, lora, s);
    }
    if (p.qtype == CR_Q_UNSIGNED_INT4_SHIFT) return launch_plain<true, false>(p, nblk, lora, s);
    return launch_plain<false, false>(p, nblk, lora, s);
  }
  p.G = (int)(p.K / 256);
  hipError_t e;
  switch (p.rot_group) {
    case 16: e = launch_rotated<16>(p, s); break;
    case 64: e = launch_rotated<64>(p, s); break;
    case 1024: e = launch_rotated<1024>(p, s); break;
    default: e = launch_rotated<256>(p, s); break;
  }
  if (e != hipSuccess || !lora) return e;
  // the low-rank down-projection reads the unrotated input: one more launch
  if (p.R == 64) hipLaunchKernelGGL((rq_plain_kernel<false, true, 64, false>), dim3(nblk), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((rq_plain_kernel<false, true, 32, false>), dim3(nblk), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace cr
