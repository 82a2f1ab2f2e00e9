// Internal interface between the C-ABI host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/convrot.h"

namespace cr {

struct RQParams {
  const uint16_t* x;
  int64_t rows, K, ldx;
  int rot_group, qtype, gran, q_group;
  float shift;
  const uint16_t* lora_down;
  int R;
  void* lora_act;
  int lora_f32;
  void* codes;
  void* scales;
  void* zeros;
  float* ws;            // TENSOR: block maxima (two-pass) or the one-pass exchange area
  int nblk;             // blocks of the TENSOR passes
  int G;                // 256-groups per row
  int rpb;              // rows per block (16 >> lg_spr)
  int lg_spr;           // log2(16-lane segments per row)
  int tiled;            // int4 codes: 0 natural, 1 [rows/16][K/64][512 B] int8-core fragments,
                        // 2 fp6 E2M3 fragments [rows/32][K/64][1536 B]; int8 codes: 3 fp16 values [rows, K]
  void* codes8;         // dual output: int8 codes [rows, K] (codes / scales hold the int4 set)
  void* scales8;
  const float* smooth;  // optional per-channel multiplier [K] applied to x first
};

struct RQGeometry {
  int gps;       // 256-groups per 16-lane segment
  int lg_spr;    // log2(segments per row)
  int rpb;       // rows per block
  int64_t gx, gy, nblk;  // grid (group tiles x row tiles) and its size
};

// gran_kind: 2 ROW (whole rows per block), 3 ROW_GROUP(64), 4 ASYM(16); nr: rotation group size
RQGeometry rq_geometry(int64_t rows, int64_t K, int gran_kind, int nr);
// blocks of each pass of the two-pass per-tensor kernel (one float of workspace each)
int rq_tensor_grid(int64_t rows, int64_t K, int nr);
// per-tensor rotate+quantize on the current device: one block (TINY), one
// launch with a grid-wide exchange of block maxima (ONEPASS, u groups per
// segment, nb blocks) or two launches (TWOPASS)
enum { RQT_TINY = 0, RQT_ONEPASS = 1, RQT_TWOPASS = 2 };
struct TensorPlan {
  int kind, u, nb;
};
TensorPlan rq_tensor_plan(int64_t rows, int64_t K, int nr);
// launches of a per-tensor rotate+quantize on the current device (1 or 2)
int rq_tensor_launches(int64_t rows, int64_t K, int nr);
// largest grid of the one-pass kernel (also at most one block per CU)
constexpr int kOnepassMaxBlocks = 2048;
// workspace bytes of a per-tensor rotate+quantize, whichever plan a device takes
size_t rq_tensor_ws_bytes(int64_t rows, int64_t K, int nr);
hipError_t launch_rotate_quantize(RQParams p, hipStream_t s);
// device address of this GPU's fixed scratch array for the allocation-free
// rotate+quantize (kNoallocScratchFloats block maxima)
constexpr int kNoallocScratchFloats = 65536;
hipError_t rq_noalloc_scratch(float** out);
// per-tensor INT4 and INT8 codes of one rotation (plan as rq_tensor_plan)
hipError_t launch_rotate_quantize_dual(RQParams p, hipStream_t s);

struct PackParams {
  const uint8_t* codes;
  const void* scales;
  const uint8_t* zeros;
  int64_t N, K;
  int qtype, gran, q_group;
  uint8_t* packed;
  void* packed_scales;
  uint8_t* packed_zeros;
  float* w_sum;
};
hipError_t launch_pack(const PackParams& p, hipStream_t s);
// natural int4 [N, K/2] -> fp6 E2M3 fragments [N/32][K/64][1536 B]
hipError_t launch_pack_f6(const uint8_t* codes, int64_t N, int64_t K, uint8_t* packed, hipStream_t s);
// low-rank up-projection L1 [N, R] bf16 -> tiled [N/128][R][128]
hipError_t launch_pack_lora_up(const uint16_t* up, int64_t N, int R, uint16_t* out, hipStream_t s);
// tile-packed int4 [N/128][K/64][4096 B] -> fp6 E2M3 fragments [N/32][K/64][1536 B]
hipError_t launch_expand_f6(const uint8_t* tiles, int64_t N, int64_t K, uint8_t* packed, hipStream_t s);

struct MergeParams {
  const uint8_t* codes;      // natural codes: int4 [N, K/2] (SYM_INT4, ASYM_UINT4) or int8 [N, K]
  const void* scales;        // float32 [1] / [N] / [N, K/64]; fp16 [N, K/16] for ASYM_UINT4
  const uint8_t* zeros;      // ASYM_UINT4: [N, K/32]
  int64_t N, K;
  int qtype, gran, rot_group;
  const uint16_t* up;        // optional bf16 [N, R]
  const uint16_t* down;      // bf16 [R, K]
  int R;
  uint16_t* out;             // bf16 [N, K]
};
hipError_t launch_merge(const MergeParams& p, hipStream_t s);

enum ActKind { ACT_S4 = 0, ACT_U4 = 1, ACT_I8 = 2 };
enum WgtKind { WGT_S4T = 0, WGT_I8N = 1 };

struct GemmParams {
  const uint8_t* a;          // activation codes
  const float* a_scales;
  int a_gran;
  int act;                   // ActKind
  float a_shift;
  const uint8_t* w;          // tile-packed int4 or natural int8
  const float* w_scales;
  int w_gran;
  int wgt;                   // WgtKind
  const float* w_sum;
  const void* lora_act;
  int lora_f32;
  const uint16_t* lora_up;   // L1, tiled [N/128][R][128] bf16
  int R;
  const uint16_t* bias;
  void* out;
  int out_type;
  int64_t ldc;
  int64_t M, N, K;
  int grouped;               // ROW_GROUP(64) x ROW_GROUP(64)
  int a_tiled;               // int4 activation codes in the [M/16][K/64][512 B] layout
  // W4A8 only
  const uint16_t* w_scales16;
  const uint8_t* w_zeros;
  int a_f16;                 // int8 activation codes carried as fp16 values [M, K]
  int k_lo, k_hi;            // W4A8 int32 output: k-tiles [k_lo, k_hi) of this launch (k_hi 0: all)
};
hipError_t launch_gemm_int(const GemmParams& p, hipStream_t s);   // INT8 x INT8
hipError_t launch_gemm_a8w4(const GemmParams& p, hipStream_t s);  // INT8 x tile-packed INT4
hipError_t launch_gemm_w4a4(const GemmParams& p, hipStream_t s);  // INT4 x tile-packed INT4
hipError_t launch_gemm_w4a8(const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_f6(const GemmParams& p, hipStream_t s);    // fp6 fragments x fp6 fragments

}  // namespace cr
