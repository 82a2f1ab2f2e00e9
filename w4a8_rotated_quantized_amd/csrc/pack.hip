// Weight packer (gfx950): natural int4 codes -> tile-packed fragments.
//
// "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Tile-Packed Weight Format:
// weights reorganised into an (N/128, K/64) grid of 32 x 128-byte tiles with
// (N/128, K/64, 128) group scales. "Qwen3-4B ConvRot W4A4" page, Format: the
// natural [rows, cols/2] INT4 container. Offline (once per layer).
//
// Inner tile orders (this library's choice: one matrix-core operand fragment
// of 64 lanes is contiguous):
//   SYM_INT4: tile byte nb*512 + l*8 + j <- natural byte (row 16 nb + l%16,
//             tile byte column 8 (l/16) + j)
//   ASYM_UINT4: tile byte kg*1024 + nb*256 + l*4 + i holds the nibbles of
//             k0 + i (low) and k0 + 4 + i (high), k0 = 16 kg + 8 (l/32), row
//             32 nb + l%32, so widening a lane's word gives natural k order.
#include "common.h"
#include "kernels.h"

namespace cr {

__global__ __launch_bounds__(256) void pack_sym_kernel(PackParams p) {
  const int64_t K = p.K;
  const int64_t chunks = p.N * K / 16;           // 8-byte chunks
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  // tile-order index: c = ((tile * 8 + nb) * 64 + l)
  const int l = (int)(c & 63);
  const int nb = (int)((c >> 6) & 7);
  const int64_t tile = c >> 9;
  const int64_t ktn = K / 64;
  const int64_t tn = tile / ktn, kt = tile % ktn;
  const int64_t row = tn * 128 + nb * 16 + (l & 15);
  const int64_t col = kt * 32 + (l >> 4) * 8;
  *reinterpret_cast<u32x2*>(p.packed + c * 8) =
      *reinterpret_cast<const u32x2*>(p.codes + row * (K / 2) + col);
}

__global__ __launch_bounds__(256) void pack_asym_kernel(PackParams p) {
  const int64_t K = p.K;
  const int64_t words = p.N * K / 8;             // 4-byte words
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= words) return;
  // c = ((tile * 4 + kg) * 4 + nb) * 64 + l
  const int l = (int)(c & 63);
  const int nb = (int)((c >> 6) & 3);
  const int kg = (int)((c >> 8) & 3);
  const int64_t tile = c >> 10;
  const int64_t ktn = K / 64;
  const int64_t tn = tile / ktn, kt = tile % ktn;
  const int64_t row = tn * 128 + nb * 32 + (l & 31);
  const int64_t k0 = kt * 64 + kg * 16 + (l >> 5) * 8;
  // natural bytes k0/2 .. k0/2+3 hold nibbles k0..k0+7 (even k low)
  const uint32_t x = *reinterpret_cast<const uint32_t*>(p.codes + row * (K / 2) + k0 / 2);
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = (x >> (4 * i)) & 0xF;        // k0 + i
    uint32_t hi = (x >> (4 * (i + 4))) & 0xF;  // k0 + 4 + i
    out |= (lo | (hi << 4)) << (8 * i);
  }
  reinterpret_cast<uint32_t*>(p.packed)[c] = out;
}

// g64 scales [N, K/64] -> [N/128][K/64][128]
__global__ __launch_bounds__(256) void pack_g64_scales_kernel(PackParams p) {
  const int64_t G = p.K / 64;
  const int64_t total = p.N * G;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= total) return;
  const int64_t i = c & 127, g = (c >> 7) % G, tn = (c >> 7) / G;
  reinterpret_cast<float*>(p.packed_scales)[c] =
      reinterpret_cast<const float*>(p.scales)[(tn * 128 + i) * G + g];
}

// g16 scales (fp16 [N, K/16]) and zeros (packed uint4 [N, K/32]) -> [N/128][K/64][4][128]
__global__ __launch_bounds__(256) void pack_g16_meta_kernel(PackParams p) {
  const int64_t G = p.K / 16;
  const int64_t total = p.N * G;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= total) return;
  const int64_t i = c & 127;
  const int64_t kg = (c >> 7) & 3;
  const int64_t tk = c >> 9;                      // tile index tn * (K/64) + kt
  const int64_t ktn = p.K / 64;
  const int64_t tn = tk / ktn, kt = tk % ktn;
  const int64_t row = tn * 128 + i;
  const int64_t g = kt * 4 + kg;
  reinterpret_cast<uint16_t*>(p.packed_scales)[c] = reinterpret_cast<const uint16_t*>(p.scales)[row * G + g];
  const uint8_t zb = p.zeros[row * (p.K / 32) + g / 2];
  p.packed_zeros[c] = (g & 1) ? (zb >> 4) : (zb & 0xF);
}

// w_sum[n] = sum_k dequantized weight, summed group by group in k order.
__global__ __launch_bounds__(256) void wsum_kernel(PackParams p) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= p.N) return;
  const int64_t K = p.K;
  const uint8_t* row = p.codes + n * (K / 2);
  const float* sc = reinterpret_cast<const float*>(p.scales);
  float acc = 0.f;
  if (p.gran == CR_GRAN_ROW_GROUP) {
    for (int64_t g = 0; g < K / 64; ++g) {
      int s = 0;
      for (int j = 0; j < 32; ++j) {
        int b = row[g * 32 + j];
        s += ((b & 0xF) ^ 8) - 8;
        s += ((b >> 4) ^ 8) - 8;
      }
      acc += (float)s * sc[n * (K / 64) + g];
    }
  } else {
    int s = 0;
    for (int64_t j = 0; j < K / 2; ++j) {
      int b = row[j];
      s += ((b & 0xF) ^ 8) - 8;
      s += ((b >> 4) ^ 8) - 8;
    }
    acc = (float)s * (p.gran == CR_GRAN_TENSOR ? sc[0] : sc[n]);
  }
  p.w_sum[n] = acc;
}

static inline unsigned nblocks(int64_t n) { return (unsigned)((n + 255) / 256); }

// Natural signed int4 codes -> the fp6 E2M3 fragment layout of the fp6
// matrix-core GEMM ([N/32][K/64][1536 B]; lane l of a fragment holds row
// l % 32, columns 32 (l / 32) .. +31 of its 64-deep k-tile as six-bit fields,
// bytes 0..15 at l * 16 and 16..23 at 1024 + l * 8). One thread per lane
// slot, consecutive threads on consecutive slots. Natural byte j holds
// columns 2j (low nibble) and 2j + 1 (high), and the conversion interleaves
// its two sources the same way (field 2i from the first, 2i + 1 from the
// second), so the fields come out in column order. Codes in [-7, 7] are
// E2M3 values; the conversion is exact.
__global__ __launch_bounds__(256) void pack_f6_kernel(const uint8_t* __restrict__ codes, int64_t N, int64_t K,
                                                      uint8_t* __restrict__ packed) {
  const int64_t KT = K / 64;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (N / 32) * KT * 64) return;     // one thread per fragment lane slot
  const int lm = (int)(c & 63);
  const int64_t rest = c >> 6;
  const int64_t kt = rest % KT, rb = rest / KT;
  const int64_t row = rb * 32 + (lm & 31);
  const u32x4 x = *reinterpret_cast<const u32x4*>(codes + row * (K / 2) + kt * 32 + (lm >> 5) * 16);
  v16f lo, hi;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t b = (x[j >> 2] >> (8 * (j & 3))) & 0xFFu;
    lo[j] = (float)((int)(b << 28) >> 28);
    hi[j] = (float)((int)(b << 24) >> 28);
  }
  const auto o = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(lo, hi, 1.0f);
  uint8_t* frag = packed + rest * 1536;
  *reinterpret_cast<u32x4*>(frag + lm * 16) = u32x4{o[0], o[1], o[2], o[3]};
  *reinterpret_cast<u32x2*>(frag + 1024 + lm * 8) = u32x2{o[4], o[5]};
}

// Tile-packed signed int4 weights (w4_pack_weights: [N/128][K/64][8][64
// lanes][8 B], lane l of 16-row block nb holding row 16 nb + l % 16 and the
// 16 codes k = 16 (l / 16) .. of the k-tile, two per byte in natural order)
// -> the fp6 fragments of the fp6 matrix-core GEMM. The GEMM runs this once
// per call into its workspace, so the weights stay at 4 bits per code in
// memory. Fragment lane l of 32-row block b (row 32 b + l % 32, codes
// 32 (l / 32) .. + 31 of the k-tile) is tile lanes 2 (l / 32) and
// 2 (l / 32) + 1 of 16-row block 2 (b % 4) + (l % 32) / 16 of tile b / 4:
// 16 bytes in natural order, converted as in pack_f6_kernel.
__global__ __launch_bounds__(256) void expand_f6_kernel(const uint8_t* __restrict__ tiles, int64_t N, int64_t K,
                                                        uint8_t* __restrict__ packed) {
  const int64_t KT = K / 64;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (N / 32) * KT * 64) return;     // one thread per fragment lane slot
  const int lm = (int)(c & 63);
  const int64_t rest = c >> 6;
  const int64_t kt = rest % KT, rb = rest / KT;
  const int r32 = lm & 31, h = lm >> 5;
  const uint8_t* tile = tiles + ((rb >> 2) * KT + kt) * 4096 + (2 * (rb & 3) + (r32 >> 4)) * 512;
  const u32x2 x0 = *reinterpret_cast<const u32x2*>(tile + (32 * h + (r32 & 15)) * 8);
  const u32x2 x1 = *reinterpret_cast<const u32x2*>(tile + (32 * h + 16 + (r32 & 15)) * 8);
  const u32x4 x = u32x4{x0[0], x0[1], x1[0], x1[1]};
  v16f lo, hi;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t b = (x[j >> 2] >> (8 * (j & 3))) & 0xFFu;
    lo[j] = (float)((int)(b << 28) >> 28);
    hi[j] = (float)((int)(b << 24) >> 28);
  }
  const auto o = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(lo, hi, 1.0f);
  uint8_t* frag = packed + rest * 1536;
  *reinterpret_cast<u32x4*>(frag + lm * 16) = u32x4{o[0], o[1], o[2], o[3]};
  *reinterpret_cast<u32x2*>(frag + 1024 + lm * 8) = u32x2{o[4], o[5]};
}

hipError_t launch_expand_f6(const uint8_t* tiles, int64_t N, int64_t K, uint8_t* packed, hipStream_t s) {
  hipLaunchKernelGGL(expand_f6_kernel, dim3(nblocks((N / 32) * (K / 64) * 64)), dim3(256), 0, s, tiles, N, K, packed);
  return hipGetLastError();
}

// L1 [N, R] bf16 -> [N/128][R][128]: one thread per output element (the
// writes are contiguous, the reads gather R-strided 2-byte entries)
__global__ __launch_bounds__(256) void pack_lora_up_kernel(const uint16_t* __restrict__ up, int64_t N, int R,
                                                           uint16_t* __restrict__ out) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= N * R) return;
  const int64_t tn = o / (128 * (int64_t)R);
  const int r = (int)((o / 128) % R);
  const int i = (int)(o % 128);
  out[o] = up[(tn * 128 + i) * R + r];
}

hipError_t launch_pack_lora_up(const uint16_t* up, int64_t N, int R, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(pack_lora_up_kernel, dim3(nblocks(N * R)), dim3(256), 0, s, up, N, R, out);
  return hipGetLastError();
}

hipError_t launch_pack_f6(const uint8_t* codes, int64_t N, int64_t K, uint8_t* packed, hipStream_t s) {
  hipLaunchKernelGGL(pack_f6_kernel, dim3(nblocks((N / 32) * (K / 64) * 64)), dim3(256), 0, s, codes, N, K, packed);
  return hipGetLastError();
}

hipError_t launch_pack(const PackParams& p, hipStream_t s) {
  if (p.qtype == CR_Q_ASYM_UINT4) {
    hipLaunchKernelGGL(pack_asym_kernel, dim3(nblocks(p.N * p.K / 8)), dim3(256), 0, s, p);
    hipLaunchKernelGGL(pack_g16_meta_kernel, dim3(nblocks(p.N * p.K / 16)), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(pack_sym_kernel, dim3(nblocks(p.N * p.K / 16)), dim3(256), 0, s, p);
  if (p.gran == CR_GRAN_ROW_GROUP)
    hipLaunchKernelGGL(pack_g64_scales_kernel, dim3(nblocks(p.N * p.K / 64)), dim3(256), 0, s, p);
  if (p.w_sum) hipLaunchKernelGGL(wsum_kernel, dim3(nblocks(p.N)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace cr
