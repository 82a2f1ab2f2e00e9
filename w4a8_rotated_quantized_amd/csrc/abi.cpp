// C-ABI host layer: argument validation (before any HIP call), device /
// architecture check, dispatch to the gfx950 kernels, status strings and
// dispatch counters.
//
// "Qwen3-4B ConvRot W4A4" page, Hardware: a converter that runs only when the
// native kernels resolve, because a dequantizing backend would silently stand
// in for them; "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4" page, Runtime
// requirement: an unsupported format fails with a clear "format not
// available" error. Both are this layer's conventions: no fallback exists,
// unsupported inputs return a status. Dispatch counting follows the kernel
// call / dequantize counts of the Qwen3-4B page ("What it actually looks like").
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/convrot.h"
#include "kernels.h"

namespace {

std::atomic<uint64_t> g_launch[8];
thread_local int g_last_hip = 0;

enum { E_RQ = 0, E_PACK = 1, E_W4A4 = 2, E_W4A8 = 3, E_INT8 = 4 };

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

cr_status hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return CR_ERR_HIP;
}

// per-device cache: 0 unknown, 1 gfx950, 2 other
std::mutex g_dev_mu;
int g_dev_kind[64];

cr_status device_check() {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return CR_ERR_NO_DEVICE;
  }
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return CR_ERR_NO_DEVICE;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_kind[dev] == 0) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return hip_fail(e);
      g_dev_kind[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    if (g_dev_kind[dev] != 1) return CR_ERR_UNSUPPORTED_ARCH;
  }
  return CR_OK;
}

// CONVROT_LOG=1 in the environment (read once per process): one line on
// stderr for every call that enqueues work, with the entry point, its sizes
// and format arguments (as each entry tags them) and the kernels enqueued.
bool log_on() {
  static const bool on = [] {
    const char* v = std::getenv("CONVROT_LOG");
    return v && v[0] == '1' && v[1] == 0;
  }();
  return on;
}
struct CallInfo {
  const char* name;
  long long d[3];
  int f[3];
};
thread_local CallInfo g_call{};
struct CallTag {   // first statement of an entry point that enqueues work
  CallTag(const char* name, int64_t d0, int64_t d1, int64_t d2, int f0 = 0, int f1 = 0, int f2 = 0) {
    g_call = CallInfo{name, {(long long)d0, (long long)d1, (long long)d2}, {f0, f1, f2}};
  }
};

cr_status finish_launch(hipError_t e, int entry, uint64_t n) {
  if (log_on() && g_call.name)
    std::fprintf(stderr, "[convrot] %s sizes %lld %lld %lld formats %d %d %d: %llu kernel(s), %s\n", g_call.name,
                 g_call.d[0], g_call.d[1], g_call.d[2], g_call.f[0], g_call.f[1], g_call.f[2],
                 (unsigned long long)n, e == hipSuccess ? "enqueued" : hipGetErrorString(e));
  if (e != hipSuccess) return hip_fail(e);
  g_launch[entry].fetch_add(n, std::memory_order_relaxed);
  return CR_OK;
}

constexpr int64_t KMAX = 32768;
constexpr int64_t DIM_MAX = (int64_t)1 << 31;

}  // namespace

extern "C" {

const char* convrot_status_string(cr_status s) {
  switch (s) {
    case CR_OK: return "ok";
    case CR_ERR_INVALID_ARGUMENT: return "invalid argument";
    case CR_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case CR_ERR_UNSUPPORTED_FORMAT: return "format not available";
    case CR_ERR_NO_DEVICE: return "no HIP device";
    case CR_ERR_UNSUPPORTED_ARCH: return "device is not gfx950 (MI355X); no fallback path exists";
    case CR_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case CR_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int convrot_last_hip_error(void) { return g_last_hip; }

cr_status convrot_device_check(void) { return device_check(); }

void convrot_get_counters(cr_counters* out) {
  if (!out) return;
  for (int i = 0; i < 8; ++i) out->launches[i] = g_launch[i].load(std::memory_order_relaxed);
  out->fallbacks = 0;
}

void convrot_reset_counters(void) {
  for (int i = 0; i < 8; ++i) g_launch[i].store(0, std::memory_order_relaxed);
}

// ---------------------------------------------------------------------------
// rotate + quantize
// ---------------------------------------------------------------------------
static cr_status rq_validate(const void* x, int64_t rows, int64_t K, int64_t ldx, int rot_group,
                             cr_qtype qtype, cr_gran gran, int q_group, const void* lora_down, int R,
                             const void* lora_act, const void* codes, const void* scales, const void* zeros) {
  if (!x || !codes || !scales) return CR_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return CR_ERR_INVALID_ARGUMENT;
  if ((int)qtype < 0 || (int)qtype > 3 || (int)gran < 0 || (int)gran > 2) return CR_ERR_INVALID_ARGUMENT;
  if (rows < 1 || K < 1 || ldx < K || rows >= DIM_MAX || ldx >= DIM_MAX) return CR_ERR_UNSUPPORTED_SHAPE;
  if (ldx % 8 != 0 || K > KMAX) return CR_ERR_UNSUPPORTED_SHAPE;
  if (rot_group != 0 && rot_group != 16 && rot_group != 64 && rot_group != 256 && rot_group != 1024)
    return CR_ERR_UNSUPPORTED_FORMAT;
  if (lora_down) {
    if (R != 32 && R != 64) return CR_ERR_UNSUPPORTED_FORMAT;
    if (!lora_act || !aligned16(lora_down) || !aligned16(lora_act)) return CR_ERR_INVALID_ARGUMENT;
    if (qtype == CR_Q_ASYM_UINT4) return CR_ERR_UNSUPPORTED_FORMAT;   // weights have no low-rank input branch
  }
  if (rot_group != 0) {
    if (K % 256 != 0 || K % rot_group != 0) return CR_ERR_UNSUPPORTED_SHAPE;
    if (qtype == CR_Q_SYM_INT4 || qtype == CR_Q_SYM_INT8) {
      if (gran == CR_GRAN_ROW_GROUP && q_group != 64) return CR_ERR_UNSUPPORTED_FORMAT;
    } else if (qtype == CR_Q_ASYM_UINT4) {
      if (rot_group != 256) return CR_ERR_UNSUPPORTED_FORMAT;   // the W4A8 format is defined with 256
      if (gran != CR_GRAN_ROW_GROUP || q_group != 16) return CR_ERR_UNSUPPORTED_FORMAT;
      if (!zeros || !aligned16(zeros)) return CR_ERR_INVALID_ARGUMENT;
    } else {
      return CR_ERR_UNSUPPORTED_FORMAT;   // the shift path is for unrotated post-GELU inputs
    }
  } else {
    if (K % 64 != 0) return CR_ERR_UNSUPPORTED_SHAPE;
    if (!(qtype == CR_Q_SYM_INT4 || qtype == CR_Q_UNSIGNED_INT4_SHIFT)) return CR_ERR_UNSUPPORTED_FORMAT;
    if (gran != CR_GRAN_ROW_GROUP || q_group != 64) return CR_ERR_UNSUPPORTED_FORMAT;
  }
  return CR_OK;
}

size_t convrot_rq_workspace_size(int64_t rows, int64_t K, int rot_group, cr_qtype qtype, cr_gran gran,
                                 int q_group) {
  (void)q_group;
  if (rot_group == 0 || gran != CR_GRAN_TENSOR || rows < 1 || K < 256 || K % 256) return 0;
  if (rows >= DIM_MAX || K > KMAX) return 0;   // shapes convrot_rotate_quantize refuses
  if (!(rot_group == 16 || rot_group == 64 || rot_group == 256 || (rot_group == 1024 && K % 1024 == 0))) return 0;
  if (!(qtype == CR_Q_SYM_INT4 || qtype == CR_Q_SYM_INT8)) return 0;
  return cr::rq_tensor_ws_bytes(rows, K, rot_group);
}

// noalloc: the block maxima go to the library's fixed device scratch array
// (the workspace arguments are ignored)
static cr_status rotate_quantize_impl(const void* x, int64_t rows, int64_t K, int64_t ldx, int rot_group,
                                      cr_qtype qtype, cr_gran gran, int q_group, float shift, const float* smooth,
                                      const void* lora_down, int R, void* lora_act, int lora_act_f32,
                                      void* codes, cr_layout layout, void* scales, void* zeros, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream, bool noalloc) {
  cr_status st = rq_validate(x, rows, K, ldx, rot_group, qtype, gran, q_group, lora_down, R, lora_act,
                             codes, scales, zeros);
  if (st != CR_OK) return st;
  if (!((int)layout == CR_LAYOUT_NATURAL || (int)layout == CR_LAYOUT_TILED || (int)layout == CR_LAYOUT_F6 ||
        (int)layout == CR_LAYOUT_F16))
    return CR_ERR_INVALID_ARGUMENT;
  if (layout == CR_LAYOUT_TILED && !(qtype == CR_Q_SYM_INT4 || qtype == CR_Q_UNSIGNED_INT4_SHIFT))
    return CR_ERR_UNSUPPORTED_FORMAT;
  if (layout == CR_LAYOUT_F16) {   // rotated SYM_INT8 codes as fp16 values (the W4A8 activation operand)
    if (qtype != CR_Q_SYM_INT8 || rot_group == 0) return CR_ERR_UNSUPPORTED_FORMAT;
    if (rows * K * 2 >= ((int64_t)1 << 40)) return CR_ERR_UNSUPPORTED_SHAPE;
  }
  if (layout == CR_LAYOUT_F6) {   // signed INT4 codes, or unsigned shifted ones (unrotated); rows pad to 32
    if (!(qtype == CR_Q_SYM_INT4 || qtype == CR_Q_UNSIGNED_INT4_SHIFT)) return CR_ERR_UNSUPPORTED_FORMAT;
    if (((rows + 31) / 32) * (K / 64) * 1536 >= ((int64_t)1 << 32)) return CR_ERR_UNSUPPORTED_SHAPE;
  }
  if (smooth) {   // without rotation, or the 256 rotation with per-row / per-64-group scales
    if (!aligned16(smooth)) return CR_ERR_INVALID_ARGUMENT;
    if (rot_group != 0 && !(rot_group == 256 && (gran == CR_GRAN_ROW || gran == CR_GRAN_ROW_GROUP) &&
                            (qtype == CR_Q_SYM_INT4 || qtype == CR_Q_SYM_INT8)))
      return CR_ERR_UNSUPPORTED_FORMAT;
  }
  const size_t need = convrot_rq_workspace_size(rows, K, rot_group, qtype, gran, q_group);
  if (noalloc) {
    if (need > (size_t)cr::kNoallocScratchFloats * sizeof(float)) return CR_ERR_WORKSPACE_TOO_SMALL;
  } else if (need > 0) {
    if (!workspace || !aligned16(workspace)) return CR_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < need) return CR_ERR_WORKSPACE_TOO_SMALL;
  }
  st = device_check();
  if (st != CR_OK) return st;
  if (noalloc && need > 0) {
    float* sp = nullptr;
    const hipError_t e = cr::rq_noalloc_scratch(&sp);
    if (e != hipSuccess) return hip_fail(e);
    workspace = sp;
  }
  cr::RQParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.rows = rows;
  p.K = K;
  p.ldx = ldx;
  p.rot_group = rot_group;
  p.qtype = qtype;
  p.gran = gran;
  p.q_group = q_group;
  p.shift = shift;
  p.smooth = smooth;
  p.lora_down = static_cast<const uint16_t*>(lora_down);
  p.R = R;
  p.lora_act = lora_act;
  p.lora_f32 = lora_act_f32;
  p.codes = codes;
  p.scales = scales;
  p.zeros = zeros;
  p.ws = static_cast<float*>(workspace);
  p.tiled = layout == CR_LAYOUT_TILED ? 1 : (layout == CR_LAYOUT_F6 ? 2 : (layout == CR_LAYOUT_F16 ? 3 : 0));
  const uint64_t nl = ((rot_group != 0 && gran == CR_GRAN_TENSOR && qtype != CR_Q_ASYM_UINT4)
                           ? (uint64_t)cr::rq_tensor_launches(rows, K, rot_group) : 1) +
                      ((rot_group != 0 && lora_down) ? 1 : 0);
  return finish_launch(cr::launch_rotate_quantize(p, stream), E_RQ, nl);
}

cr_status convrot_rotate_quantize(const void* x, int64_t rows, int64_t K, int64_t ldx, int rot_group,
                                  cr_qtype qtype, cr_gran gran, int q_group, float shift, const float* smooth,
                                  const void* lora_down, int R, void* lora_act, int lora_act_f32,
                                  void* codes, cr_layout layout, void* scales, void* zeros, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  CallTag tag_("convrot_rotate_quantize", rows, K, rot_group, qtype, gran, layout);
  return rotate_quantize_impl(x, rows, K, ldx, rot_group, qtype, gran, q_group, shift, smooth, lora_down, R,
                              lora_act, lora_act_f32, codes, layout, scales, zeros, workspace, workspace_bytes,
                              stream, false);
}

cr_status convrot_rotate_quantize_noalloc(const void* x, int64_t rows, int64_t K, int64_t ldx, int rot_group,
                                          cr_qtype qtype, cr_gran gran, int q_group, float shift,
                                          const float* smooth, const void* lora_down, int R, void* lora_act,
                                          int lora_act_f32, void* codes, cr_layout layout, void* scales, void* zeros,
                                          hipStream_t stream) {
  CallTag tag_("convrot_rotate_quantize_noalloc", rows, K, rot_group, qtype, gran, layout);
  return rotate_quantize_impl(x, rows, K, ldx, rot_group, qtype, gran, q_group, shift, smooth, lora_down, R,
                              lora_act, lora_act_f32, codes, layout, scales, zeros, nullptr, 0, stream, true);
}

cr_status convrot_rotate_quantize_dual(const void* x, int64_t rows, int64_t K, int64_t ldx, int rot_group,
                                       void* codes4, cr_layout layout4, float* scale4, void* codes8, float* scale8,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CallTag tag_("convrot_rotate_quantize_dual", rows, K, rot_group, layout4);
  if (rot_group == 0) return CR_ERR_UNSUPPORTED_FORMAT;       // the per-tensor rotated path only
  cr_status st = rq_validate(x, rows, K, ldx, rot_group, CR_Q_SYM_INT4, CR_GRAN_TENSOR, 0, nullptr, 0, nullptr,
                             codes4, scale4, nullptr);
  if (st != CR_OK) return st;
  if (!codes8 || !scale8 || !aligned16(codes8) || !aligned16(scale8)) return CR_ERR_INVALID_ARGUMENT;
  if (!((int)layout4 == CR_LAYOUT_NATURAL || (int)layout4 == CR_LAYOUT_TILED || (int)layout4 == CR_LAYOUT_F6))
    return CR_ERR_INVALID_ARGUMENT;
  if (layout4 == CR_LAYOUT_F6 && ((rows + 31) / 32) * (K / 64) * 1536 >= ((int64_t)1 << 32))
    return CR_ERR_UNSUPPORTED_SHAPE;
  const size_t need = convrot_rq_workspace_size(rows, K, rot_group, CR_Q_SYM_INT4, CR_GRAN_TENSOR, 0);
  if (!workspace || !aligned16(workspace)) return CR_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return CR_ERR_WORKSPACE_TOO_SMALL;
  st = device_check();
  if (st != CR_OK) return st;
  cr::RQParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.rows = rows;
  p.K = K;
  p.ldx = ldx;
  p.rot_group = rot_group;
  p.qtype = CR_Q_SYM_INT4;
  p.gran = CR_GRAN_TENSOR;
  p.codes = codes4;
  p.scales = scale4;
  p.codes8 = codes8;
  p.scales8 = scale8;
  p.ws = static_cast<float*>(workspace);
  p.tiled = layout4 == CR_LAYOUT_TILED ? 1 : (layout4 == CR_LAYOUT_F6 ? 2 : 0);
  return finish_launch(cr::launch_rotate_quantize_dual(p, stream), E_RQ,
                       (uint64_t)cr::rq_tensor_launches(rows, K, rot_group));
}

// ---------------------------------------------------------------------------
// weight dequantization (LoRA merge)
// ---------------------------------------------------------------------------
cr_status convrot_dequantize_weights(const void* codes, const void* scales, const void* zeros, int64_t N, int64_t K,
                                     cr_qtype qtype, cr_gran gran, int q_group, int rot_group,
                                     const void* delta_up, const void* delta_down, int R, void* out,
                                     hipStream_t stream) {
  CallTag tag_("convrot_dequantize_weights", N, K, rot_group, qtype, gran, q_group);
  if (!codes || !scales || !out) return CR_ERR_INVALID_ARGUMENT;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(out)) return CR_ERR_INVALID_ARGUMENT;
  if ((int)qtype < 0 || (int)qtype > 3 || (int)gran < 0 || (int)gran > 2) return CR_ERR_INVALID_ARGUMENT;
  if (N < 1 || K < 256 || K % 256 || K > KMAX || N >= DIM_MAX) return CR_ERR_UNSUPPORTED_SHAPE;
  if (rot_group != 0 && rot_group != 16 && rot_group != 64 && rot_group != 256 && rot_group != 1024)
    return CR_ERR_UNSUPPORTED_FORMAT;
  if (rot_group && K % rot_group) return CR_ERR_UNSUPPORTED_SHAPE;
  if (qtype == CR_Q_SYM_INT4) {
    if (gran == CR_GRAN_ROW_GROUP && q_group != 64) return CR_ERR_UNSUPPORTED_FORMAT;
  } else if (qtype == CR_Q_SYM_INT8) {
    if (gran == CR_GRAN_ROW_GROUP) return CR_ERR_UNSUPPORTED_FORMAT;
  } else if (qtype == CR_Q_ASYM_UINT4) {
    if (gran != CR_GRAN_ROW_GROUP || q_group != 16) return CR_ERR_UNSUPPORTED_FORMAT;
    if (rot_group != 0 && rot_group != 256) return CR_ERR_UNSUPPORTED_FORMAT;
    if (!zeros || !aligned16(zeros)) return CR_ERR_INVALID_ARGUMENT;
  } else {
    return CR_ERR_UNSUPPORTED_FORMAT;                 // activation-only format
  }
  if (delta_up || delta_down) {
    if (!delta_up || !delta_down || R < 1 || R > 256) return CR_ERR_INVALID_ARGUMENT;
    if (!aligned16(delta_up) || !aligned16(delta_down)) return CR_ERR_INVALID_ARGUMENT;
  }
  cr_status st = device_check();
  if (st != CR_OK) return st;
  cr::MergeParams p{};
  p.codes = static_cast<const uint8_t*>(codes);
  p.scales = scales;
  p.zeros = static_cast<const uint8_t*>(zeros);
  p.N = N;
  p.K = K;
  p.qtype = qtype;
  p.gran = gran;
  p.rot_group = rot_group;
  p.up = static_cast<const uint16_t*>(delta_up);
  p.down = static_cast<const uint16_t*>(delta_down);
  p.R = delta_up ? R : 0;
  p.out = static_cast<uint16_t*>(out);
  return finish_launch(cr::launch_merge(p, stream), E_PACK, 1);
}

// ---------------------------------------------------------------------------
// weight packing
// ---------------------------------------------------------------------------
size_t w4_packed_bytes(int64_t N, int64_t K, cr_qtype qtype, cr_gran gran, int q_group, int which) {
  if (N < 128 || K < 64 || N % 128 || K % 64 || K > KMAX || N >= DIM_MAX) return 0;
  switch (which) {
    case 0: return (size_t)(N * K / 2);
    case 1:
      if (qtype == CR_Q_ASYM_UINT4) return (size_t)(N * (K / 16) * 2);
      if (gran == CR_GRAN_ROW_GROUP && q_group == 64) return (size_t)(N * (K / 64) * 4);
      return 0;
    case 2: return qtype == CR_Q_ASYM_UINT4 ? (size_t)(N * (K / 16)) : 0;
  }
  return 0;
}

size_t w4_packed_f6_bytes(int64_t N, int64_t K) {
  if (N < 128 || K < 128 || N % 128 || K % 128 || K > KMAX || N >= DIM_MAX) return 0;
  return (size_t)((N / 32) * (K / 64) * 1536);
}

cr_status w4_pack_weights_f6(const void* codes, int64_t N, int64_t K, void* packed, hipStream_t stream) {
  CallTag tag_("w4_pack_weights_f6", N, K, 0);
  if (!codes || !packed || !aligned16(codes) || !aligned16(packed)) return CR_ERR_INVALID_ARGUMENT;
  if (N < 128 || K < 128 || N % 128 || K % 128 || K > KMAX || N >= DIM_MAX) return CR_ERR_UNSUPPORTED_SHAPE;
  if ((N / 32) * (K / 64) * 1536 >= ((int64_t)1 << 32)) return CR_ERR_UNSUPPORTED_SHAPE;
  cr_status st = device_check();
  if (st != CR_OK) return st;
  return finish_launch(cr::launch_pack_f6(static_cast<const uint8_t*>(codes), N, K, static_cast<uint8_t*>(packed),
                                          stream),
                       E_PACK, 1);
}

cr_status w4_pack_lora_up(const void* up, int64_t N, int R, void* packed, hipStream_t stream) {
  CallTag tag_("w4_pack_lora_up", N, R, 0);
  if (!up || !packed || !aligned16(up) || !aligned16(packed)) return CR_ERR_INVALID_ARGUMENT;
  if (N < 128 || N % 128 || N >= DIM_MAX) return CR_ERR_UNSUPPORTED_SHAPE;
  if (R != 32 && R != 64) return CR_ERR_UNSUPPORTED_FORMAT;
  cr_status st = device_check();
  if (st != CR_OK) return st;
  return finish_launch(cr::launch_pack_lora_up(static_cast<const uint16_t*>(up), N, R, static_cast<uint16_t*>(packed),
                                               stream),
                       E_PACK, 1);
}

cr_status w4_expand_weights_f6(const void* tiles, int64_t N, int64_t K, void* f6, hipStream_t stream) {
  CallTag tag_("w4_expand_weights_f6", N, K, 0);
  if (!tiles || !f6 || !aligned16(tiles) || !aligned16(f6)) return CR_ERR_INVALID_ARGUMENT;
  if (N < 128 || K < 128 || N % 128 || K % 128 || K > KMAX || N >= DIM_MAX) return CR_ERR_UNSUPPORTED_SHAPE;
  if ((N / 32) * (K / 64) * 1536 >= ((int64_t)1 << 32)) return CR_ERR_UNSUPPORTED_SHAPE;
  cr_status st = device_check();
  if (st != CR_OK) return st;
  return finish_launch(cr::launch_expand_f6(static_cast<const uint8_t*>(tiles), N, K, static_cast<uint8_t*>(f6), stream),
                       E_PACK, 1);
}

cr_status w4_pack_weights(const void* codes, const void* scales, const void* zeros, int64_t N, int64_t K,
                          cr_qtype qtype, cr_gran gran, int q_group, void* packed, void* packed_scales,
                          void* packed_zeros, float* w_sum, hipStream_t stream) {
  CallTag tag_("w4_pack_weights", N, K, 0, qtype, gran, q_group);
  if (!codes || !packed || !scales) return CR_ERR_INVALID_ARGUMENT;
  if (!aligned16(codes) || !aligned16(packed) || !aligned16(scales)) return CR_ERR_INVALID_ARGUMENT;
  if ((int)qtype < 0 || (int)qtype > 3 || (int)gran < 0 || (int)gran > 2) return CR_ERR_INVALID_ARGUMENT;
  if (N < 128 || K < 64 || N % 128 || K % 64 || K > KMAX || N >= DIM_MAX) return CR_ERR_UNSUPPORTED_SHAPE;
  if (qtype == CR_Q_SYM_INT4) {
    if (gran == CR_GRAN_ROW_GROUP) {
      if (q_group != 64) return CR_ERR_UNSUPPORTED_FORMAT;
      if (!packed_scales || !aligned16(packed_scales)) return CR_ERR_INVALID_ARGUMENT;
    }
    if (w_sum && !aligned16(w_sum)) return CR_ERR_INVALID_ARGUMENT;
  } else if (qtype == CR_Q_ASYM_UINT4) {
    if (gran != CR_GRAN_ROW_GROUP || q_group != 16) return CR_ERR_UNSUPPORTED_FORMAT;
    if (!zeros || !packed_scales || !packed_zeros) return CR_ERR_INVALID_ARGUMENT;
    if (!aligned16(zeros) || !aligned16(packed_scales) || !aligned16(packed_zeros)) return CR_ERR_INVALID_ARGUMENT;
    if (w_sum) return CR_ERR_INVALID_ARGUMENT;             // the W4A8 GEMM needs no column sums
  } else {
    return CR_ERR_UNSUPPORTED_FORMAT;
  }
  cr_status st = device_check();
  if (st != CR_OK) return st;
  cr::PackParams p{};
  p.codes = static_cast<const uint8_t*>(codes);
  p.scales = scales;
  p.zeros = static_cast<const uint8_t*>(zeros);
  p.N = N;
  p.K = K;
  p.qtype = qtype;
  p.gran = gran;
  p.q_group = q_group;
  p.packed = static_cast<uint8_t*>(packed);
  p.packed_scales = packed_scales;
  p.packed_zeros = static_cast<uint8_t*>(packed_zeros);
  p.w_sum = w_sum;
  uint64_t nl = 1 + (qtype == CR_Q_ASYM_UINT4 ? 1 : 0) + (gran == CR_GRAN_ROW_GROUP && qtype == CR_Q_SYM_INT4) +
                (w_sum ? 1 : 0);
  return finish_launch(cr::launch_pack(p, stream), E_PACK, nl);
}

// ---------------------------------------------------------------------------
// GEMMs
// ---------------------------------------------------------------------------
static cr_status gemm_common(const void* a, const void* w, const void* out, cr_out out_type, int64_t ldc,
                             int64_t M, int64_t N, int64_t K, const void* bias) {
  if (!a || !w || !out) return CR_ERR_INVALID_ARGUMENT;
  if (!aligned16(a) || !aligned16(w) || !aligned16(out)) return CR_ERR_INVALID_ARGUMENT;
  if (bias && !aligned16(bias)) return CR_ERR_INVALID_ARGUMENT;
  if ((int)out_type < 0 || (int)out_type > 2) return CR_ERR_INVALID_ARGUMENT;
  if (M < 1 || N < 128 || K < 128 || N % 128 || K % 128 || K > KMAX) return CR_ERR_UNSUPPORTED_SHAPE;
  if (M >= DIM_MAX || N >= DIM_MAX || ldc < N || ldc % 8 != 0 || ldc >= DIM_MAX) return CR_ERR_UNSUPPORTED_SHAPE;
  return CR_OK;
}

size_t w4a4_gemm_workspace_size(int64_t N, int64_t K, cr_layout a_layout, cr_layout w_layout) {
  if (a_layout != CR_LAYOUT_F6 || w_layout != CR_LAYOUT_TILED) return 0;
  if (N < 128 || K < 128 || N % 128 || K % 128 || K > KMAX || N >= DIM_MAX) return 0;
  return (size_t)((N / 32) * (K / 64) * 1536);   // the weights as fp6 fragments
}

cr_status w4a4_gemm(const void* a_codes, cr_layout a_layout, const float* a_scales, cr_gran a_gran,
                    int a_unsigned, float a_shift,
                    const void* w_packed, cr_layout w_layout, const float* w_scales, cr_gran w_gran,
                    const float* w_sum, const void* lora_act, int lora_act_f32, const void* lora_up, int R,
                    const void* bias, void* out, cr_out out_type, int64_t ldc, int64_t M, int64_t N, int64_t K,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CallTag tag_("w4a4_gemm", M, N, K, a_layout, w_layout, out_type);
  cr_status st = gemm_common(a_codes, w_packed, out, out_type, ldc, M, N, K, bias);
  if (st != CR_OK) return st;
  if (!a_scales || !w_scales || !aligned16(a_scales) || !aligned16(w_scales)) return CR_ERR_INVALID_ARGUMENT;
  if ((int)a_gran < 0 || (int)a_gran > 2 || (int)w_gran < 0 || (int)w_gran > 2) return CR_ERR_INVALID_ARGUMENT;
  if ((int)a_layout < 0 || (int)a_layout > 3) return CR_ERR_INVALID_ARGUMENT;
  if (!((int)w_layout == CR_LAYOUT_TILED || (int)w_layout == CR_LAYOUT_F6)) return CR_ERR_INVALID_ARGUMENT;
  const bool a8 = a_layout == CR_LAYOUT_INT8;
  const bool f6 = a_layout == CR_LAYOUT_F6;
  if (w_layout == CR_LAYOUT_F6 && !f6) return CR_ERR_UNSUPPORTED_FORMAT;   // fp6 weights pair with fp6 codes
  if (f6) {   // fp6 fragments on both sides; unsigned codes and the low-rank branch with 64-group scales only
    if (a_gran != CR_GRAN_ROW_GROUP && (a_unsigned || lora_act || lora_up)) return CR_ERR_UNSUPPORTED_FORMAT;
    if (((M + 31) / 32) * (K / 64) * 1536 >= ((int64_t)1 << 32) || (N / 32) * (K / 64) * 1536 >= ((int64_t)1 << 32))
      return CR_ERR_UNSUPPORTED_SHAPE;
  }
  if (!f6 && (((M + 15) / 16) * 16 * (a8 ? K : K / 2) >= ((int64_t)1 << 32) || N * (K / 2) >= ((int64_t)1 << 32)))
    return CR_ERR_UNSUPPORTED_SHAPE;
  const bool grouped = a_gran == CR_GRAN_ROW_GROUP;
  if (grouped != (w_gran == CR_GRAN_ROW_GROUP)) return CR_ERR_UNSUPPORTED_FORMAT;
  if (a8 && (a_unsigned || grouped || lora_act || lora_up)) return CR_ERR_UNSUPPORTED_FORMAT;
  if (a_unsigned) {
    if (!w_sum || !aligned16(w_sum)) return CR_ERR_INVALID_ARGUMENT;
  }
  if (lora_act || lora_up) {
    if (!lora_act || !lora_up || (R != 32 && R != 64)) return CR_ERR_UNSUPPORTED_FORMAT;
    if (!aligned16(lora_act) || !aligned16(lora_up)) return CR_ERR_INVALID_ARGUMENT;
  }
  const size_t need = w4a4_gemm_workspace_size(N, K, a_layout, w_layout);
  if (need > 0) {
    if (!workspace || !aligned16(workspace)) return CR_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < need) return CR_ERR_WORKSPACE_TOO_SMALL;
  }
  st = device_check();
  if (st != CR_OK) return st;
  cr::GemmParams p{};
  p.a = static_cast<const uint8_t*>(a_codes);
  p.a_scales = a_scales;
  p.a_gran = a_gran;
  p.act = a8 ? cr::ACT_I8 : (a_unsigned ? cr::ACT_U4 : cr::ACT_S4);
  p.a_shift = a_shift;
  p.w = static_cast<const uint8_t*>(w_packed);
  p.w_scales = w_scales;
  p.w_gran = w_gran;
  p.wgt = cr::WGT_S4T;
  p.w_sum = w_sum;
  p.lora_act = lora_act;
  p.lora_f32 = lora_act_f32;
  p.lora_up = static_cast<const uint16_t*>(lora_up);
  p.R = R;
  p.bias = static_cast<const uint16_t*>(bias);
  p.out = out;
  p.out_type = out_type;
  p.ldc = ldc;
  p.M = M;
  p.N = N;
  p.K = K;
  p.grouped = grouped ? 1 : 0;
  p.a_tiled = a_layout == CR_LAYOUT_TILED ? 1 : 0;
  if (a8) return finish_launch(cr::launch_gemm_a8w4(p, stream), E_W4A4, 1);
  if (f6) {
    if (need > 0) {   // int4 tiles -> fp6 fragments in the workspace, then the fp6 GEMM on them
      hipError_t e = cr::launch_expand_f6(p.w, N, K, static_cast<uint8_t*>(workspace), stream);
      if (e != hipSuccess) return hip_fail(e);
      p.w = static_cast<const uint8_t*>(workspace);
    }
    return finish_launch(cr::launch_gemm_f6(p, stream), E_W4A4, need > 0 ? 2 : 1);
  }
  return finish_launch(cr::launch_gemm_w4a4(p, stream), E_W4A4, 1);
}

cr_status w4a8_gemm(const void* a_codes, cr_layout a_layout, const float* a_scales, cr_gran a_gran,
                    const void* w_packed, const void* w_scales, const void* w_zeros, int group,
                    const void* lora_act, int lora_act_f32, const void* lora_up, int R, const void* bias,
                    void* out, cr_out out_type, int64_t ldc, int64_t M, int64_t N, int64_t K, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  CallTag tag_("w4a8_gemm", M, N, K, a_layout, a_gran, out_type);
  (void)workspace;
  (void)workspace_bytes;
  cr_status st = gemm_common(a_codes, w_packed, out, out_type, ldc, M, N, K, bias);
  if (st != CR_OK) return st;
  if (!((int)a_layout == CR_LAYOUT_NATURAL || (int)a_layout == CR_LAYOUT_F16)) return CR_ERR_INVALID_ARGUMENT;
  if (!a_scales || !w_scales || !w_zeros) return CR_ERR_INVALID_ARGUMENT;
  if (!aligned16(a_scales) || !aligned16(w_scales) || !aligned16(w_zeros)) return CR_ERR_INVALID_ARGUMENT;
  if (lora_act || lora_up) {
    if (!lora_act || !lora_up || (R != 32 && R != 64)) return CR_ERR_UNSUPPORTED_FORMAT;
    if (!aligned16(lora_act) || !aligned16(lora_up)) return CR_ERR_INVALID_ARGUMENT;
  }
  if (group != 16) return CR_ERR_UNSUPPORTED_FORMAT;
  if (!(a_gran == CR_GRAN_ROW || a_gran == CR_GRAN_TENSOR)) return CR_ERR_UNSUPPORTED_FORMAT;
  if (M * K * (a_layout == CR_LAYOUT_F16 ? 2 : 1) >= ((int64_t)1 << 40)) return CR_ERR_UNSUPPORTED_SHAPE;
  st = device_check();
  if (st != CR_OK) return st;
  cr::GemmParams p{};
  p.a = static_cast<const uint8_t*>(a_codes);
  p.a_f16 = a_layout == CR_LAYOUT_F16 ? 1 : 0;
  p.a_scales = a_scales;
  p.a_gran = a_gran;
  p.act = cr::ACT_I8;
  p.w = static_cast<const uint8_t*>(w_packed);
  p.w_scales16 = static_cast<const uint16_t*>(w_scales);
  p.w_zeros = static_cast<const uint8_t*>(w_zeros);
  p.lora_act = lora_act;
  p.lora_f32 = lora_act_f32 ? 1 : 0;
  p.lora_up = static_cast<const uint16_t*>(lora_up);
  p.R = R;
  p.bias = static_cast<const uint16_t*>(bias);
  p.out = out;
  p.out_type = out_type;
  p.ldc = ldc;
  p.M = M;
  p.N = N;
  p.K = K;
  return finish_launch(cr::launch_gemm_w4a8(p, stream), E_W4A8, 1);
}

cr_status int8_tensorwise_gemm(const void* a_codes, const float* a_scale, const void* w, const float* w_scale,
                               const void* bias, void* out, cr_out out_type, int64_t ldc, int64_t M, int64_t N,
                               int64_t K, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CallTag tag_("int8_tensorwise_gemm", M, N, K, out_type);
  (void)workspace;
  (void)workspace_bytes;
  cr_status st = gemm_common(a_codes, w, out, out_type, ldc, M, N, K, bias);
  if (st != CR_OK) return st;
  if (!a_scale || !w_scale || !aligned16(a_scale) || !aligned16(w_scale)) return CR_ERR_INVALID_ARGUMENT;
  st = device_check();
  if (st != CR_OK) return st;
  cr::GemmParams p{};
  p.a = static_cast<const uint8_t*>(a_codes);
  p.a_scales = a_scale;
  p.a_gran = CR_GRAN_TENSOR;
  p.act = cr::ACT_I8;
  p.w = static_cast<const uint8_t*>(w);
  p.w_scales = w_scale;
  p.w_gran = CR_GRAN_TENSOR;
  p.wgt = cr::WGT_I8N;
  p.bias = static_cast<const uint16_t*>(bias);
  p.out = out;
  p.out_type = out_type;
  p.ldc = ldc;
  p.M = M;
  p.N = N;
  p.K = K;
  return finish_launch(cr::launch_gemm_int(p, stream), E_INT8, 1);
}

}  // extern "C"
