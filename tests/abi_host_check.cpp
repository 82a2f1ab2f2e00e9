// Host-side check of the C-ABI layer, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_abi_sanitize_cpu.py (abi.cpp and
// this file instrumented; the kernel objects linked as built).
//
// It runs only where no HIP device is visible: every call then ends in
// argument validation or in the device check, so no kernel is launched and
// the fake addresses below are never dereferenced. Where a device is visible
// it prints "skipped" and calls nothing else.
//
// Coverage: every exported entry point over seeded random combinations of
// null, aligned and misaligned pointers, in-range and out-of-range enums,
// and sizes from 0 to 2^40 (negative ones included), plus the size queries
// over the same sizes; a handful of exact statuses are asserted. The
// sanitizers turn any out-of-bounds access, signed overflow or invalid shift
// in the host code into a failing exit.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "convrot.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {   // SplitMix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
template <typename T, size_t N>
T pick(const T (&a)[N]) { return a[next_u64() % N]; }

void* const A = reinterpret_cast<void*>(0x100000);          // aligned, never dereferenced
void* const MIS = reinterpret_cast<void*>(0x100004);        // misaligned
void* const PTRS[] = {nullptr, A, A, A, MIS};
const int64_t DIMS[] = {-1, 0, 1, 2, 17, 32, 64, 128, 255, 256, 512, 1024, 3072, 4096, 12288,
                        18432, 32768, 32769, 65536, (int64_t)1 << 31, (int64_t)1 << 40};
const int ENUMS[] = {-1, 0, 1, 2, 3, 4, 5, 99};
const int GROUPS[] = {-1, 0, 1, 16, 32, 64, 128, 256, 1024};
const int RANKS[] = {-1, 0, 16, 32, 64, 128};
const size_t WSB[] = {0, 16, 1u << 20, (size_t)1 << 40, ~(size_t)0};

int g_fail = 0;
long g_calls = 0;

void expect(cr_status got, cr_status want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d\n", what, (int)got, (int)want);
    g_fail = 1;
  }
}

void check(cr_status s, const char* what) {   // no device here: never CR_OK
  ++g_calls;
  if ((int)s < 1 || (int)s > 7) {
    std::printf("FAIL %s: status %d\n", what, (int)s);
    g_fail = 1;
  }
}

}  // namespace

int main() {
  if (convrot_device_check() != CR_ERR_NO_DEVICE) {
    std::printf("skipped: a HIP device is visible\n");
    return 0;
  }
  for (int s = -1; s <= 8; ++s)
    if (!convrot_status_string((cr_status)s)) g_fail = 1;
  convrot_get_counters(nullptr);
  cr_counters c;
  convrot_reset_counters();
  convrot_get_counters(&c);
  if (c.fallbacks != 0) g_fail = 1;
  (void)convrot_last_hip_error();

  // exact statuses of a few calls
  const float* F = static_cast<const float*>(A);
  expect(convrot_rotate_quantize(nullptr, 64, 512, 512, 256, CR_Q_SYM_INT4, CR_GRAN_TENSOR, 0, 0.f, nullptr, nullptr,
                                 0, nullptr, 0, A, CR_LAYOUT_NATURAL, A, nullptr, A, 1u << 20, nullptr),
         CR_ERR_INVALID_ARGUMENT, "rq null input");
  expect(convrot_rotate_quantize(A, 64, 500, 512, 256, CR_Q_SYM_INT4, CR_GRAN_TENSOR, 0, 0.f, nullptr, nullptr, 0,
                                 nullptr, 0, A, CR_LAYOUT_NATURAL, A, nullptr, A, 1u << 20, nullptr),
         CR_ERR_UNSUPPORTED_SHAPE, "rq K not a multiple of 256");
  expect(convrot_rotate_quantize(A, 64, 512, 512, 256, CR_Q_SYM_INT4, CR_GRAN_TENSOR, 0, 0.f, nullptr, nullptr, 0,
                                 nullptr, 0, A, CR_LAYOUT_NATURAL, A, nullptr, A, 1u << 20, nullptr),
         CR_ERR_NO_DEVICE, "rq valid");
  expect(int8_tensorwise_gemm(A, F, A, F, nullptr, A, CR_OUT_BF16, 3072, 64, 3072, 3072, nullptr, 0, nullptr),
         CR_ERR_NO_DEVICE, "int8 valid");
  expect(int8_tensorwise_gemm(A, F, A, F, nullptr, A, CR_OUT_BF16, 3072, 64, 3000, 3072, nullptr, 0, nullptr),
         CR_ERR_UNSUPPORTED_SHAPE, "int8 N not a multiple of 128");

  const int ROUNDS = 20000;
  for (int r = 0; r < ROUNDS; ++r) {
    const int64_t d0 = pick(DIMS), d1 = pick(DIMS), d2 = pick(DIMS);
    const int e0 = pick(ENUMS), e1 = pick(ENUMS), e2 = pick(ENUMS), e3 = pick(ENUMS);
    const int qg = pick(GROUPS), rot = pick(GROUPS), R = pick(RANKS);
    const size_t wsb = pick(WSB);
    const int64_t ld = (next_u64() & 1) ? d1 : pick(DIMS);

    (void)convrot_rq_workspace_size(d0, d1, rot, (cr_qtype)e0, (cr_gran)e1, qg);
    (void)w4_packed_bytes(d0, d1, (cr_qtype)e0, (cr_gran)e1, qg, e2);
    (void)w4_packed_f6_bytes(d0, d1);
    (void)w4a4_gemm_workspace_size(d0, d1, (cr_layout)e0, (cr_layout)e1);

    check(convrot_rotate_quantize(pick(PTRS), d0, d1, ld, rot, (cr_qtype)e0, (cr_gran)e1, qg, 0.171875f,
                                  static_cast<const float*>(pick(PTRS)), pick(PTRS), R, pick(PTRS), e2 & 1,
                                  pick(PTRS), (cr_layout)e3, pick(PTRS), pick(PTRS), pick(PTRS), wsb, nullptr),
          "convrot_rotate_quantize");
    check(convrot_rotate_quantize_noalloc(pick(PTRS), d0, d1, ld, rot, (cr_qtype)e0, (cr_gran)e1, qg, 0.f,
                                          static_cast<const float*>(pick(PTRS)), pick(PTRS), R, pick(PTRS), e2 & 1,
                                          pick(PTRS), (cr_layout)e3, pick(PTRS), pick(PTRS), nullptr),
          "convrot_rotate_quantize_noalloc");
    check(convrot_rotate_quantize_dual(pick(PTRS), d0, d1, ld, rot, pick(PTRS), (cr_layout)e3,
                                       static_cast<float*>(pick(PTRS)), pick(PTRS), static_cast<float*>(pick(PTRS)),
                                       pick(PTRS), wsb, nullptr),
          "convrot_rotate_quantize_dual");
    check(w4_pack_weights(pick(PTRS), pick(PTRS), pick(PTRS), d0, d1, (cr_qtype)e0, (cr_gran)e1, qg, pick(PTRS),
                          pick(PTRS), pick(PTRS), static_cast<float*>(pick(PTRS)), nullptr),
          "w4_pack_weights");
    check(w4_pack_weights_f6(pick(PTRS), d0, d1, pick(PTRS), nullptr), "w4_pack_weights_f6");
    check(w4_pack_lora_up(pick(PTRS), d0, R, pick(PTRS), nullptr), "w4_pack_lora_up");
    check(w4_expand_weights_f6(pick(PTRS), d0, d1, pick(PTRS), nullptr), "w4_expand_weights_f6");
    check(convrot_dequantize_weights(pick(PTRS), pick(PTRS), pick(PTRS), d0, d1, (cr_qtype)e0, (cr_gran)e1, qg, rot,
                                     pick(PTRS), pick(PTRS), R, pick(PTRS), nullptr),
          "convrot_dequantize_weights");
    check(w4a4_gemm(pick(PTRS), (cr_layout)e0, static_cast<const float*>(pick(PTRS)), (cr_gran)e1, e2 & 1, 0.171875f,
                    pick(PTRS), (cr_layout)e3, static_cast<const float*>(pick(PTRS)), (cr_gran)pick(ENUMS),
                    static_cast<const float*>(pick(PTRS)), pick(PTRS), (int)(next_u64() & 1), pick(PTRS), R,
                    pick(PTRS), pick(PTRS), (cr_out)pick(ENUMS), ld, d0, d1, d2, pick(PTRS), wsb, nullptr),
          "w4a4_gemm");
    check(w4a8_gemm(pick(PTRS), (cr_layout)e0, static_cast<const float*>(pick(PTRS)), (cr_gran)e1, pick(PTRS),
                    pick(PTRS), pick(PTRS), qg, pick(PTRS), e2 & 1, pick(PTRS), R, pick(PTRS), pick(PTRS),
                    (cr_out)e3, ld, d0, d1, d2, pick(PTRS), wsb, nullptr),
          "w4a8_gemm");
    check(int8_tensorwise_gemm(pick(PTRS), static_cast<const float*>(pick(PTRS)), pick(PTRS),
                               static_cast<const float*>(pick(PTRS)), pick(PTRS), pick(PTRS), (cr_out)e0, ld, d0, d1,
                               d2, pick(PTRS), wsb, nullptr),
          "int8_tensorwise_gemm");
  }
  convrot_get_counters(&c);
  for (int i = 0; i < 8; ++i)
    if (c.launches[i] != 0) {
      std::printf("FAIL launches counted without a device\n");
      g_fail = 1;
    }
  std::printf("%s: %ld calls\n", g_fail ? "FAILED" : "all ok", g_calls);
  return g_fail;
}
