/*
 * convrot.h - C ABI of the ConvRot-rotated low-bit quantized linear layer
 *             for AMD Instinct MI355X (gfx950).
 *
 * The method (from the pages this library follows, cited by title/section):
 *   - "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4 (+ConvRot, mixed int8
 *     fallback)", intro and Measurements: weights are packed signed INT4 (two
 *     per byte), rotated offline with a group-256 regular Hadamard (ConvRot);
 *     activations are rotated online with the same matrix and quantized
 *     dynamically; an INT8 tensorwise format serves the sensitive layers.
 *   - "Qwen-Image-Edit-2511-W4A8-ConvRot", build table / file layout:
 *     asymmetric 4-bit weights, group 16, ConvRot 256, 8-bit activations.
 *   - "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Quantization Method,
 *     Key Technical Optimizations, Kernel Engineering: the two-call structure
 *     (quantize, then scaled matmul), the tile-packed weight format
 *     (N/128, K/64, 32, 128) with (N/128, K/64, 128) group scales, a low-rank
 *     branch whose down-projection is computed once with the quantization
 *     and whose up-projection is fused into the GEMM epilogue, an unsigned
 *     post-GELU activation path shifted by +0.171875, and an FP32 switch for
 *     the low-rank activations.
 *   - "Qwen3-4B - ConvRot W4A4 (ComfyUI text encoder)", Format / Hardware:
 *     the [rows, cols/2] INT4 container with a float32 [rows] scale, and the
 *     rule that a missing native path is refused rather than replaced by
 *     dequantized math.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller. The library
 *     never allocates, frees or synchronizes; all work is enqueued on `stream`
 *     (NULL = the default stream) and returns immediately.
 *   - Arguments are validated BEFORE any HIP call. On any error nothing is
 *     enqueued and a status is returned; the library never aborts.
 *   - The device must be gfx950; otherwise CR_ERR_UNSUPPORTED_ARCH. There is
 *     no fallback path of any kind (no dequantized or CPU math).
 *   - bf16 = IEEE bfloat16 bit patterns; all matrices are row-major with the
 *     leading dimension in elements; every pointer must be 16-byte aligned.
 *   - int4 codes, natural layout: [rows, K/2] bytes, element 2j in the low
 *     nibble of byte j, element 2j+1 in the high nibble, two's complement for
 *     signed codes (unsigned 0..15 for unsigned / asymmetric codes).
 *   - Rotation: the unnormalised regular Hadamard H (entries +-1, H H^T =
 *     256 I, rows summing to 16, H = (D S D) with S Sylvester and D[j] =
 *     (-1)^(#zero base-4 digits of j)) is applied to each contiguous group of
 *     256 columns, in float32, in the butterfly order h = 1, 2, ..., 128.
 *     The orthonormal factor 1/16 is carried by the stored scale, so
 *     scale * code approximates the orthonormally rotated value.
 *   - Quantization (symmetric): A = max |v| over the scale group,
 *     r = fl32(qmax / A), code = clamp(rint_half_even(fl32(v * r)), -qmax,
 *     qmax), scale = fl32(A / qmax) (times 1/16 when rotated); an all-zero
 *     group has scale 0 and zero codes. qmax = 7 (INT4) or 127 (INT8).
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cr_status {
  CR_OK = 0,
  CR_ERR_INVALID_ARGUMENT = 1,    /* null / misaligned pointer, bad enum, negative size   */
  CR_ERR_UNSUPPORTED_SHAPE = 2,   /* K, N or group alignment not met, sizes out of range    */
  CR_ERR_UNSUPPORTED_FORMAT = 3,  /* "format not available": this qtype/granularity combo   */
  CR_ERR_NO_DEVICE = 4,           /* no HIP device visible                                  */
  CR_ERR_UNSUPPORTED_ARCH = 5,    /* current device is not gfx950: refused, no fallback     */
  CR_ERR_WORKSPACE_TOO_SMALL = 6, /* workspace_bytes below the *_workspace_size() result    */
  CR_ERR_HIP = 7                  /* a HIP runtime call failed; see convrot_last_hip_error() */
} cr_status;

typedef enum cr_qtype {
  CR_Q_SYM_INT4 = 0,             /* signed codes in [-7, 7], packed two per byte            */
  CR_Q_SYM_INT8 = 1,             /* signed codes in [-127, 127], one byte each              */
  CR_Q_UNSIGNED_INT4_SHIFT = 2,  /* codes of v + shift in [0, 15] (post-GELU path, no rotation) */
  CR_Q_ASYM_UINT4 = 3            /* weights only: uint4 codes, fp16 scale and uint4 zero per group of 16 */
} cr_qtype;

typedef enum cr_gran {
  CR_GRAN_TENSOR = 0,     /* one scale, float32 [1]                                          */
  CR_GRAN_ROW = 1,        /* one scale per row (token or output channel), float32 [rows]     */
  CR_GRAN_ROW_GROUP = 2   /* one per row and q_group columns: float32 [rows, K/q_group]      */
} cr_gran;

typedef enum cr_out {
  CR_OUT_BF16 = 0,        /* y rounded half-to-even to bf16                                   */
  CR_OUT_F32 = 1,         /* y as float32                                                     */
  CR_OUT_I32_RAW = 2      /* the exact integer sum_k qa*(qw - z); scales/epilogue skipped     */
} cr_out;

typedef enum cr_layout {
  CR_LAYOUT_NATURAL = 0,  /* int4 codes [rows, K/2], row-major                                 */
  CR_LAYOUT_TILED = 1,    /* int4 codes [ceil(rows/16)][K/64][512 B]: byte l*8 + j of block    */
                          /* (b, kt) is natural byte (row 16b + l%16, 32kt + 8(l/16) + j), the */
                          /* operand-fragment order of the W4A4 GEMM; rows past `rows` in the  */
                          /* last block hold unspecified codes (allocate ceil(rows/16)*16 rows)*/
  CR_LAYOUT_INT8 = 2,     /* w4a4_gemm only: int8 codes [rows, K] row-major (SYM_INT8), the    */
                          /* 8-bit-activation branch for W4A4-format weights                   */
  CR_LAYOUT_F6 = 3,       /* signed int4 codes (values -7..7) as fp6 E2M3 (bit 5 sign, bits    */
                          /* 4:3 exponent with bias 1, bits 2:0 mantissa; every code is exact; */
                          /* an unsigned code u in 0..15 is stored as the exact value u/2)     */
                          /* in 32 x 64 operand fragments [ceil(rows/32)][K/64][1536 B]: lane  */
                          /* l (0..63) of a fragment covers row 32b + l%32 and columns          */
                          /* 64kt + 32(l/32) + i, i = 0..31, field i at bits 6i..6i+5 of its 24 */
                          /* bytes, bytes 0..15 at l*16 and bytes 16..23 at 1024 + l*8. Input   */
                          /* of the fp6 matrix-core W4A4 GEMM (its weights in the same layout)  */
                          /* rows past `rows` in the last block hold unspecified codes (any     */
                          /* 6-bit field is a finite value; allocate ceil(rows/32)*32 rows)      */
  CR_LAYOUT_F16 = 4       /* SYM_INT8 codes as IEEE fp16 values [rows, K] row-major (every code */
                          /* -127..127 is exact; zero is +0): the activation operand of         */
                          /* w4a8_gemm's fp16 matrix cores, used without conversion              */
} cr_layout;

/* Status text, e.g. "format not available" for CR_ERR_UNSUPPORTED_FORMAT. */
const char* convrot_status_string(cr_status status);
/* The hipError_t value behind the last CR_ERR_HIP on this thread (0 if none). */
int convrot_last_hip_error(void);
/* CR_OK when a gfx950 device is current; CR_ERR_NO_DEVICE / CR_ERR_UNSUPPORTED_ARCH otherwise. */
cr_status convrot_device_check(void);

/* Dispatch counters: kernel launches per entry point (index = order of the
 * entry points below: 0 rotate_quantize, 1 pack, 2 w4a4, 3 w4a8, 4 int8)
 * and the count of non-native fallbacks, which is always 0 because no
 * fallback exists. Process-wide, thread-safe. */
typedef struct cr_counters {
  uint64_t launches[8];
  uint64_t fallbacks;
} cr_counters;
void convrot_get_counters(cr_counters* out);
void convrot_reset_counters(void);

/* Launch log: with CONVROT_LOG=1 in the environment (read once per process)
 * every call that enqueues work writes one line to stderr:
 *   [convrot] <entry point> sizes <a> <b> <c> formats <x> <y> <z>: <n> kernel(s), enqueued
 * sizes are (rows or M, K or N, rotation group or K) and formats the call's
 * enum arguments (quantizer type, granularity, layout; for the GEMMs the
 * layouts or granularity and the output type), as each entry lists them.
 * Calls refused by validation write nothing (their status says why). */

/* ------------------------------------------------------------------------
 * convrot_rotate_quantize - online rotation + dynamic quantization of
 * activations, and the offline rotation + quantization of weights.
 *
 * Cites: "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4" page, intro (rotate
 * online, quantize dynamically, same rotation offline on the weights);
 * "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Key Technical
 * Optimizations (quantization and LoRA-down computed once and shared by split
 * projections) and Kernel Engineering (unsigned +0.171875 post-GELU path,
 * LoRA-down staged in bf16); Environment Variables (FP32 LoRA activations).
 *
 *   x            bf16 [rows, K], leading dimension ldx >= K
 *   rot_group    256 (rotate each 256-column group with the regular Hadamard
 *                matrix of order 256), 16, 64 or 1024 (the other ConvRot group
 *                sizes of the W4A4 recipe: "Qwen-Image-Edit-2511-W4A8-ConvRot"
 *                card, group-size notes), or 0 (no rotation). The stored scale
 *                carries the factor 1/sqrt(rot_group).
 *   qtype/gran/q_group, supported combinations:
 *       rot 16/64/256/1024: SYM_INT4 or SYM_INT8 with TENSOR, ROW or
 *                ROW_GROUP(q_group 64);
 *       rot 256: also ASYM_UINT4 with ROW_GROUP(q_group 16)
 *       rot 0:   SYM_INT4 with ROW_GROUP(64); UNSIGNED_INT4_SHIFT with ROW_GROUP(64)
 *       anything else returns CR_ERR_UNSUPPORTED_FORMAT.
 *   shift        UNSIGNED_INT4_SHIFT only: codes quantize v + shift (e.g. 0.171875)
 *   smooth       optional float32 [K]: per-channel multiplier applied to x first,
 *                v = fl(x * smooth[k]), before the shift and the rotation (the
 *                smoothing factor of "Qwen-Image-Edit-2511 INT4 (ComfyUI
 *                Optimized)", Key Technical Optimizations, shared by split
 *                projections; the caller passes the multiplier the activation
 *                needs, the weight columns carry its inverse). Supported without
 *                rotation, and with the 256 rotation for ROW / ROW_GROUP(64)
 *                scales; elsewhere CR_ERR_UNSUPPORTED_FORMAT. The low-rank
 *                down-projection reads the unsmoothed input.
 *   lora_down    optional bf16 [R, K], R = 32 or 64 (not with ASYM_UINT4): also
 *                writes lora_act[m, r] = sum_k x[m, k] * lora_down[r, k] (float32
 *                accumulation of the unshifted, unrotated input), stored as
 *                bf16 (lora_act_f32 = 0) or float32 (1), [rows, R] row-major.
 *                Without rotation it is fused into the quantization pass; with
 *                rotation it is one more launch over the same input (the
 *                low-rank bypass of a LoRA kept beside quantized weights:
 *                "Qwen-Image-Edit-2511-W4A8-ConvRot" card, passage on LoRA merge
 *                versus bypass)
 *   codes        SYM_INT4 / UNSIGNED / ASYM: uint8 [rows, K/2] natural int4;
 *                SYM_INT8: int8 [rows, K] (CR_LAYOUT_F16: fp16 [rows, K])
 *   layout       CR_LAYOUT_NATURAL, or CR_LAYOUT_TILED for SYM_INT4 / UNSIGNED
 *                codes (the input layout of w4a4_gemm's int8-core path), or
 *                CR_LAYOUT_F6 for SYM_INT4 or UNSIGNED codes (the input of
 *                w4a4_gemm's fp6-core path; ceil(rows/32)(K/64) 1536 bytes;
 *                an unsigned code u is stored as the E2M3 value u/2), or
 *                CR_LAYOUT_F16 for rotated SYM_INT8 codes (the activation
 *                operand of w4a8_gemm, same integers as fp16 values)
 *   scales       float32 [1] | [rows] | [rows, K/q_group]; ASYM: fp16 [rows, K/16]
 *   zeros        ASYM only: uint8 [rows, K/32], two uint4 zero points per byte
 *                (group 2j low nibble); NULL otherwise
 *   workspace    device scratch of at least convrot_rq_workspace_size(...)
 *                (0 when the call needs none or refuses the shape)
 *                bytes (needed by TENSOR granularity; may be NULL when that
 *                size is 0). Per-tensor scaling takes one launch for inputs
 *                of at most 64 groups of 256 (one workgroup), one launch
 *                whose workgroups exchange their maxima through the
 *                workspace while the grid fits one workgroup per compute
 *                unit (e.g. 512 x 3072 on MI355X), else two launches (the
 *                first writes one maximum per workgroup there). Any contents
 *                on entry are valid: the exchange keeps an epoch counter in
 *                the workspace and tags every value it writes with it, so the
 *                workspace needs no clearing between calls (nor between
 *                replays of a captured graph). Calls sharing a workspace must
 *                not run concurrently. The exchange needs its whole grid
 *                resident at once (at most one workgroup of 4 waves per
 *                compute unit, so it shares the GPU with kernels on other
 *                streams); if other work kept compute units from it until
 *                its bounded wait (about a second) ended, the scale would
 *                come out NaN rather than the call hanging.
 * Shape: rows >= 1, K % 256 == 0 and K % rot_group == 0 when rotating,
 *        K % 64 == 0 otherwise, K <= 32768.
 * Result is deterministic and bit-identical to the reference definition for
 * finite inputs. Concurrent calls sharing one workspace race.
 */
size_t convrot_rq_workspace_size(int64_t rows, int64_t K, int rot_group,
                                 cr_qtype qtype, cr_gran gran, int q_group);

cr_status convrot_rotate_quantize(const void* x, int64_t rows, int64_t K, int64_t ldx,
                                  int rot_group, cr_qtype qtype, cr_gran gran, int q_group,
                                  float shift, const float* smooth,
                                  const void* lora_down, int R, void* lora_act, int lora_act_f32,
                                  void* codes, cr_layout layout, void* scales, void* zeros,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * convrot_rotate_quantize_noalloc - convrot_rotate_quantize for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, formats and results (bit for bit) as
 * convrot_rotate_quantize without the workspace pair: what the per-tensor
 * passes keep in the workspace (block maxima, the one-launch exchange) goes
 * to a fixed array of CONVROT_NOALLOC_SCRATCH_FLOATS
 * floats (256 KiB) in device memory that the library holds on each GPU it runs
 * on until the process ends. The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine). Inputs whose per-tensor pass
 * needs more block maxima than that, i.e. convrot_rq_workspace_size(...)
 * above CONVROT_NOALLOC_SCRATCH_FLOATS * 4 bytes (one maximum per 16 rows x
 * 1024 columns for large inputs: beyond about 2^30 elements, e.g. 65536 x
 * 16384), return CR_ERR_WORKSPACE_TOO_SMALL with nothing enqueued. Every call on a GPU
 * shares that GPU's array: calls that may overlap on one GPU (different
 * streams, no ordering between them) race; calls ordered on one stream do
 * not. The array's contents on entry are valid whatever they are (see the
 * workspace of convrot_rotate_quantize).
 */
#define CONVROT_NOALLOC_SCRATCH_FLOATS 65536
cr_status convrot_rotate_quantize_noalloc(const void* x, int64_t rows, int64_t K, int64_t ldx,
                                          int rot_group, cr_qtype qtype, cr_gran gran, int q_group,
                                          float shift, const float* smooth,
                                          const void* lora_down, int R, void* lora_act, int lora_act_f32,
                                          void* codes, cr_layout layout, void* scales, void* zeros,
                                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * convrot_rotate_quantize_dual - per-tensor INT4 and INT8 codes of the same
 * rotated activation, from one rotation.
 *
 * Cites: "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Key Technical
 * Optimizations (quantize an activation once and share it between the
 * projections that read it); "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4"
 * page, intro (Q/K projections in INT4, value projection in INT8 tensorwise,
 * all reading the same attention input).
 *
 * Equivalent, bit for bit, to convrot_rotate_quantize(x, ..., rot_group,
 * SYM_INT4, TENSOR, codes4, layout4, scale4) followed by the same call with
 * SYM_INT8, TENSOR, codes8 (natural int8 [rows, K]), scale8: both share the
 * maximum of the rotated tensor, which is computed once (the launches of one
 * per-tensor convrot_rotate_quantize instead of twice that).
 *   codes4   uint8 int4 codes, layout4 CR_LAYOUT_NATURAL [rows, K/2],
 *            CR_LAYOUT_TILED or CR_LAYOUT_F6; scale4 float32 [1]
 *   codes8   int8 [rows, K]; scale8 float32 [1]
 *   workspace  at least convrot_rq_workspace_size(rows, K, rot_group,
 *            SYM_INT4, TENSOR, 0) bytes
 *   rot_group  16, 64, 256 or 1024 (0 returns CR_ERR_UNSUPPORTED_FORMAT)
 * Shape and alignment as convrot_rotate_quantize.
 */
cr_status convrot_rotate_quantize_dual(const void* x, int64_t rows, int64_t K, int64_t ldx, int rot_group,
                                       void* codes4, cr_layout layout4, float* scale4,
                                       void* codes8, float* scale8,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * w4_pack_weights - natural int4 weight codes -> tile-packed layout.
 *
 * Cites: "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Tile-Packed Weight
 * Format (outer (N/128, K/64) grid of 32x128-byte tiles; group scales as
 * (N/128, K/64, 128)); "Qwen3-4B ConvRot W4A4" page, Format (natural
 * [rows, cols/2] container).
 *
 *   codes    natural uint8 [N, K/2] as written by convrot_rotate_quantize
 *   qtype    SYM_INT4 (W4A4 formats) or ASYM_UINT4 (W4A8 g16 format)
 *   gran     SYM_INT4: TENSOR, ROW or ROW_GROUP(q_group 64); ASYM: ROW_GROUP(16)
 *   scales   as written by convrot_rotate_quantize for that (qtype, gran)
 *   zeros    ASYM only: uint8 [N, K/32]
 * Outputs (sizes from w4_packed_bytes):
 *   packed         uint8 [N/128][K/64][4096]  (inner byte order: one 64-lane
 *                  matrix-core operand fragment per 512 B (SYM) / 256 B (ASYM))
 *   packed_scales  ROW_GROUP(64): float32 [N/128][K/64][128];
 *                  ASYM: fp16 [N/128][K/64][4][128]; NULL for TENSOR / ROW
 *   packed_zeros   ASYM: uint8 [N/128][K/64][4][128], one zero point per byte; else NULL
 *   w_sum          optional float32 [N], SYM_INT4 only: sum_k of the
 *                  dequantized weight row (float32 accumulation), the
 *                  correction vector of the unsigned-shift path; must be NULL
 *                  for ASYM_UINT4
 * Shape: N % 128 == 0, K % 64 == 0 (K % 256 for ROW_GROUP 64 is not required),
 * K <= 32768, N < 2^31. w4_packed_bytes returns 0 for a shape or format that
 * w4_pack_weights refuses.
 */
size_t w4_packed_bytes(int64_t N, int64_t K, cr_qtype qtype, cr_gran gran, int q_group,
                       int which /* 0 packed codes, 1 packed scales, 2 packed zeros */);

cr_status w4_pack_weights(const void* codes, const void* scales, const void* zeros,
                          int64_t N, int64_t K, cr_qtype qtype, cr_gran gran, int q_group,
                          void* packed, void* packed_scales, void* packed_zeros, float* w_sum,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * w4_pack_weights_f6 - natural signed int4 weight codes -> CR_LAYOUT_F6
 * fragments, the weight operand of w4a4_gemm with a_layout CR_LAYOUT_F6.
 *
 * Cites: "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Tile-Packed Weight
 * Format (weights reorganised offline into the GEMM's operand tiles);
 * "Qwen3-4B ConvRot W4A4" page, Format (natural [rows, cols/2] container).
 *
 *   codes    natural uint8 [N, K/2] SYM_INT4 codes (low nibble = even column);
 *            every code must lie in [-7, 7] (a -8 nibble has no exact E2M3
 *            value and is not checked)
 *   packed   uint8, w4_packed_f6_bytes(N, K) = (N/32)(K/64) 1536 bytes
 * The weight scales (TENSOR [1] or ROW [N]) are used as they are.
 * Shape: N % 128 == 0, K % 128 == 0, K <= 32768, N < 2^31 (w4_packed_f6_bytes
 * returns 0 outside it). One launch on `stream`.
 */
size_t w4_packed_f6_bytes(int64_t N, int64_t K);
cr_status w4_pack_weights_f6(const void* codes, int64_t N, int64_t K, void* packed, hipStream_t stream);

/* ------------------------------------------------------------------------
 * w4_pack_lora_up - the low-rank up-projection L1 into its tiled layout, the
 * form w4a4_gemm and w4a8_gemm read.
 *
 * Cites: "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Tile-Packed Weight
 * Format (LoRA-up stored (N/128, R, 128) beside the weight tiles).
 *
 *   up      bf16 [N, R], row n = output channel (16-byte aligned)
 *   packed  bf16 [N/128][R][128]: element (t, r, i) = up[128 t + i, r]
 * A call of its own, so that a LoRA can be swapped without repacking the
 * quantized weight. Shape: N % 128 == 0, R = 32 or 64. One launch on `stream`.
 */
cr_status w4_pack_lora_up(const void* up, int64_t N, int R, void* packed, hipStream_t stream);

/* ------------------------------------------------------------------------
 * w4_expand_weights_f6 - tile-packed INT4 weights -> CR_LAYOUT_F6 fragments:
 * the expansion that w4a4_gemm runs in its workspace for CR_LAYOUT_F6 codes
 * against CR_LAYOUT_TILED weights, as a call of its own, so that a caller
 * can run it on another stream ahead of the GEMM (it reads weights only) and
 * then call w4a4_gemm with w_layout CR_LAYOUT_F6 on the result.
 *
 * Cites: "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Tile-Packed Weight
 * Format (weights stored at 4 bits in the GEMM's operand tiles).
 *
 *   tiles   uint8 [N/128][K/64][4096]: SYM_INT4 codes from w4_pack_weights
 *           (CR_GRAN_TENSOR or CR_GRAN_ROW), 4 bits per code; every code must
 *           lie in [-7, 7] (as the quantizer produces them)
 *   f6      uint8, w4_packed_f6_bytes(N, K) bytes: receives the same bytes as
 *           w4_pack_weights_f6 of the natural codes
 * Shape: N % 128 == 0, K % 128 == 0, K <= 32768. One streaming launch on
 * `stream` (reads N K / 2 bytes, writes 3 N K / 4).
 */
cr_status w4_expand_weights_f6(const void* tiles, int64_t N, int64_t K, void* f6, hipStream_t stream);

/* ------------------------------------------------------------------------
 * convrot_dequantize_weights - quantized weights back to bf16 in the
 * original (unrotated) basis, plus an optional low-rank delta: merging a LoRA
 * into quantized weights.
 *
 * Cites: "Qwen-Image-Edit-2511-W4A8-ConvRot" card, passage on LoRA merge
 * versus bypass (a LoRA loaded onto a quantized weight dequantizes it, adds
 * the delta and quantizes the result again).
 *
 *   codes      natural codes as written by convrot_rotate_quantize: int4
 *              [N, K/2] (SYM_INT4, ASYM_UINT4) or int8 [N, K] (SYM_INT8)
 *   scales     float32 [1] / [N] / [N, K/64] (SYM_INT4 TENSOR / ROW /
 *              ROW_GROUP(64)), float32 [1] / [N] (SYM_INT8); ASYM_UINT4 g16:
 *              fp16 [N, K/16] with zeros uint8 [N, K/32]
 *   rot_group  the rotation the weights were quantized with (0, 16, 64, 256,
 *              1024; ASYM: 0 or 256)
 *   delta_up   optional bf16 [N, R] and delta_down bf16 [R, K] (1 <= R <= 256):
 *              adds sum_j up[n, j] down[j, k]
 *   out        bf16 [N, K]
 * Per element (float32, fixed order, one bf16 rounding at the end):
 *   r = fl(s q) (ASYM: s16 (q - z), exact); w = H r / sqrt(rot_group) per
 *   group with the forward rotation's butterflies (H / sqrt(n) is its own
 *   inverse); d = sum over j in increasing order of up[n, j] down[j, k];
 *   out = bf16_rne(fl(w + d)) (a zero as +0). Requantize with convrot_rotate_quantize and
 *   w4_pack_weights. Shape: K % 256 == 0 and K % rot_group == 0.
 */
cr_status convrot_dequantize_weights(const void* codes, const void* scales, const void* zeros,
                                     int64_t N, int64_t K, cr_qtype qtype, cr_gran gran, int q_group,
                                     int rot_group, const void* delta_up, const void* delta_down, int R,
                                     void* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * w4a4_gemm - INT4 activations x tile-packed INT4 weights with a fused
 * epilogue, on the int8 matrix cores (exact int4 -> int8 widening, int32
 * accumulation) or on the fp6 matrix cores (int4 codes carried as exact
 * E2M3 values, exact float32 sums).
 *
 * Cites: "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4" page, intro (packed
 * signed INT4 weights, two per byte) and Measurements (fused rotation + INT4
 * matmul with a rank-one scale); "Qwen-Image-Edit-2511 INT4 (ComfyUI
 * Optimized)", Tile-Packed Weight Format, Fused LoRA-Up Epilogue, Kernel
 * Engineering (unsigned shifted activations, scale staging).
 *
 *   a_codes     int4 codes (signed, or unsigned when a_unsigned) in a_layout:
 *               CR_LAYOUT_TILED or CR_LAYOUT_NATURAL [M, K/2] (int8 matrix
 *               cores); CR_LAYOUT_INT8: int8 codes [M, K] (SYM_INT8, TENSOR or
 *               ROW scales), the 8-bit-activation branch for these weights
 *               ("Qwen3-4B ConvRot W4A4" page, INT8 branch comparison): no
 *               a_unsigned, no 64-group scales and no low-rank branch with it;
 *               CR_LAYOUT_F6: fp6 E2M3 fragments (signed codes, or unsigned
 *               codes as u/2), run on the fp6 matrix cores (the products and
 *               their float32 sums are exact, so the int32 output equals the
 *               int8-core path's): a_unsigned and the low-rank branch need
 *               ROW_GROUP(64) scales on both sides; TENSOR / ROW scales take
 *               signed codes and no low-rank branch
 *   a_scales    float32: TENSOR [1], ROW [M], ROW_GROUP(64) [M, K/64]
 *   a_unsigned  1 for UNSIGNED_INT4_SHIFT codes: y -= a_shift * w_sum[n]
 *   w_packed    w_layout CR_LAYOUT_TILED: the tile-packed INT4 weights of
 *               w4_pack_weights (SYM_INT4, 4 bits per code), with any a_layout.
 *               With CR_LAYOUT_F6 codes the call first expands the tiles into
 *               fp6 fragments in `workspace` (one streaming pass, enqueued on
 *               `stream` before the GEMM) and runs the fp6 GEMM on them.
 *               w_layout CR_LAYOUT_F6: fragments already expanded by
 *               w4_pack_weights_f6 (6 bits per code; CR_LAYOUT_F6 codes only)
 *   w_scales    TENSOR [1], ROW [N], ROW_GROUP(64): packed [N/128][K/64][128]
 *   scale pairs: (TENSOR|ROW) x (TENSOR|ROW), or ROW_GROUP x ROW_GROUP (group 64)
 *   w_sum       float32 [N], required iff a_unsigned
 *   lora_act    optional [M, R] (bf16, or float32 if lora_act_f32), R = 32 or 64;
 *   lora_up     L1 (row n = output channel) in the tiled layout of
 *               w4_pack_lora_up, bf16 [N/128][R][128]: y += lora_act @ L1^T
 *   bias        optional bf16 [N]
 *   out         CR_OUT_BF16: bf16 [M, ldc]; CR_OUT_F32: float32; CR_OUT_I32_RAW:
 *               int32 sum_k qa*qw (lora/bias/scales ignored)
 *   workspace   at least w4a4_gemm_workspace_size(N, K, a_layout, w_layout)
 *               (0 when the call needs none or refuses the shape)
 *               bytes (nonzero only for CR_LAYOUT_F6 codes with CR_LAYOUT_TILED
 *               weights), 16-byte aligned; its contents are overwritten. Calls
 *               sharing a workspace must be ordered on one stream.
 * Epilogue: y = s_a s_w acc  (or sum_g a_s[m,g] w_s[n,g] P[m,n,g]) - shift
 * term + low-rank + bias, evaluated in float32, stored once.
 * Shape: M >= 1, N % 128 == 0, K % 128 == 0, K <= 32768, ldc >= N (ldc % 8 == 0),
 * M*K/2 and N*K/2 below 2^32 bytes.
 */
size_t w4a4_gemm_workspace_size(int64_t N, int64_t K, cr_layout a_layout, cr_layout w_layout);

cr_status w4a4_gemm(const void* a_codes, cr_layout a_layout, const float* a_scales, cr_gran a_gran,
                    int a_unsigned, float a_shift,
                    const void* w_packed, cr_layout w_layout, const float* w_scales, cr_gran w_gran,
                    const float* w_sum,
                    const void* lora_act, int lora_act_f32, const void* lora_up, int R,
                    const void* bias,
                    void* out, cr_out out_type, int64_t ldc,
                    int64_t M, int64_t N, int64_t K,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * w4a8_gemm - per-token INT8 activations x asymmetric uint4 g16 weights.
 *
 * Cites: "Qwen-Image-Edit-2511-W4A8-ConvRot" card, build table and file
 * layout (asym_w4a8_int8, group_size 16, convrot_groupsize 256); the same
 * card's passage on LoRA merge versus bypass (low-rank branch);
 * "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)", Environment Variables
 * (FP32 low-rank activations).
 *
 *   a_codes    SYM_INT8 codes from convrot_rotate_quantize: a_layout
 *              CR_LAYOUT_NATURAL int8 [M, K], or CR_LAYOUT_F16 fp16 [M, K]
 *              (the same integers; no conversion in the GEMM)
 *   a_scales   float32 ROW [M] (or TENSOR [1])
 *   w_packed, w_scales (fp16), w_zeros (uint8): from w4_pack_weights (ASYM_UINT4)
 *   lora_act   optional [M, R], bf16 (lora_act_f32 = 0) or float32 (1), R = 32
 *              or 64 (e.g. from convrot_rotate_quantize's lora_down with
 *              rotation), with lora_up = L1 in the tiled layout of
 *              w4_pack_lora_up (bf16 [N/128][R][128]): the low-rank bypass of
 *              a LoRA kept beside the quantized weight, y += la @ L1^T
 *   Every 16-deep group's partial P[m, n, g] = sum_{k in g} qa[m,k] (qw[n,k] -
 *   z[n, g]) is formed exactly (fp16 matrix cores on the exact integers).
 *   CR_OUT_BF16 / CR_OUT_F32: y[m, n] = s_a[m] * acc[m, n] (+ low rank) + bias[n]
 *              with acc accumulated in float32, one fused multiply-add
 *              acc += s_w[n, g] * P[m, n, g] per group in increasing k.
 *   CR_OUT_I32_RAW: sum_g P[m, n, g] exactly (low rank, bias, scales ignored).
 * Shape: M >= 1, N % 128 == 0, K % 128 == 0, K <= 32768, ldc >= N (ldc % 8 == 0). group must be 16.
 * workspace: unused (pass NULL, 0).
 */
cr_status w4a8_gemm(const void* a_codes, cr_layout a_layout, const float* a_scales, cr_gran a_gran,
                    const void* w_packed, const void* w_scales, const void* w_zeros, int group,
                    const void* lora_act, int lora_act_f32, const void* lora_up, int R,
                    const void* bias, void* out, cr_out out_type, int64_t ldc,
                    int64_t M, int64_t N, int64_t K,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * int8_tensorwise_gemm - INT8 x INT8 with per-tensor scales (the INT8
 * fallback layers of the mixed recipe, with or without ConvRot).
 *
 * Cites: "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4" page, intro (value /
 * output projections and adaLN modulation kept as int8_tensorwise) and
 * Measurements (int8_tensorwise kernels); "Qwen Image 2.1 - Hybrid W4A8 /
 * INT8 ConvRot", Quantization recipe.
 *
 *   a_codes int8 [M, K]; a_scale float32 [1]; w int8 [N, K] natural; w_scale float32 [1]
 *   y = s_a s_w sum_k qa qw + bias
 * Shape: M >= 1, N % 128 == 0, K % 128 == 0, K <= 32768, ldc >= N (ldc % 8 == 0).
 */
cr_status int8_tensorwise_gemm(const void* a_codes, const float* a_scale,
                               const void* w, const float* w_scale,
                               const void* bias, void* out, cr_out out_type, int64_t ldc,
                               int64_t M, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
