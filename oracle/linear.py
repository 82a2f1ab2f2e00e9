"""Composed reference of the ConvRot low-bit linear: rotate+quantize, weight
preparation, integer GEMM and the float epilogue.

Sources:
  [P1] intro / "Measurements": W4A4 tensorwise with online ConvRot rotation of
       the activations and a fused rotation+INT4 matrix-multiply kernel;
       INT8 tensorwise layers in the same model (v/o projections, adaLN).
  [P2] build table, file layout: W4A8 asymmetric, group 16, ConvRot 256.
  [P3] Quantization Method / Key Technical Optimizations / Kernel Engineering:
       W = low-rank + residual (SVDQuant), the residual quantized to W4A4 with
       per-group scales; LoRA-down computed once from the activation and
       shared by the split Q/K/V projections; LoRA-up fused into the GEMM
       epilogue; unsigned post-GELU activations shifted by +0.171875;
       LoRA activations optionally kept in FP32.

Epilogue (computed in float64 from the exact integers and the STORED scales,
then rounded once to float32 — the reference the bf16 GPU output is compared
with by relative L2 error):
  tensor / row:  y[m,n] = s_a[m] * s_w[n] * acc[m,n]
  g16 (W4A8):    y[m,n] = s_a[m] * sum_g s_w[n,g] * P[m,n,g]
  g64 (W4A4):    y[m,n] = sum_g a_s[m,g] * w_s[n,g] * P[m,n,g]
  unsigned shift (reading of the shift convention, which the pages do not
  spell out): the codes encode v + c, so y -= c * sum_k w_hat[n,k] with
  w_hat the dequantized weight;
  low rank:      y += sum_r la[m,r] * L1[n,r], la = X @ L2^T from the
                 unrotated, unshifted bf16 input, stored as bf16 (RNE) or
                 float32;
  bias:          y += b[n].
"""
from __future__ import annotations

import numpy as np

from . import hadamard, quant, pack, gemm

SHIFT_POST_GELU = 0.171875   # [P3] Kernel Engineering


def _f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 value of its bf16 rounding (half-to-even)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return b.astype(np.uint32).view(np.float32)


# ---------------------------------------------------------------------------
# rotate + quantize (mirrors the library call of the same name)
# ---------------------------------------------------------------------------

def rotate_quantize(x_bits: np.ndarray, rot_group: int, qtype: str, gran: str,
                    q_group: int | None = None, shift: float = 0.0, smooth: np.ndarray | None = None):
    """x_bits: bf16 bit patterns [rows, K]. smooth: optional float32 [K]
    per-channel multiplier applied to the input before anything else,
    v = fl(x * smooth[k]) (the smoothing factor of [P3] Key Technical
    Optimizations, given as the multiplier the activation needs; the matching
    weight columns carry its inverse offline).
    qtype: 'int4' | 'int8' | 'uint4_shift' | 'asym_u4'.
    Returns a dict with
      'values' : the codes as integers [rows, K]
      'codes'  : the stored codes (int4: uint8 [rows, K/2] two per byte;
                 int8: int8 [rows, K])
      'scales' : float32 (float16 for asym_u4)
      'zeros'  : asym_u4 only, uint8 [rows, K/16] (one per group) and
      'zeros_packed' : [rows, K/32] two per byte."""
    x = _f32(x_bits)
    if smooth is not None:
        x = (x * np.asarray(smooth, dtype=np.float32)[None, :]).astype(np.float32)
    if rot_group:
        v = hadamard.rotate(x, rot_group)
        post = np.float32(1.0 / np.sqrt(rot_group))          # exact power of two
    else:
        v = x
        post = np.float32(1.0)
    out = {}
    if qtype in ("int4", "int8"):
        qmax = quant.QMAX_INT4 if qtype == "int4" else quant.QMAX_INT8
        q, s = quant.quantize_sym(v, qmax, gran, q_group, scale_mul=post)
        out["values"] = q
        out["codes"] = pack.pack_int4(q) if qtype == "int4" else q
        out["scales"] = s
    elif qtype == "uint4_shift":
        if rot_group:
            raise ValueError("the unsigned shift path applies to unrotated post-GELU inputs")
        q, s = quant.quantize_unsigned_shift(v, shift, gran, q_group)
        out["values"] = q
        out["codes"] = pack.pack_int4(q)
        out["scales"] = s
    elif qtype == "asym_u4":
        vv = (v * post).astype(np.float32)                  # orthonormal rotated weight
        q, s16, z = quant.quantize_asym(vv, q_group or 16)
        out["values"] = q
        out["codes"] = pack.pack_int4(q)
        out["scales"] = s16
        out["zeros"] = z
        out["zeros_packed"] = pack.pack_zeros_u4(z)
    else:
        raise ValueError(qtype)
    return out


def lora_down(x_bits: np.ndarray, l2_bits: np.ndarray, act_f32: bool = False) -> np.ndarray:
    """la = X @ L2^T [rows, R] from the unrotated bf16 input; float64 sum,
    rounded to float32, then to bf16 unless act_f32. Returned as float32."""
    la = (_f32(x_bits).astype(np.float64) @ _f32(l2_bits).astype(np.float64).T).astype(np.float32)
    return la if act_f32 else _bf16_round(la)


def weight_sum(values: np.ndarray, scales: np.ndarray, gran: str, group: int | None = None) -> np.ndarray:
    """sum_k w_hat[n, k] for symmetric codes (float64 -> float32)."""
    return quant.dequant_sym(values, scales, gran, group).sum(axis=1).astype(np.float32)


def dequantize_weights(values, scales, qtype, gran, group=None, zeros=None, rot_group=256,
                       up_bits=None, down_bits=None) -> np.ndarray:
    """Quantized weights back to bf16 bits [N, K] in the unrotated basis, plus
    an optional low-rank delta up @ down (a LoRA merged into the weight; the
    "Qwen-Image-Edit-2511-W4A8-ConvRot" card's passage on LoRA merge versus
    bypass: dequantize, add the delta, quantize again).

    Float32 throughout, in this order: r = fl(s * q) (asymmetric: s16 (q - z),
    exact); w = rotate(r) / sqrt(n) (H / sqrt(n) is its own inverse; the
    forward rotation's butterflies); d accumulated over the ranks in
    increasing order (bf16 products are exact in float32); one bf16 rounding
    of fl(w + d). Zeros are +0 (the rotation's sign bookkeeping is free to
    produce either)."""
    q = np.asarray(values)
    N, K = q.shape
    if qtype == "asym_u4":
        r = quant.dequant_asym(q, scales, zeros, group).astype(np.float32)
    else:
        s = np.asarray(scales, dtype=np.float32)
        if gran == "tensor":
            sv = np.full((N, K), s.reshape(-1)[0], dtype=np.float32)
        elif gran == "row":
            sv = np.repeat(s.reshape(N, 1), K, axis=1)
        else:
            sv = np.repeat(s.reshape(N, K // group), group, axis=1)
        r = (sv * q.astype(np.float32)).astype(np.float32)
    w = r
    if rot_group:
        w = (hadamard.rotate(r, rot_group) * np.float32(1.0 / np.sqrt(rot_group))).astype(np.float32)
    if up_bits is not None:
        up, down = _f32(up_bits), _f32(down_bits)
        d = np.zeros((N, K), dtype=np.float32)
        for j in range(up.shape[1]):
            d = (d + up[:, j:j + 1] * down[j:j + 1, :]).astype(np.float32)
        w = (w + d).astype(np.float32)
    w = (w + np.float32(0.0)).astype(np.float32)          # a zero comes out as +0
    b = np.ascontiguousarray(w, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return b.astype(np.uint16)


# ---------------------------------------------------------------------------
# epilogues
# ---------------------------------------------------------------------------

def _scale_vec(s: np.ndarray, gran: str, n: int) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64).reshape(-1)
    return np.full(n, s[0]) if gran == "tensor" else s


def epilogue_scalar(acc, a_scales, a_gran, w_scales, w_gran, shift=0.0, wsum=None,
                    la=None, l1_bits=None, bias_bits=None) -> np.ndarray:
    M, N = acc.shape
    sa = _scale_vec(a_scales, a_gran, M)
    sw = _scale_vec(w_scales, w_gran, N)
    y = sa[:, None] * sw[None, :] * acc.astype(np.float64)
    return _finish(y, shift, wsum, la, l1_bits, bias_bits)


def epilogue_g64(P, a_scales, w_scales, shift=0.0, wsum=None, la=None, l1_bits=None,
                 bias_bits=None) -> np.ndarray:
    """P [M, N, G] exact partials, a_scales [M, G], w_scales [N, G]."""
    a = np.asarray(a_scales, dtype=np.float64)
    w = np.asarray(w_scales, dtype=np.float64)
    y = np.einsum("mg,ng,mng->mn", a, w, P.astype(np.float64))
    return _finish(y, shift, wsum, la, l1_bits, bias_bits)


def epilogue_g16(P, a_scales, a_gran, w_scales16, bias_bits=None, la=None, l1_bits=None) -> np.ndarray:
    M, N, G = P.shape
    sa = _scale_vec(a_scales, a_gran, M)
    w = np.asarray(w_scales16, dtype=np.float64)
    y = sa[:, None] * np.einsum("ng,mng->mn", w, P.astype(np.float64))
    return _finish(y, 0.0, None, la, l1_bits, bias_bits)


def _finish(y, shift, wsum, la, l1_bits, bias_bits):
    if shift:
        y = y - np.float64(shift) * np.asarray(wsum, dtype=np.float64)[None, :]
    if la is not None:
        y = y + np.asarray(la, dtype=np.float64) @ _f32(l1_bits).astype(np.float64).T
    if bias_bits is not None:
        y = y + _f32(bias_bits).astype(np.float64)[None, :]
    return y.astype(np.float32)


# ---------------------------------------------------------------------------
# composed reference linears (used by tests and the CPU baseline)
# ---------------------------------------------------------------------------

def prepare_w4a4(w_bits, rot_group=256, gran="tensor", q_group=None):
    """Offline weight preparation of a W4A4 layer: rotate, quantize to
    symmetric INT4, tile-pack; g64 scales tile-packed; weight sums."""
    r = rotate_quantize(w_bits, rot_group, "int4", gran, q_group)
    r["tiles"] = pack.tile_pack_w4a4(r["codes"])
    if gran == "row_group":
        r["scales_tiles"] = pack.tile_pack_g64_scales(r["scales"])
    r["wsum"] = weight_sum(r["values"], r["scales"], gran, q_group)
    return r


def prepare_w4a8(w_bits, rot_group=256, group=16):
    r = rotate_quantize(w_bits, rot_group, "asym_u4", "row_group", group)
    r["tiles"] = pack.tile_pack_w4a8(r["values"])
    r["scales_tiles"] = pack.tile_pack_g16(r["scales"])
    r["zeros_tiles"] = pack.tile_pack_g16(r["zeros"])
    return r


def w4a4_linear(x_bits, w_bits, rot_group=256, a_gran="tensor", w_gran="tensor",
                group=None, shift=0.0, l1_bits=None, l2_bits=None, act_f32=False,
                bias_bits=None, wprep=None):
    """Reference y (float32 [M, N]) and raw integer result for the W4A4 path."""
    unsigned = shift != 0.0
    xa = rotate_quantize(x_bits, rot_group, "uint4_shift" if unsigned else "int4",
                         a_gran, group, shift)
    wp = wprep if wprep is not None else prepare_w4a4(w_bits, rot_group, w_gran, group)
    la = lora_down(x_bits, l2_bits, act_f32) if l2_bits is not None else None
    if a_gran == "row_group":
        P = gemm.group_partials(xa["values"], wp["values"], group)
        y = epilogue_g64(P, xa["scales"], wp["scales"], shift, wp["wsum"], la, l1_bits, bias_bits)
        raw = P.sum(axis=2)
    else:
        raw = gemm.int_gemm(xa["values"], wp["values"])
        y = epilogue_scalar(raw, xa["scales"], a_gran, wp["scales"], w_gran, shift,
                            wp["wsum"], la, l1_bits, bias_bits)
    return {"y": y, "raw": raw, "x": xa, "w": wp, "la": la}


def int8_linear(x_bits, w_bits, rot_group=256, bias_bits=None):
    xa = rotate_quantize(x_bits, rot_group, "int8", "tensor")
    wq = rotate_quantize(w_bits, rot_group, "int8", "tensor")
    raw = gemm.int_gemm(xa["values"], wq["values"])
    y = epilogue_scalar(raw, xa["scales"], "tensor", wq["scales"], "tensor", bias_bits=bias_bits)
    return {"y": y, "raw": raw, "x": xa, "w": wq}


def a8w4_linear(x_bits, w_bits, rot_group=256, a_gran="row", w_gran="tensor", bias_bits=None, wprep=None):
    """8-bit activations (symmetric INT8, per token or per tensor) against
    W4A4-format weights (symmetric INT4, per tensor or per row): the INT8
    branch the "Qwen3-4B ConvRot W4A4" page compares with the INT4 one,
    y = s_a[m] s_w[n] sum_k qa qw + b."""
    xa = rotate_quantize(x_bits, rot_group, "int8", a_gran)
    wp = wprep if wprep is not None else prepare_w4a4(w_bits, rot_group, w_gran)
    raw = gemm.int_gemm(xa["values"], wp["values"])
    y = epilogue_scalar(raw, xa["scales"], a_gran, wp["scales"], w_gran, bias_bits=bias_bits)
    return {"y": y, "raw": raw, "x": xa, "w": wp}


def w4a8_linear(x_bits, w_bits, rot_group=256, group=16, bias_bits=None, wprep=None, l1_bits=None, l2_bits=None,
                act_f32=False):
    """l1_bits [N, R] / l2_bits [R, K] (bf16): a LoRA kept as a bypass beside
    the quantized weight, y += (X L2^T) L1^T with X the unrotated input and
    the low-rank activations bf16 (float32 with act_f32)."""
    xa = rotate_quantize(x_bits, rot_group, "int8", "row")
    wp = wprep if wprep is not None else prepare_w4a8(w_bits, rot_group, group)
    la = lora_down(x_bits, l2_bits, act_f32) if l2_bits is not None else None
    P = gemm.group_partials(xa["values"], wp["values"], group, wp["zeros"])
    y = epilogue_g16(P, xa["scales"], "row", wp["scales"], bias_bits, la, l1_bits)
    return {"y": y, "raw": P.sum(axis=2), "x": xa, "w": wp, "la": la}


def float_linear(x_bits, w_bits) -> np.ndarray:
    """Unquantized float64 X @ W^T of the bf16 inputs (sanity reference)."""
    return _f32(x_bits).astype(np.float64) @ _f32(w_bits).astype(np.float64).T
