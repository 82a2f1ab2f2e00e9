"""Dynamic quantizers of the ConvRot low-bit linear.

Sources:
  [P1] intro and "Runtime requirement": signed INT4 weights (two per byte),
       activations quantized dynamically at run time, tensorwise scales
       (int4_tensorwise / int8_tensorwise).
  [P5] Format: a per-output-row float32 weight scale is also used
       (weight_scale F32 [rows]).
  [P2] build table and file layout: asymmetric 4-bit weights with group size
       16 along K, ConvRot group 256, 8-bit activations.
  [P3] Kernel Engineering: an unsigned activation path with a +0.171875
       shift for post-GELU layers; Quantization Method: SVDQuant (W4A4 with a
       low-rank branch).

Readings where the pages are silent (each one also fixes what the GPU path
must reproduce bit for bit):
  * symmetric codes are confined to [-qmax, qmax] with qmax = 7 (INT4) or
    127 (INT8): the INT4 code -8 is never produced;
  * A = max |v| over the scale group; r = qmax / A and s = A / qmax, each ONE
    correctly rounded float32 division; code = clamp(rint(fl32(v * r))) where
    the product is rounded to float32 first and rint is round-half-to-even
    (no fused multiply-add);
  * an all-zero scale group gets s = 0 and all-zero codes;
  * when the values come from the unnormalised rotation (hadamard.rotate),
    the stored scale is multiplied by 1/sqrt(group) (a power of two), which
    makes s the scale of the orthonormally rotated tensor; codes do not
    depend on that factor;
  * unsigned-shift path: v' = fl32(v + shift), A = max v', r = 15 / A,
    code = clamp(rint(fl32(v' * r)), 0, 15), s = A / 15 (A <= 0 gives s = 0
    and zero codes);
  * asymmetric g16 (weights only): lo = min(0, min v), hi = max(0, max v),
    s = fp16(fl32(hi - lo) / 15) (round-half-to-even to fp16),
    z = clamp(rint(fl32(-lo / s)), 0, 15),
    code = clamp(rint(fl32(v / s)) + z, 0, 15); hi == lo (or s rounding to
    0 in fp16) gives s = 1, z = 0 and zero codes; dequantized value
    s * (code - z).
"""
from __future__ import annotations

import numpy as np

QMAX_INT4 = 7
QMAX_INT8 = 127


def _group_view(v: np.ndarray, gran: str, group: int | None) -> np.ndarray:
    """Reshape [rows, K] to [n_scale_groups, elements_per_group] following
    the granularity: 'tensor' (one group), 'row' (one per row) or 'row_group'
    (one per row and per `group` consecutive columns)."""
    rows, K = v.shape
    if gran == "tensor":
        return v.reshape(1, rows * K)
    if gran == "row":
        return v.reshape(rows, K)
    if gran == "row_group":
        if group is None or K % group:
            raise ValueError("row_group needs K % group == 0")
        return v.reshape(rows * (K // group), group)
    raise ValueError(f"unknown granularity {gran}")


def _scale_shape(rows: int, K: int, gran: str, group: int | None):
    if gran == "tensor":
        return (1,)
    if gran == "row":
        return (rows,)
    return (rows, K // group)


def quantize_sym(v: np.ndarray, qmax: int, gran: str, group: int | None = None,
                 scale_mul: float = 1.0):
    """Symmetric dynamic quantization. v: float32 [rows, K].
    Returns (codes int8 [rows, K], scales float32 of the granularity's shape).
    scale_mul: exact power-of-two factor applied to the stored scale."""
    v = np.asarray(v, dtype=np.float32)
    rows, K = v.shape
    g = _group_view(v, gran, group)
    A = np.max(np.abs(g), axis=1)                           # exact
    nz = A > 0
    qm = np.float32(qmax)
    r = np.zeros_like(A)
    s = np.zeros_like(A)
    r[nz] = qm / A[nz]                                      # float32 division
    s[nz] = A[nz] / qm
    s = (s * np.float32(scale_mul)).astype(np.float32)
    prod = (g * r[:, None]).astype(np.float32)              # rounded to float32
    q = np.clip(np.rint(prod), -qmax, qmax)                 # half-to-even
    q[~nz, :] = 0
    return q.astype(np.int8).reshape(rows, K), s.reshape(_scale_shape(rows, K, gran, group))


def quantize_unsigned_shift(v: np.ndarray, shift: float, gran: str, group: int | None = None):
    """Unsigned 4-bit codes of v + shift (post-GELU path). Returns
    (codes uint8 in [0, 15], scales float32)."""
    v = np.asarray(v, dtype=np.float32)
    rows, K = v.shape
    vs = (v + np.float32(shift)).astype(np.float32)
    g = _group_view(vs, gran, group)
    A = np.max(g, axis=1)
    pos = A > 0
    r = np.zeros_like(A)
    s = np.zeros_like(A)
    r[pos] = np.float32(15) / A[pos]
    s[pos] = A[pos] / np.float32(15)
    prod = (g * r[:, None]).astype(np.float32)
    q = np.clip(np.rint(prod), 0, 15)
    q[~pos, :] = 0
    return q.astype(np.uint8).reshape(rows, K), s.reshape(_scale_shape(rows, K, gran, group))


def quantize_asym(v: np.ndarray, group: int = 16):
    """Asymmetric uint4 quantization per `group` consecutive columns of each
    row. Returns (codes uint8 [rows, K] in [0,15], scales float16
    [rows, K/group], zeros uint8 [rows, K/group] in [0,15])."""
    v = np.asarray(v, dtype=np.float32)
    rows, K = v.shape
    g = v.reshape(rows * (K // group), group)
    lo = np.minimum(np.float32(0), g.min(axis=1))
    hi = np.maximum(np.float32(0), g.max(axis=1))
    span = (hi - lo).astype(np.float32)
    s16 = (span / np.float32(15)).astype(np.float32).astype(np.float16)
    const = (hi == lo) | (s16 == 0)
    s16[const] = np.float16(1.0)
    sf = s16.astype(np.float32)
    z = np.clip(np.rint((-lo / sf).astype(np.float32)), 0, 15)
    z[const] = 0
    q = np.clip(np.rint((g / sf[:, None]).astype(np.float32)) + z[:, None], 0, 15)
    q[const, :] = 0
    return (q.astype(np.uint8).reshape(rows, K),
            s16.reshape(rows, K // group),
            z.astype(np.uint8).reshape(rows, K // group))


def dequant_sym(codes: np.ndarray, scales: np.ndarray, gran: str, group: int | None = None):
    """float64 s * q with the scale broadcast over its group."""
    q = codes.astype(np.float64)
    rows, K = q.shape
    s = np.asarray(scales, dtype=np.float64)
    if gran == "tensor":
        return q * s[0]
    if gran == "row":
        return q * s[:, None]
    return (q.reshape(rows, K // group, group) * s[:, :, None]).reshape(rows, K)


def dequant_asym(codes: np.ndarray, scales16: np.ndarray, zeros: np.ndarray, group: int = 16):
    rows, K = codes.shape
    q = codes.astype(np.float64).reshape(rows, K // group, group)
    z = zeros.astype(np.float64)[:, :, None]
    s = scales16.astype(np.float64)[:, :, None]
    return (s * (q - z)).reshape(rows, K)
