"""Thin Python binding of libconvrot.so, the gfx950 ConvRot low-bit linear.

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/convrot.h. PyTorch provides device
memory and the current stream. There is no fallback: if the library is
missing this module raises at import, and every non-OK status raises
ConvRotError with the library's status text.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "ConvRotError", "lib", "Q", "GRAN", "OUT", "LAYOUT",
    "convrot_rotate_quantize", "convrot_rotate_quantize_dual", "convrot_dequantize_weights", "w4_pack_weights",
    "w4_pack_weights_f6", "w4_packed_f6_bytes", "w4_expand_weights_f6", "w4_pack_lora_up",
    "w4a4_gemm", "w4a4_gemm_workspace_size", "w4a8_gemm",
    "int8_tensorwise_gemm", "convrot_rq_workspace_size", "w4_packed_bytes",
    "get_counters", "reset_counters", "device_check", "status_string",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libconvrot.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run __graft_entry__.build() "
        "(hipcc --offload-arch=gfx950). There is no non-HIP fallback.")

lib = ctypes.CDLL(LIB_PATH)


class Q:
    SYM_INT4 = 0
    SYM_INT8 = 1
    UNSIGNED_INT4_SHIFT = 2
    ASYM_UINT4 = 3


class GRAN:
    TENSOR = 0
    ROW = 1
    ROW_GROUP = 2


class OUT:
    BF16 = 0
    F32 = 1
    I32_RAW = 2


class LAYOUT:
    NATURAL = 0
    TILED = 1
    INT8 = 2
    F6 = 3
    F16 = 4


class _Counters(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_uint64 * 8), ("fallbacks", ctypes.c_uint64)]


_vp, _i64, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "convrot_status_string": (ctypes.c_char_p, [_i]),
    "convrot_last_hip_error": (_i, []),
    "convrot_device_check": (_i, []),
    "convrot_get_counters": (None, [ctypes.POINTER(_Counters)]),
    "convrot_reset_counters": (None, []),
    "convrot_rq_workspace_size": (_sz, [_i64, _i64, _i, _i, _i, _i]),
    "convrot_rotate_quantize": (_i, [_vp, _i64, _i64, _i64, _i, _i, _i, _i, _f, _vp, _vp, _i, _vp, _i,
                                     _vp, _i, _vp, _vp, _vp, _sz, _vp]),
    "convrot_rotate_quantize_noalloc": (_i, [_vp, _i64, _i64, _i64, _i, _i, _i, _i, _f, _vp, _vp, _i, _vp, _i,
                                             _vp, _i, _vp, _vp, _vp]),
    "convrot_rotate_quantize_dual": (_i, [_vp, _i64, _i64, _i64, _i, _vp, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "convrot_dequantize_weights": (_i, [_vp, _vp, _vp, _i64, _i64, _i, _i, _i, _i, _vp, _vp, _i, _vp, _vp]),
    "w4_packed_bytes": (_sz, [_i64, _i64, _i, _i, _i, _i]),
    "w4_pack_weights": (_i, [_vp, _vp, _vp, _i64, _i64, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "w4_packed_f6_bytes": (_sz, [_i64, _i64]),
    "w4_pack_weights_f6": (_i, [_vp, _i64, _i64, _vp, _vp]),
    "w4_expand_weights_f6": (_i, [_vp, _i64, _i64, _vp, _vp]),
    "w4_pack_lora_up": (_i, [_vp, _i64, _i, _vp, _vp]),
    "w4a4_gemm_workspace_size": (_sz, [_i64, _i64, _i, _i]),
    "w4a4_gemm": (_i, [_vp, _i, _vp, _i, _i, _f, _vp, _i, _vp, _i, _vp, _vp, _i, _vp, _i, _vp,
                       _vp, _i, _i64, _i64, _i64, _i64, _vp, _sz, _vp]),
    "w4a8_gemm": (_i, [_vp, _i, _vp, _i, _vp, _vp, _vp, _i, _vp, _i, _vp, _i, _vp, _vp, _i, _i64, _i64, _i64, _i64,
                       _vp, _sz, _vp]),
    "int8_tensorwise_gemm": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i64, _i64, _i64, _i64,
                                  _vp, _sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class ConvRotError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.convrot_status_string(status).decode()
        if status == 7:
            msg += f" (hipError {lib.convrot_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def status_string(status: int) -> str:
    return lib.convrot_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise ConvRotError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def device_check() -> int:
    return lib.convrot_device_check()


def get_counters():
    c = _Counters()
    lib.convrot_get_counters(ctypes.byref(c))
    return {"rotate_quantize": c.launches[0], "pack": c.launches[1], "w4a4": c.launches[2],
            "w4a8": c.launches[3], "int8": c.launches[4], "fallbacks": c.fallbacks}


def reset_counters():
    lib.convrot_reset_counters()


def convrot_rq_workspace_size(rows, K, rot_group, qtype, gran, q_group=0) -> int:
    return lib.convrot_rq_workspace_size(rows, K, rot_group, qtype, gran, q_group)


def w4_packed_bytes(N, K, qtype, gran, q_group, which) -> int:
    return lib.w4_packed_bytes(N, K, qtype, gran, q_group, which)


def _scale_numel(rows, K, qtype, gran, q_group):
    if gran == GRAN.TENSOR:
        return (1,)
    if gran == GRAN.ROW:
        return (rows,)
    return (rows, K // q_group)


def convrot_rotate_quantize(x, rot_group=256, qtype=Q.SYM_INT4, gran=GRAN.TENSOR, q_group=0,
                            shift=0.0, lora_down=None, lora_act_f32=False, layout=LAYOUT.NATURAL,
                            codes=None, scales=None, zeros=None, lora_act=None, workspace=None,
                            stream=None, smooth=None):
    """x: bf16 [rows, K] (row stride may exceed K). Returns
    (codes, scales, zeros, lora_act); outputs are allocated when not given.
    Tiled int4 codes come back as uint8 [ceil(rows/16), K/64, 512], fp6
    fragments (layout F6) as uint8 [ceil(rows/32), K/64, 1536]."""
    rows, K = x.shape
    ldx = x.stride(0)
    dev = x.device
    if codes is None:
        if qtype == Q.SYM_INT8:
            codes = torch.empty((rows, K), dtype=torch.float16 if layout == LAYOUT.F16 else torch.int8, device=dev)
        elif layout == LAYOUT.TILED:
            codes = torch.empty(((rows + 15) // 16, K // 64, 512), dtype=torch.uint8, device=dev)
        elif layout == LAYOUT.F6:
            codes = torch.empty(((rows + 31) // 32, K // 64, 1536), dtype=torch.uint8, device=dev)
        else:
            codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        sdt = torch.float16 if qtype == Q.ASYM_UINT4 else torch.float32
        scales = torch.empty(_scale_numel(rows, K, qtype, gran, q_group), dtype=sdt, device=dev)
    if zeros is None and qtype == Q.ASYM_UINT4:
        zeros = torch.empty((rows, K // 32), dtype=torch.uint8, device=dev)
    R = 0
    if lora_down is not None:
        R = lora_down.shape[0]
        if lora_act is None:
            lora_act = torch.empty((rows, R), dtype=torch.float32 if lora_act_f32 else torch.bfloat16,
                                   device=dev)
    need = convrot_rq_workspace_size(rows, K, rot_group, qtype, gran, q_group)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.convrot_rotate_quantize(_ptr(x), rows, K, ldx, rot_group, qtype, gran, q_group,
                                     float(shift), _ptr(smooth), _ptr(lora_down), R, _ptr(lora_act),
                                     int(bool(lora_act_f32)), _ptr(codes), int(layout), _ptr(scales), _ptr(zeros),
                                     _ptr(workspace), wsb, _stream(stream))
    _check(st, "convrot_rotate_quantize")
    return codes, scales, zeros, lora_act


def convrot_rotate_quantize_dual(x, rot_group=256, layout4=LAYOUT.NATURAL, codes4=None, scale4=None,
                                 codes8=None, scale8=None, workspace=None, stream=None):
    """Per-tensor INT4 and INT8 codes of one rotation of x (bf16 [rows, K]).
    Returns (codes4, scale4, codes8, scale8)."""
    rows, K = x.shape
    dev = x.device
    if codes4 is None:
        shape = {LAYOUT.TILED: ((rows + 15) // 16, K // 64, 512),
                 LAYOUT.F6: ((rows + 31) // 32, K // 64, 1536)}.get(layout4, (rows, K // 2))
        codes4 = torch.empty(shape, dtype=torch.uint8, device=dev)
    if scale4 is None:
        scale4 = torch.empty(1, dtype=torch.float32, device=dev)
    if codes8 is None:
        codes8 = torch.empty((rows, K), dtype=torch.int8, device=dev)
    if scale8 is None:
        scale8 = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        need = convrot_rq_workspace_size(rows, K, rot_group, Q.SYM_INT4, GRAN.TENSOR, 0)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    st = lib.convrot_rotate_quantize_dual(_ptr(x), rows, K, x.stride(0), rot_group, _ptr(codes4), int(layout4),
                                          _ptr(scale4), _ptr(codes8), _ptr(scale8), _ptr(workspace), wsb,
                                          _stream(stream))
    _check(st, "convrot_rotate_quantize_dual")
    return codes4, scale4, codes8, scale8


def convrot_dequantize_weights(codes, scales, N, K, qtype=Q.SYM_INT4, gran=GRAN.TENSOR, q_group=0, rot_group=256,
                               zeros=None, delta_up=None, delta_down=None, out=None, stream=None):
    """Quantized weights (natural codes) -> bf16 [N, K] in the unrotated basis,
    plus delta_up [N, R] @ delta_down [R, K] when given (the LoRA merge)."""
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=codes.device)
    R = 0 if delta_up is None else delta_up.shape[1]
    st = lib.convrot_dequantize_weights(_ptr(codes), _ptr(scales), _ptr(zeros), N, K, qtype, gran, q_group,
                                        rot_group, _ptr(delta_up), _ptr(delta_down), R, _ptr(out), _stream(stream))
    _check(st, "convrot_dequantize_weights")
    return out


def w4_pack_weights(codes, scales, N, K, qtype=Q.SYM_INT4, gran=GRAN.TENSOR, q_group=0, zeros=None,
                    want_wsum=False, stream=None):
    """Returns (packed, packed_scales, packed_zeros, w_sum)."""
    dev = codes.device
    packed = torch.empty(w4_packed_bytes(N, K, qtype, gran, q_group, 0), dtype=torch.uint8, device=dev)
    nsc = w4_packed_bytes(N, K, qtype, gran, q_group, 1)
    packed_scales = None
    if nsc:
        packed_scales = torch.empty(nsc, dtype=torch.uint8, device=dev)
    nz = w4_packed_bytes(N, K, qtype, gran, q_group, 2)
    packed_zeros = torch.empty(nz, dtype=torch.uint8, device=dev) if nz else None
    w_sum = torch.empty(N, dtype=torch.float32, device=dev) if want_wsum else None
    st = lib.w4_pack_weights(_ptr(codes), _ptr(scales), _ptr(zeros), N, K, qtype, gran, q_group,
                             _ptr(packed), _ptr(packed_scales), _ptr(packed_zeros), _ptr(w_sum),
                             _stream(stream))
    _check(st, "w4_pack_weights")
    if packed_scales is not None:
        packed_scales = packed_scales.view(torch.float16 if qtype == Q.ASYM_UINT4 else torch.float32)
    return packed, packed_scales, packed_zeros, w_sum


def w4_packed_f6_bytes(N, K) -> int:
    return lib.w4_packed_f6_bytes(N, K)


def w4_pack_weights_f6(codes, N, K, packed=None, stream=None):
    """Natural signed int4 codes [N, K/2] -> fp6 E2M3 fragments
    uint8 [N/32, K/64, 1536], the weight operand of the fp6 W4A4 GEMM."""
    if packed is None:
        packed = torch.empty((N // 32, K // 64, 1536), dtype=torch.uint8, device=codes.device)
    st = lib.w4_pack_weights_f6(_ptr(codes), N, K, _ptr(packed), _stream(stream))
    _check(st, "w4_pack_weights_f6")
    return packed


def w4_pack_lora_up(up, packed=None, stream=None):
    """Low-rank up-projection L1 bf16 [N, R] -> tiled bf16 [N/128, R, 128]
    (the lora_up operand of w4a4_gemm and w4a8_gemm)."""
    N, R = up.shape
    if packed is None:
        packed = torch.empty((N // 128, R, 128), dtype=torch.bfloat16, device=up.device)
    st = lib.w4_pack_lora_up(_ptr(up), N, R, _ptr(packed), _stream(stream))
    _check(st, "w4_pack_lora_up")
    return packed


def w4_expand_weights_f6(tiles, N, K, f6=None, stream=None):
    """Tile-packed INT4 weights (w4_pack_weights) -> fp6 E2M3 fragments
    uint8 [N/32, K/64, 1536] (w_layout F6 of w4a4_gemm)."""
    if f6 is None:
        f6 = torch.empty((N // 32, K // 64, 1536), dtype=torch.uint8, device=tiles.device)
    st = lib.w4_expand_weights_f6(_ptr(tiles), N, K, _ptr(f6), _stream(stream))
    _check(st, "w4_expand_weights_f6")
    return f6


def _out(M, N, out_type, dev, out):
    if out is not None:
        return out
    dt = {OUT.BF16: torch.bfloat16, OUT.F32: torch.float32, OUT.I32_RAW: torch.int32}[out_type]
    return torch.empty((M, N), dtype=dt, device=dev)


def _lora_rank(lora_up, N):
    """R of the tiled low-rank up-projection [N/128, R, 128] (0 without one)"""
    if lora_up is None:
        return 0
    if lora_up.dim() != 3 or lora_up.shape[0] * 128 != N or lora_up.shape[2] != 128:
        raise ValueError("lora_up must be tiled [N/128, R, 128] (w4_pack_lora_up)")
    return lora_up.shape[1]


def w4a4_gemm_workspace_size(N, K, a_layout, w_layout) -> int:
    return lib.w4a4_gemm_workspace_size(N, K, int(a_layout), int(w_layout))


def w4a4_gemm(a_codes, a_scales, a_gran, w_packed, w_scales, w_gran, M, N, K,
              a_unsigned=False, a_shift=0.0, w_sum=None, lora_act=None, lora_up=None,
              bias=None, out_type=OUT.BF16, out=None, a_layout=None, w_layout=None, workspace=None, stream=None):
    """a_layout defaults to F6 for [M/32, K/64, 1536] codes, TILED for
    [M/16, K/64, 512], else NATURAL. w_layout defaults to F6 for
    [N/32, K/64, 1536] weights (w4_pack_weights_f6), else TILED
    (w4_pack_weights). With F6 codes and TILED weights the call needs a
    workspace of w4a4_gemm_workspace_size bytes (allocated here when not
    given) into which it expands the weights before the fp6 GEMM.
    lora_up is L1 tiled by w4_pack_lora_up [N/128, R, 128]."""
    if a_layout is None:
        if a_codes.dim() == 3:
            a_layout = LAYOUT.F6 if a_codes.shape[-1] == 1536 else LAYOUT.TILED
        else:
            a_layout = LAYOUT.NATURAL
    if w_layout is None:
        w_layout = LAYOUT.F6 if (w_packed.dim() == 3 and w_packed.shape[-1] == 1536) else LAYOUT.TILED
    need = w4a4_gemm_workspace_size(N, K, a_layout, w_layout)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=a_codes.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    out = _out(M, N, out_type, a_codes.device, out)
    lora_f32 = int(lora_act is not None and lora_act.dtype == torch.float32)
    R = _lora_rank(lora_up, N)
    st = lib.w4a4_gemm(_ptr(a_codes), int(a_layout), _ptr(a_scales), a_gran, int(bool(a_unsigned)), float(a_shift),
                       _ptr(w_packed), int(w_layout), _ptr(w_scales), w_gran, _ptr(w_sum),
                       _ptr(lora_act), lora_f32, _ptr(lora_up), R, _ptr(bias),
                       _ptr(out), out_type, out.stride(0), M, N, K, _ptr(workspace), wsb, _stream(stream))
    _check(st, "w4a4_gemm")
    return out


def w4a8_gemm(a_codes, a_scales, a_gran, w_packed, w_scales, w_zeros, M, N, K, group=16,
              bias=None, out_type=OUT.BF16, out=None, stream=None, lora_act=None, lora_up=None, a_layout=None):
    """a_codes: int8 [M, K] (NATURAL) or float16 [M, K] (F16, the quantizer's
    fp16-carried codes); a_layout defaults from the dtype. lora_act [M, R]
    (bf16 or float32) with L1 bf16 (R = 32 or 64) adds the
    low-rank bypass; lora_up is L1 tiled by w4_pack_lora_up [N/128, R, 128]."""
    if a_layout is None:
        a_layout = LAYOUT.F16 if a_codes.dtype == torch.float16 else LAYOUT.NATURAL
    out = _out(M, N, out_type, a_codes.device, out)
    R = _lora_rank(lora_up, N)
    lora_f32 = int(lora_act is not None and lora_act.dtype == torch.float32)
    st = lib.w4a8_gemm(_ptr(a_codes), int(a_layout), _ptr(a_scales), a_gran, _ptr(w_packed), _ptr(w_scales),
                       _ptr(w_zeros), group, _ptr(lora_act), lora_f32, _ptr(lora_up), R, _ptr(bias),
                       _ptr(out), out_type, out.stride(0),
                       M, N, K, None, 0, _stream(stream))
    _check(st, "w4a8_gemm")
    return out


def int8_tensorwise_gemm(a_codes, a_scale, w, w_scale, M, N, K, bias=None, out_type=OUT.BF16,
                         out=None, stream=None):
    out = _out(M, N, out_type, a_codes.device, out)
    st = lib.int8_tensorwise_gemm(_ptr(a_codes), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(bias),
                                  _ptr(out), out_type, out.stride(0), M, N, K, None, 0,
                                  _stream(stream))
    _check(st, "int8_tensorwise_gemm")
    return out
