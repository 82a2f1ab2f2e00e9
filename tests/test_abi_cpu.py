"""The C-ABI library loads, exports every symbol include/convrot.h declares,
and rejects bad arguments with the documented status BEFORE touching a
device. No compute call runs here (no GPU in this environment); a call with
valid arguments reaches the device check and reports the missing device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")
LIB = os.path.join(ROOT, "w4a8_rotated_quantized_amd", "libconvrot.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libconvrot.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted({n for n in names if n not in ("if", "while", "sizeof")})


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    names = _declared_functions()
    assert {"convrot_rotate_quantize", "w4_pack_weights", "w4a4_gemm", "w4a8_gemm",
            "int8_tensorwise_gemm"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


@pytest.fixture(scope="module")
def cr():
    import w4a8_rotated_quantized_amd as m
    return m


class _FakeDev:
    """Stands in for a device tensor: a 16-byte aligned non-null address that
    is never dereferenced (validation happens before any device access)."""
    def __init__(self, addr=0x10000):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _p(v):
    return ctypes.c_void_p(v)


A = 0x10000  # aligned fake device address


def test_status_strings(cr):
    assert cr.status_string(3) == "format not available"
    assert "gfx950" in cr.status_string(5)
    assert cr.status_string(0) == "ok"


def test_counters_have_no_fallback(cr):
    c = cr.get_counters()
    assert c["fallbacks"] == 0


def test_device_check_reports_no_device_here(cr):
    assert cr.device_check() in (4, 5)


def _rq(cr, x=A, rows=64, K=512, ldx=512, rot=256, q=0, g=0, qg=0, lora=None, R=0, la=None,
        codes=A, scales=A, zeros=None, ws=A, wsb=1 << 20, layout=0, smooth=None):
    return cr.lib.convrot_rotate_quantize(_p(x), rows, K, ldx, rot, q, g, qg, 0.0, _p(smooth), _p(lora), R, _p(la),
                                          0, _p(codes), layout, _p(scales), _p(zeros), _p(ws), wsb, None)


def test_rq_validation(cr):
    assert _rq(cr, x=None) == 1                              # null input
    assert _rq(cr, x=A + 4) == 1                             # misaligned
    assert _rq(cr, K=300, ldx=304) == 2                      # K % 256 with rotation
    assert _rq(cr, ldx=500) == 2                             # ldx < K
    assert _rq(cr, rows=0) == 2
    assert _rq(cr, K=65536, ldx=65536) == 2                  # above K limit
    assert _rq(cr, rot=128) == 3                             # group size not available
    assert _rq(cr, rot=32) == 3
    for rot in (16, 64, 1024):                               # the other ConvRot groups (power-of-four sizes)
        assert _rq(cr, rot=rot, K=1024, ldx=1024) == 4
    assert _rq(cr, rot=1024, K=512, ldx=512) == 2            # K % 1024 with the 1024 rotation
    assert _rq(cr, rot=64, q=3, g=2, qg=16, zeros=A) == 3    # asymmetric g16 weights: 256 only
    assert _rq(cr, q=2) == 3                                 # shift path needs rot 0
    assert _rq(cr, q=3, g=2, qg=16) == 1                     # asym needs zeros
    assert _rq(cr, q=3, g=0) == 3                            # asym needs ROW_GROUP(16)
    assert _rq(cr, g=2, qg=32) == 3                          # group 32 not available
    assert _rq(cr, rot=0, g=0) == 3                          # rot 0 needs ROW_GROUP(64)
    assert _rq(cr, rot=0, g=2, qg=64, lora=A, R=16, la=A) == 3   # rank must be 32 or 64
    assert _rq(cr, rot=256, lora=A, R=32, la=A) == 4          # low rank beside the rotation (bypass)
    assert _rq(cr, rot=256, lora=A, R=64, la=A) == 4
    assert _rq(cr, rot=256, lora=A, R=64) == 1                # needs its output
    assert _rq(cr, q=3, g=2, qg=16, zeros=A, lora=A, R=32, la=A) == 3   # not for asymmetric weights
    assert _rq(cr, wsb=0) == 6                               # TENSOR needs workspace
    assert _rq(cr, q=1, layout=1) == 3                       # tiled layout is for int4 codes
    assert _rq(cr, layout=2) == 1
    assert _rq(cr, layout=5) == 1
    assert _rq(cr, layout=4) == 3                            # fp16-carried codes are int8 codes
    assert _rq(cr, layout=4, q=1) == 4
    assert _rq(cr, layout=4, q=1, g=1, ws=None, wsb=0) == 4
    assert _rq(cr, layout=4, q=1, rot=0, g=2, qg=64, ws=None, wsb=0) == 3   # rotated codes only
    assert _rq(cr, layout=3) == 4                            # fp6 fragments of rotated int4 codes
    assert _rq(cr, layout=3, g=1) == 4
    assert _rq(cr, layout=3, q=1) == 3                       # not for int8 codes
    assert _rq(cr, layout=3, rot=0, g=2, qg=64, ws=None, wsb=0) == 4   # 64-group codes without rotation
    assert _rq(cr, layout=3, rot=0, q=2, g=2, qg=64, ws=None, wsb=0) == 4   # unsigned shifted codes too
    assert _rq(cr, layout=3, q=3, g=2, qg=16, zeros=A) == 3   # asymmetric weight codes: no fp6 layout
    assert _rq(cr, smooth=A, g=1) == 4                       # smoothing: rotation 256 with row scales
    assert _rq(cr, smooth=A, g=2, qg=64) == 4
    assert _rq(cr, smooth=A) == 3                            # not with per-tensor scales
    assert _rq(cr, smooth=A, rot=64, g=1) == 3               # nor other rotation sizes
    assert _rq(cr, smooth=A + 4, g=1) == 1                   # misaligned
    assert _rq(cr, smooth=A, rot=0, g=2, qg=64, ws=None, wsb=0) == 4
    assert _rq(cr, layout=1) == 4
    assert _rq(cr) == 4                                      # valid -> device check (no GPU here)
    assert _rq(cr, rot=0, g=2, qg=64, ws=None, wsb=0) == 4


def test_rq_dual_validation(cr):
    L = cr.lib
    def dual(rot=256, x=A, c8=A, s8=A, ws=A, wsb=1 << 20, layout=1, K=1024):
        return L.convrot_rotate_quantize_dual(_p(x), 64, K, K, rot, _p(A), layout, _p(A), _p(c8), _p(s8), _p(ws),
                                              wsb, None)
    assert dual(rot=0) == 3                  # the rotated per-tensor path only
    assert dual(x=None) == 1
    assert dual(c8=None) == 1
    assert dual(s8=A + 4) == 1               # misaligned
    assert dual(layout=2) == 1
    assert dual(layout=3) == 4               # fp6 fragments for the int4 set
    assert dual(ws=None) == 1
    assert dual(wsb=0) == 6
    assert dual(K=300) == 2
    for rot in (16, 64, 256, 1024):
        assert dual(rot=rot) == 4            # valid -> device check (no GPU here)


def test_dequantize_validation(cr):
    L = cr.lib
    def deq(codes=A, scales=A, zeros=None, N=128, K=1024, q=0, g=0, qg=0, rot=256, up=None, down=None, R=0, out=A):
        return L.convrot_dequantize_weights(_p(codes), _p(scales), _p(zeros), N, K, q, g, qg, rot, _p(up), _p(down),
                                            R, _p(out), None)
    assert deq(codes=None) == 1
    assert deq(out=A + 8) == 1
    assert deq(K=1000) == 2
    assert deq(rot=128) == 3
    assert deq(rot=1024, K=1536) == 2
    assert deq(q=2) == 3                         # activation-only format
    assert deq(q=1, g=2, qg=64) == 3             # int8 weights: tensor or row
    assert deq(q=3, g=2, qg=16) == 1             # asymmetric: needs zeros
    assert deq(q=3, g=2, qg=16, zeros=A, rot=64) == 3
    assert deq(up=A, R=16) == 1                  # both factors
    assert deq(up=A, down=A, R=0) == 1
    assert deq(up=A, down=A, R=16) == 4
    assert deq(q=3, g=2, qg=16, zeros=A) == 4
    assert deq() == 4


def test_rq_workspace_size(cr):
    n = cr.convrot_rq_workspace_size(4096, 3072, 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR)
    assert n > 0 and n % 4 == 0
    assert cr.convrot_rq_workspace_size(4096, 3072, 256, cr.Q.SYM_INT4, cr.GRAN.ROW) == 0
    for rot in (16, 64, 1024):
        assert cr.convrot_rq_workspace_size(4096, 3072, rot, cr.Q.SYM_INT4, cr.GRAN.TENSOR) > 0
    assert cr.convrot_rq_workspace_size(4096, 2560, 1024, cr.Q.SYM_INT4, cr.GRAN.TENSOR) == 0


def test_size_queries_return_zero_for_refused_shapes(cr):
    """Every size query answers 0 for a shape its call refuses (K above 32768,
    rows or N at 2^31 and beyond) instead of multiplying out of range."""
    big = 1 << 40
    assert cr.convrot_rq_workspace_size(1 << 31, 3072, 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR) == 0
    assert cr.convrot_rq_workspace_size(4096, 65536, 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR) == 0
    assert cr.convrot_rq_workspace_size(big, big, 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR) == 0
    for which in (0, 1, 2):
        assert cr.w4_packed_bytes(big, big, 3, 2, 16, which) == 0
        assert cr.w4_packed_bytes(1 << 31, 512, 3, 2, 16, which) == 0
        assert cr.w4_packed_bytes(256, 65536, 0, 2, 64, which) == 0
    assert cr.w4_packed_f6_bytes(big, big) == 0
    assert cr.w4_packed_f6_bytes(1 << 31, 512) == 0
    assert cr.w4_packed_f6_bytes(256, 65536) == 0
    assert cr.w4a4_gemm_workspace_size(big, big, cr.LAYOUT.F6, cr.LAYOUT.TILED) == 0
    assert cr.w4a4_gemm_workspace_size(256, 65536, cr.LAYOUT.F6, cr.LAYOUT.TILED) == 0
    # the largest accepted shapes still get their sizes
    assert cr.w4_packed_bytes((1 << 31) - 128, 32768, 0, 0, 0, 0) == ((1 << 31) - 128) * 16384
    assert cr.w4_packed_f6_bytes(12288, 32768) == 12288 * 32768 * 3 // 4
    assert cr.w4a4_gemm_workspace_size(12288, 32768, cr.LAYOUT.F6, cr.LAYOUT.TILED) == 12288 * 32768 * 3 // 4


def test_pack_validation(cr):
    L = cr.lib
    assert L.w4_pack_weights(_p(A), _p(A), None, 100, 512, 0, 0, 0, _p(A), None, None, None, None) == 2
    assert L.w4_pack_weights(None, _p(A), None, 128, 512, 0, 0, 0, _p(A), None, None, None, None) == 1
    assert L.w4_pack_weights(_p(A), _p(A), None, 128, 512, 0, 2, 32, _p(A), _p(A), None, None, None) == 3
    assert L.w4_pack_weights(_p(A), _p(A), None, 128, 512, 3, 2, 16, _p(A), _p(A), _p(A), None, None) == 1
    assert L.w4_pack_weights(_p(A), _p(A), None, 128, 512, 1, 0, 0, _p(A), None, None, None, None) == 3
    assert L.w4_pack_weights(_p(A), _p(A), None, 128, 512, 0, 0, 0, _p(A), None, None, None, None) == 4
    # ASYM_UINT4 g16: no column sums (the W4A8 GEMM takes none)
    assert L.w4_pack_weights(_p(A), _p(A), _p(A), 128, 512, 3, 2, 16, _p(A), _p(A), _p(A), _p(A), None) == 1
    assert L.w4_pack_weights(_p(A), _p(A), _p(A), 128, 512, 3, 2, 16, _p(A), _p(A), _p(A), None, None) == 4
    assert cr.w4_packed_bytes(256, 512, 0, 0, 0, 0) == 256 * 256
    assert cr.w4_packed_f6_bytes(256, 512) == 256 * 512 * 3 // 4
    assert cr.w4_packed_f6_bytes(96, 512) == 0
    assert L.w4_pack_weights_f6(_p(A), 128, 512, _p(A), None) == 4
    assert L.w4_pack_weights_f6(_p(A), 100, 512, _p(A), None) == 2
    assert L.w4_pack_weights_f6(_p(A), 128, 448, _p(A), None) == 2
    assert L.w4_pack_weights_f6(None, 128, 512, _p(A), None) == 1
    assert L.w4_pack_weights_f6(_p(A), 128, 512, _p(A + 4), None) == 1
    assert L.w4_pack_lora_up(_p(A), 256, 32, _p(A), None) == 4
    assert L.w4_pack_lora_up(_p(A), 200, 32, _p(A), None) == 2
    assert L.w4_pack_lora_up(_p(A), 256, 16, _p(A), None) == 3
    assert L.w4_pack_lora_up(None, 256, 32, _p(A), None) == 1
    assert L.w4_expand_weights_f6(_p(A), 128, 512, _p(A), None) == 4
    assert L.w4_expand_weights_f6(_p(A), 100, 512, _p(A), None) == 2
    assert L.w4_expand_weights_f6(_p(A), 128, 448, _p(A), None) == 2
    assert L.w4_expand_weights_f6(_p(A), 128, 65536, _p(A), None) == 2
    assert L.w4_expand_weights_f6(None, 128, 512, _p(A), None) == 1
    assert L.w4_expand_weights_f6(_p(A + 4), 128, 512, _p(A), None) == 1
    assert cr.w4_packed_bytes(256, 512, 0, 2, 64, 1) == 256 * 8 * 4
    assert cr.w4_packed_bytes(256, 512, 3, 2, 16, 2) == 256 * 32


def _w4a4(cr, a=A, ag=0, wg=0, uns=0, wsum=None, la=None, lu=None, R=0, out=A, ot=0, ldc=256,
          M=64, N=256, K=512, layout=1, wlayout=None, ws=None, wsb=0):
    if wlayout is None:
        wlayout = 3 if layout == 3 else 1
    return cr.lib.w4a4_gemm(_p(a), layout, _p(A), ag, uns, 0.0, _p(A), wlayout, _p(A), wg, _p(wsum), _p(la), 0,
                            _p(lu), R, None, _p(out), ot, ldc, M, N, K, _p(ws), wsb, None)


def test_gemm_validation(cr):
    assert _w4a4(cr, a=None) == 1
    assert _w4a4(cr, N=200, ldc=200) == 2
    assert _w4a4(cr, K=192) == 2
    assert _w4a4(cr, ldc=128) == 2
    assert _w4a4(cr, M=0) == 2
    assert _w4a4(cr, ag=2, wg=0) == 3                        # group x tensor scales
    assert _w4a4(cr, uns=1) == 1                             # unsigned needs w_sum
    assert _w4a4(cr, la=A, lu=None, R=32) == 3
    assert _w4a4(cr, la=A, lu=A, R=16) == 3
    assert _w4a4(cr, la=A, lu=A, R=64) == 4
    assert _w4a4(cr, ot=5) == 1
    assert _w4a4(cr, layout=5) == 1
    # fp6 codes with int4 tile-packed weights: expanded in the workspace first
    need = cr.w4a4_gemm_workspace_size(256, 512, 3, 1)
    assert need == (256 // 32) * (512 // 64) * 1536
    assert cr.w4a4_gemm_workspace_size(256, 512, 1, 1) == 0
    assert cr.w4a4_gemm_workspace_size(256, 512, 3, 3) == 0
    assert _w4a4(cr, layout=3, wlayout=1) == 1                # workspace missing
    assert _w4a4(cr, layout=3, wlayout=1, ws=A, wsb=need - 16) == 6
    assert _w4a4(cr, layout=3, wlayout=1, ws=A + 8, wsb=need) == 1
    assert _w4a4(cr, layout=3, wlayout=1, ws=A, wsb=need) == 4
    assert _w4a4(cr, layout=1, wlayout=3) == 3                # fp6 weights need fp6 codes
    assert _w4a4(cr, layout=1, wlayout=2) == 1
    assert _w4a4(cr, layout=3) == 4                          # fp6 fragments, tensor scales
    assert _w4a4(cr, layout=3, ag=1, wg=1) == 4
    assert _w4a4(cr, layout=3, ag=2, wg=2) == 4              # fp6 with 64-group scales
    assert _w4a4(cr, layout=3, ag=2, wg=2, uns=1, wsum=A, la=A, lu=A, R=64) == 4
    assert _w4a4(cr, layout=3, ag=2, wg=0) == 3
    assert _w4a4(cr, layout=3, ag=2, wg=2, uns=1) == 1        # unsigned codes need the column sums
    assert _w4a4(cr, layout=3, ag=2, wg=2, la=A, lu=A, R=16) == 3   # rank 32 or 64 only
    assert _w4a4(cr, layout=3, uns=1, wsum=A) == 3           # fp6, tensor scales: signed codes only
    assert _w4a4(cr, layout=3, la=A, lu=A, R=32) == 3        # and no low-rank branch
    assert _w4a4(cr, layout=2, uns=1, wsum=A) == 3           # 8-bit activations: signed only
    assert _w4a4(cr, layout=2, ag=2, wg=2) == 3              # no 64-group scales with them
    assert _w4a4(cr, layout=2, la=A, lu=A, R=32) == 3        # no low-rank branch with them
    assert _w4a4(cr, layout=2, ag=1) == 4
    assert _w4a4(cr, M=1 << 20, K=32768, ldc=256) == 2        # M*K/2 beyond 32-bit offsets
    assert _w4a4(cr) == 4
    L = cr.lib
    def w4a8(ag=1, group=16, la=None, lu=None, R=0, ot=0, layout=0, la_f32=0):
        return L.w4a8_gemm(_p(A), layout, _p(A), ag, _p(A), _p(A), _p(A), group, _p(la), la_f32, _p(lu), R, None,
                           _p(A), ot, 256, 64, 256, 512, None, 0, None)
    assert w4a8(group=32) == 3
    assert w4a8(ag=2) == 3
    assert w4a8(layout=1) == 1                               # int8 natural or fp16-carried codes only
    assert w4a8(layout=4) == 4
    assert w4a8(ot=2) == 4
    # low-rank bypass: rank 32 or 64, both factors; bf16 or float32 activations
    assert w4a8(la=A, lu=A, R=16) == 3
    assert w4a8(la=A, R=32) == 3
    assert w4a8(la=A, lu=A, R=64) == 4
    assert w4a8(la=A, lu=A, R=32, la_f32=1) == 4
    assert w4a8() == 4
    assert L.int8_tensorwise_gemm(_p(A), None, _p(A), _p(A), None, _p(A), 0, 256, 64, 256, 512,
                                  None, 0, None) == 1
    assert L.int8_tensorwise_gemm(_p(A), _p(A), _p(A), _p(A), None, _p(A), 0, 256, 64, 256, 512,
                                  None, 0, None) == 4


def test_noalloc_validation(cr):
    """The allocation-free rotate+quantize validates like the ordinary one and
    refuses inputs whose per-tensor block maxima exceed its fixed scratch
    array (checked before any device access: no device here)."""
    L = cr.lib
    def na(rows=64, K=512, q=0, g=0, layout=0):
        return L.convrot_rotate_quantize_noalloc(_p(A), rows, K, K, 256, q, g, 0, 0.0, None, None, 0, None, 0,
                                                 _p(A), layout, _p(A), None, None)
    assert na() == 4                                          # valid: reaches the device check
    assert na(q=1, layout=4) == 4
    assert na(layout=5) == 1
    need = cr.convrot_rq_workspace_size(1 << 21, 32768, 256, 0, 0)
    assert need > 65536 * 4
    assert na(rows=1 << 21, K=32768) == 6                     # beyond the scratch array
    assert na(rows=1 << 21, K=32768, g=1) == 4                # per-row scales use no scratch
    assert cr.convrot_rq_workspace_size(65536, 16384, 256, 0, 0) <= 65536 * 4
