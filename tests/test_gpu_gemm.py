"""GPU parity of the GEMM entry points against the CPU oracle.

The GEMMs are fed the ORACLE's codes, scales and packed weights (uploaded),
so these tests isolate the GEMM kernels from the quantizer and the packer.
Bar: int32 results (CR_OUT_I32_RAW) bit-exact; bf16 output within 2e-3
relative L2 of the oracle's float32 epilogue; float32 output within 1e-5.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from oracle import linear as ol, gemm as og, pack as opack, quant as oq  # noqa: E402
from tests.gpu_helpers import bf16_dev, bytes_of, dev, host, rel_l2, bf16_to_f32, say  # noqa: E402

GR = {"tensor": 0, "row": 1, "row_group": 2}


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_rotated_quantized_amd as m
    assert m.device_check() == 0
    return m


def _check_out(y_bf16, y_f32, ref_y, f32_tol=1e-5):
    yb = bf16_to_f32(host(y_bf16))
    assert rel_l2(yb, ref_y) <= 2e-3, rel_l2(yb, ref_y)
    assert rel_l2(host(y_f32), ref_y) <= f32_tol, rel_l2(host(y_f32), ref_y)


W4A4_CASES = [
    # M, N, K, a_gran, w_gran
    (1, 256, 512, "tensor", "tensor"),
    (200, 384, 3072, "tensor", "tensor"),     # 128x192 tiles, ragged M
    (77, 768, 256, "row", "tensor"),          # one stage (K = 256: two 128-deep stages)
    (17, 384, 3072, "tensor", "row"),
    (64, 256, 512, "row", "tensor"),
    (100, 256, 1024, "tensor", "tensor"),
    (256, 384, 3072, "row", "row"),
    (300, 512, 768, "tensor", "tensor"),
    (129, 128, 12288, "tensor", "tensor"),
]


@pytest.mark.parametrize("case", W4A4_CASES)
def test_w4a4_tensor_row(cr, case):
    M, N, K, ag, wg = case
    say(f"w4a4 {case}")
    xb = wl.activation(21, M + N + K, M, K, n_outliers=3, outlier_scale=20.0)
    wb = wl.weight(21, 7 + M + N + K, N, K)
    bias = wl.weight(21, 9, 1, N, std=0.5)[0]
    wp = ol.prepare_w4a4(wb, 256, wg)
    ref = ol.w4a4_linear(xb, wb, 256, ag, wg, wprep=wp)
    ref_b = ol.w4a4_linear(xb, wb, 256, ag, wg, bias_bits=bias, wprep=wp)
    a = dev(ref["x"]["codes"])
    sa = dev(np.asarray(ref["x"]["scales"], np.float32).reshape(-1))
    w = dev(wp["tiles"].reshape(-1))
    sw = dev(np.asarray(wp["scales"], np.float32).reshape(-1))
    raw = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=2)
    assert np.array_equal(host(raw).astype(np.int64), ref["raw"])
    at = dev(opack.tile_pack_a(ref["x"]["codes"]))
    raw_t = cr.w4a4_gemm(at, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=2)
    assert np.array_equal(host(raw_t).astype(np.int64), ref["raw"])
    yt = cr.w4a4_gemm(at, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=1)
    assert rel_l2(host(yt), ref["y"]) <= 1e-5
    _check_out(cr.w4a4_gemm(at, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=0), yt, ref["y"])
    ybias_t = cr.w4a4_gemm(at, sa, GR[ag], w, sw, GR[wg], M, N, K, bias=bf16_dev(bias), out_type=1)
    assert rel_l2(host(ybias_t), ref_b["y"]) <= 1e-5
    yb = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=0)
    yf = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=1)
    _check_out(yb, yf, ref["y"])
    ybias = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, bias=bf16_dev(bias), out_type=1)
    assert rel_l2(host(ybias), ref_b["y"]) <= 1e-5


@pytest.mark.parametrize("rot", [16, 64, 1024])
def test_w4a4_layer_other_group_sizes(cr, rot):
    """A whole W4A4 layer on the GPU path with the ConvRot groups of 16, 64
    and 1024: both operands rotated and quantized by convrot_rotate_quantize,
    weights packed by w4_pack_weights; the raw int32 result is bit-exact and
    the output matches the oracle's layer."""
    M, N, K = 200, 384, 3072
    say(f"w4a4 layer rot {rot}")
    xb = wl.activation(27, rot, M, K, n_outliers=3, outlier_scale=20.0)
    wb = wl.weight(27, rot + 1, N, K)
    ref = ol.w4a4_linear(xb, wb, rot, "tensor", "tensor")
    a, sa, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), rot, 0, 0, layout=1)
    wc, ws, _, _ = cr.convrot_rotate_quantize(bf16_dev(wb), rot, 0, 0)
    w = cr.w4_pack_weights(wc, ws, N, K)[0]
    assert np.array_equal(bytes_of(w), ref["w"]["tiles"].reshape(-1))
    raw = cr.w4a4_gemm(a, sa, 0, w, ws, 0, M, N, K, out_type=2)
    assert np.array_equal(host(raw).astype(np.int64), ref["raw"])
    yf = cr.w4a4_gemm(a, sa, 0, w, ws, 0, M, N, K, out_type=1)
    yb = cr.w4a4_gemm(a, sa, 0, w, ws, 0, M, N, K, out_type=0)
    _check_out(yb, yf, ref["y"])


A8W4_CASES = [(1, 256, 512, "row", "tensor"), (50, 384, 3072, "row", "row"), (200, 256, 1024, "tensor", "tensor"),
              (333, 512, 768, "row", "tensor")]


@pytest.mark.parametrize("case", A8W4_CASES)
def test_a8w4(cr, case):
    """8-bit per-token activations x W4A4-format weights (w4a4_gemm with
    CR_LAYOUT_INT8): int32 bit-exact, outputs to the float bars."""
    M, N, K, ag, wg = case
    say(f"a8w4 {case}")
    xb = wl.activation(28, M + K, M, K, n_outliers=3, outlier_scale=20.0)
    wb = wl.weight(28, N + K, N, K)
    bias = wl.weight(28, 3, 1, N, std=0.5)[0]
    wp = ol.prepare_w4a4(wb, 256, wg)
    ref = ol.a8w4_linear(xb, wb, 256, ag, wg, wprep=wp)
    ref_b = ol.a8w4_linear(xb, wb, 256, ag, wg, bias_bits=bias, wprep=wp)
    a, sa, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, cr.Q.SYM_INT8, GR[ag])
    assert np.array_equal(host(a).view(np.uint8), ref["x"]["codes"].view(np.uint8))
    w = dev(wp["tiles"].reshape(-1))
    sw = dev(np.asarray(wp["scales"], np.float32).reshape(-1))
    kw = dict(a_layout=cr.LAYOUT.INT8)
    raw = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=2, **kw)
    assert np.array_equal(host(raw).astype(np.int64), ref["raw"])
    yf = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=1, **kw)
    yb = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=0, **kw)
    _check_out(yb, yf, ref["y"])
    ybias = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, bias=bf16_dev(bias), out_type=1, **kw)
    assert rel_l2(host(ybias), ref_b["y"]) <= 1e-5


def test_w4a4_ldc_padding(cr):
    M, N, K = 70, 256, 512
    xb = wl.activation(22, 0, M, K)
    wb = wl.weight(22, 1, N, K)
    ref = ol.w4a4_linear(xb, wb)
    out = torch.full((M, N + 64), 7.0, dtype=torch.float32, device="cuda")
    cr.w4a4_gemm(dev(ref["x"]["codes"]), dev(ref["x"]["scales"]), 0, dev(ref["w"]["tiles"].reshape(-1)),
                 dev(ref["w"]["scales"]), 0, M, N, K, out_type=1, out=out)
    o = host(out)
    assert rel_l2(o[:, :N], ref["y"]) <= 1e-5
    assert np.all(o[:, N:] == 7.0)          # nothing written past N


@pytest.mark.parametrize("M", [2, 65, 300, 2600])
def test_int8_ldc_padding(cr, M):
    """INT8 x INT8 into rows of a wider output (ldc = N + 64): the weight
    streaming kernel (2 rows), 64 x 64 blocks (65 rows: one row in the last
    row block; 300 rows) and 256 x 128 blocks (2600 rows); int32, float32 and
    bf16 outputs; nothing written past N."""
    N, K = 384, 512
    if M == 2600:
        N = 3072                                # enough 256 x 128 tiles to fill a 256-CU part
    say(f"int8 ldc padding M {M} N {N}")
    xb = wl.activation(27, M + K, M, K)
    wb = wl.weight(27, N + K, N, K)
    ref = ol.int8_linear(xb, wb)
    a, sa = dev(ref["x"]["codes"]), dev(ref["x"]["scales"])
    w, sw = dev(ref["w"]["codes"]), dev(ref["w"]["scales"])
    raw = torch.full((M, N + 64), -5, dtype=torch.int32, device="cuda")
    cr.int8_tensorwise_gemm(a, sa, w, sw, M, N, K, out_type=2, out=raw)
    r = host(raw)
    assert np.array_equal(r[:, :N].astype(np.int64), ref["raw"])
    assert np.all(r[:, N:] == -5)
    yf = torch.full((M, N + 64), 7.0, dtype=torch.float32, device="cuda")
    cr.int8_tensorwise_gemm(a, sa, w, sw, M, N, K, out_type=1, out=yf)
    o = host(yf)
    assert rel_l2(o[:, :N], ref["y"]) <= 1e-5
    assert np.all(o[:, N:] == 7.0)
    yb = torch.full((M, N + 64), 3.0, dtype=torch.bfloat16, device="cuda")
    cr.int8_tensorwise_gemm(a, sa, w, sw, M, N, K, out_type=0, out=yb)
    ob = bf16_to_f32(host(yb))
    assert rel_l2(ob[:, :N], ref["y"]) <= 2e-3
    assert np.all(ob[:, N:] == 3.0)


G64_CASES = [
    # M, N, K, unsigned, lora(None|bf16|f32), bias
    (16, 256, 512, False, None, False),
    (40, 384, 1024, True, None, False),
    (200, 256, 3072, False, "bf16", True),
    (130, 384, 1024, True, "bf16", False),
    (64, 256, 512, True, "f32", True),
    (257, 128, 768, False, "f32", False),
    (100, 384, 128, False, None, True),      # a single 128-deep stage
]


@pytest.mark.parametrize("case", G64_CASES)
def test_w4a4_group64_lowrank(cr, case):
    M, N, K, uns, lora, use_bias = case
    say(f"w4a4 g64 {case}")
    shift = 0.171875 if uns else 0.0
    xb = wl.gelu_activation(23, M + K, M, K) if uns else wl.activation(23, M + K, M, K)
    wb = wl.weight(23, N + K, N, K)
    l1 = l2 = None
    if lora:
        l1, l2, wb = wl.lowrank_split(wb, 32)
    bias = wl.weight(23, 5, 1, N, std=0.5)[0] if use_bias else None
    wp = ol.prepare_w4a4(wb, 0, "row_group", 64)
    ref = ol.w4a4_linear(xb, wb, 0, "row_group", "row_group", 64, shift, l1, l2,
                         act_f32=(lora == "f32"), bias_bits=bias, wprep=wp)
    a = dev(ref["x"]["codes"])
    sa = dev(ref["x"]["scales"])
    w = dev(wp["tiles"].reshape(-1))
    sw = dev(wp["scales_tiles"].reshape(-1))
    wsum = dev(wp["wsum"])
    la = lu = None
    if lora:
        la = dev(ref["la"]) if lora == "f32" else bf16_dev(wl.bf16_bits_from_f32(ref["la"]))
        lu = bf16_dev(opack.tile_pack_lora_up(l1))
    kw = dict(a_unsigned=uns, a_shift=shift, w_sum=wsum, lora_act=la, lora_up=lu,
              bias=None if bias is None else bf16_dev(bias))
    raw = cr.w4a4_gemm(a, sa, 2, w, sw, 2, M, N, K, out_type=2, **kw)
    assert np.array_equal(host(raw).astype(np.int64), ref["raw"])
    at = dev(opack.tile_pack_a(ref["x"]["codes"]))
    assert np.array_equal(host(cr.w4a4_gemm(at, sa, 2, w, sw, 2, M, N, K, out_type=2, **kw)).astype(np.int64),
                          ref["raw"])
    assert rel_l2(host(cr.w4a4_gemm(at, sa, 2, w, sw, 2, M, N, K, out_type=1, **kw)), ref["y"]) <= 1e-5
    yb = cr.w4a4_gemm(a, sa, 2, w, sw, 2, M, N, K, out_type=0, **kw)
    yf = cr.w4a4_gemm(a, sa, 2, w, sw, 2, M, N, K, out_type=1, **kw)
    _check_out(yb, yf, ref["y"])


# M <= 64: weight streaming on the matrix cores (M = 1 to 5 in one 16-row
# block, the unused rows clamped; the four waves take runs of four 64-deep
# k-tiles: K = 256 leaves three waves idle, 1280 ends in a partial round);
# above: the direct-to-LDS kernel, on a 256-CU part with 64 x 64 blocks while 256 x 128
# tiles would not fill the CUs (190 x 256: 12 blocks, a ragged last row
# block; 512 x 384: 48), then 256 x 128 blocks (2600 x 3072: 264 of them, a
# ragged last row block; 8000 x 3072: 768, the three-blocks-per-CU ring,
# ragged too; with a bias the same shape keeps two blocks per CU)
INT8_CASES = [(1, 128, 256), (2, 256, 3072), (3, 384, 1280), (4, 256, 5120), (5, 128, 512), (33, 384, 512),
              (64, 128, 256), (190, 256, 1024), (512, 384, 3072), (2600, 3072, 256), (8000, 3072, 256)]


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("case", INT8_CASES)
def test_int8_tensorwise(cr, case, bias):
    M, N, K = case
    say(f"int8 {case} bias {bias}")
    xb = wl.activation(24, M + K, M, K, n_outliers=2, outlier_scale=15.0)
    wb = wl.weight(24, N + K, N, K)
    bb = wl.weight(25, N, 1, N).reshape(-1) if bias else None
    ref = ol.int8_linear(xb, wb, bias_bits=bb)
    a = dev(ref["x"]["codes"])
    sa = dev(ref["x"]["scales"])
    w = dev(ref["w"]["codes"])
    sw = dev(ref["w"]["scales"])
    b = bf16_dev(bb) if bias else None
    raw = cr.int8_tensorwise_gemm(a, sa, w, sw, M, N, K, out_type=2)
    assert np.array_equal(host(raw).astype(np.int64), ref["raw"])
    yb = cr.int8_tensorwise_gemm(a, sa, w, sw, M, N, K, bias=b, out_type=0)
    yf = cr.int8_tensorwise_gemm(a, sa, w, sw, M, N, K, bias=b, out_type=1)
    _check_out(yb, yf, ref["y"])


# M, N, K: one block, ragged M over several 256-row blocks, K past one 8192-deep int32 chunk
W4A8_CASES = [(1, 128, 512), (50, 256, 1024), (128, 256, 3072), (333, 384, 768), (520, 256, 12288)]


def _w4a8_args(cr, wp):
    return dev(wp["tiles"].reshape(-1)), dev(wp["scales_tiles"].reshape(-1)), dev(wp["zeros_tiles"].reshape(-1))


@pytest.mark.parametrize("case", W4A8_CASES)
def test_w4a8(cr, case):
    """int32 bit-exact and float outputs to the float32 / bf16 bars, from int8
    and from fp16-carried activation codes (bit-identical outputs: the
    conversion is exact)."""
    M, N, K = case
    say(f"w4a8 {case}")
    xb = wl.activation(25, M + K, M, K)
    wb = wl.weight(25, N + K, N, K)
    bias = wl.weight(25, 3, 1, N, std=0.5)[0]
    wp = ol.prepare_w4a8(wb)
    ref = ol.w4a8_linear(xb, wb, wprep=wp)
    ref_b = ol.w4a8_linear(xb, wb, bias_bits=bias, wprep=wp)
    sa = dev(ref["x"]["scales"])
    w, sw, zw = _w4a8_args(cr, wp)
    for a in (dev(ref["x"]["codes"]), dev(ref["x"]["codes"].astype(np.float16))):
        raw = cr.w4a8_gemm(a, sa, 1, w, sw, zw, M, N, K, out_type=2)
        assert np.array_equal(host(raw).astype(np.int64), ref["raw"])
        yb = cr.w4a8_gemm(a, sa, 1, w, sw, zw, M, N, K, out_type=0)
        yf = cr.w4a8_gemm(a, sa, 1, w, sw, zw, M, N, K, out_type=1)
        _check_out(yb, yf, ref["y"])
        ybias = cr.w4a8_gemm(a, sa, 1, w, sw, zw, M, N, K, bias=bf16_dev(bias), out_type=1)
        assert rel_l2(host(ybias), ref_b["y"]) <= 1e-5
        if a.dtype == torch.int8:
            y8 = (host(yb), host(yf))
        else:
            assert np.array_equal(host(yb), y8[0]) and np.array_equal(host(yf).view(np.uint32), y8[1].view(np.uint32))


@pytest.mark.parametrize("K", [256, 1024])
def test_w4a8_float_partials_exact(cr, K):
    """The float-output kernel forms each 16-group partial exactly: with unit
    scales its float32 output is the integer sum itself, and with power-of-two
    scales (token and channel-group) it is the exact dyadic value of
    s_a sum_g s_w P, bit for bit (both fit float32 at these sizes)."""
    M, N = 300, 256
    say(f"w4a8 exact partials K={K}")
    xb = wl.activation(31, K, M, K)
    wb = wl.weight(31, K + 1, N, K)
    wp = ol.prepare_w4a8(wb)
    xa = ol.rotate_quantize(xb, 256, "int8", "row")
    w, _, zw = _w4a8_args(cr, wp)
    P = og.group_partials(xa["values"], wp["values"], 16, wp["zeros"])
    ones16 = np.ones_like(wp["scales"], dtype=np.float16)
    y = cr.w4a8_gemm(dev(xa["codes"]), dev(np.ones(M, np.float32)), 1, w, dev(opack.tile_pack_g16(ones16).reshape(-1)),
                     zw, M, N, K, out_type=1)
    assert np.array_equal(host(y).astype(np.int64), P.sum(axis=2))
    rng = np.random.default_rng(K)
    ea, ew = rng.integers(-3, 1, M), rng.integers(-3, 1, (N, K // 16))
    sa2 = np.ldexp(1.0, ea).astype(np.float32)
    sw2 = np.ldexp(1.0, ew).astype(np.float16)
    y2 = cr.w4a8_gemm(dev(xa["codes"]), dev(sa2), 1, w, dev(opack.tile_pack_g16(sw2).reshape(-1)), zw, M, N, K,
                      out_type=1)
    exact = np.ldexp(1.0, ea)[:, None] * np.einsum("ng,mng->mn", np.ldexp(1.0, ew), P.astype(np.float64))
    assert np.max(np.abs(exact)) < 2.0 ** 21
    assert np.array_equal(host(y2).astype(np.float64), exact)
    assert np.array_equal(host(y2), ol.epilogue_g16(P, sa2, "row", sw2))


@pytest.mark.parametrize("R,la_f32", [(32, False), (64, False), (32, True)])
def test_w4a8_lora_bypass(cr, R, la_f32):
    """A LoRA kept as a low-rank branch beside the W4A8 weight: la from the
    rotate+quantize call on the unrotated input (bf16, or float32 with the
    FP32 switch), the up-projection fused into the GEMM epilogue; the output
    against the oracle's linear with the same branch."""
    M, N, K = 333, 256, 3072
    say(f"w4a8 lora R={R} f32={la_f32}")
    xb = wl.activation(29, R, M, K)
    wb = wl.weight(29, R + 1, N, K)
    l1 = wl.weight(29, R + 2, N, R, std=0.05)
    l2 = wl.weight(29, R + 3, R, K, std=0.05)
    bias = wl.weight(29, R + 4, 1, N, std=0.5)[0]
    wp = ol.prepare_w4a8(wb)
    ref = ol.w4a8_linear(xb, wb, wprep=wp, l1_bits=l1, l2_bits=l2, bias_bits=bias, act_f32=la_f32)
    a, sa, _, la = cr.convrot_rotate_quantize(bf16_dev(xb), 256, cr.Q.SYM_INT8, cr.GRAN.ROW, lora_down=bf16_dev(l2),
                                              lora_act_f32=la_f32, layout=cr.LAYOUT.F16)
    assert np.array_equal(host(a).astype(np.int64), ref["x"]["values"].astype(np.int64))
    args = (a, sa, 1, *_w4a8_args(cr, wp), M, N, K)
    # the epilogue on the oracle's la (identical inputs): float32 bar
    la_ref = dev(ref["la"]) if la_f32 else bf16_dev(wl.bf16_bits_from_f32(ref["la"]))
    kw = dict(lora_act=la_ref, lora_up=bf16_dev(opack.tile_pack_lora_up(l1)), bias=bf16_dev(bias))
    _check_out(cr.w4a8_gemm(*args, out_type=0, **kw), cr.w4a8_gemm(*args, out_type=1, **kw), ref["y"])
    # end to end with the GPU's la (its rounding may differ by one ulp): bf16 bar
    ye = cr.w4a8_gemm(*args, out_type=0, lora_act=la, lora_up=bf16_dev(opack.tile_pack_lora_up(l1)), bias=bf16_dev(bias))
    assert rel_l2(bf16_to_f32(host(ye)), ref["y"]) <= 2e-3


@pytest.mark.parametrize("R", [32, 64])
def test_w4a4_lora_rank(cr, R):
    """W4A4 tensorwise with ConvRot and a rank-R bypass (la from the rotated
    rotate+quantize call), against the oracle's linear."""
    M, N, K = 200, 384, 3072
    say(f"w4a4 lora R={R}")
    xb = wl.activation(30, R, M, K, n_outliers=3, outlier_scale=20.0)
    wb = wl.weight(30, R + 1, N, K)
    l1 = wl.weight(30, R + 2, N, R, std=0.05)
    l2 = wl.weight(30, R + 3, R, K, std=0.05)
    wp = ol.prepare_w4a4(wb, 256, "tensor")
    ref = ol.w4a4_linear(xb, wb, 256, "tensor", "tensor", l1_bits=l1, l2_bits=l2, wprep=wp)
    a, sa, _, la = cr.convrot_rotate_quantize(bf16_dev(xb), 256, 0, 0, layout=1, lora_down=bf16_dev(l2))
    w = dev(wp["tiles"].reshape(-1))
    sw = dev(np.asarray(wp["scales"], np.float32).reshape(-1))
    # the epilogue on the oracle's la (identical inputs): float32 bar
    la_ref = bf16_dev(wl.bf16_bits_from_f32(ref["la"]))
    yf = cr.w4a4_gemm(a, sa, 0, w, sw, 0, M, N, K, lora_act=la_ref, lora_up=bf16_dev(opack.tile_pack_lora_up(l1)), out_type=1)
    yb = cr.w4a4_gemm(a, sa, 0, w, sw, 0, M, N, K, lora_act=la_ref, lora_up=bf16_dev(opack.tile_pack_lora_up(l1)), out_type=0)
    _check_out(yb, yf, ref["y"])
    # end to end with the GPU's la (its bf16 rounding may differ by one ulp): bf16 bar
    ye = cr.w4a4_gemm(a, sa, 0, w, sw, 0, M, N, K, lora_act=la, lora_up=bf16_dev(opack.tile_pack_lora_up(l1)), out_type=0)
    assert rel_l2(bf16_to_f32(host(ye)), ref["y"]) <= 2e-3


def test_extreme_codes_no_overflow(cr):
    # all codes at +-qmax over the largest K: the int32 accumulators must stay exact
    M, N, K = 64, 128, 32768
    qa = np.full((M, K), 7, np.int64)
    qa[::2] = -7
    qw = np.full((N, K), -7, np.int64)
    from oracle import pack as opack
    a = dev(opack.pack_int4(qa))
    w = dev(opack.tile_pack_w4a4(opack.pack_int4(qw)).reshape(-1))
    one = dev(np.ones(1, np.float32))
    raw = cr.w4a4_gemm(a, one, 0, w, one, 0, M, N, K, out_type=2)
    assert np.array_equal(host(raw).astype(np.int64), og.int_gemm(qa, qw))
    # int8: 127 * 127 * 16384 = 264,257,536 < 2^31
    K8 = 16384
    q8 = np.full((M, K8), 127, np.int64)
    w8 = np.full((N, K8), -127, np.int64)
    raw8 = cr.int8_tensorwise_gemm(dev(q8.astype(np.int8)), one, dev(w8.astype(np.int8)), one, M, N, K8,
                                   out_type=2)
    assert np.array_equal(host(raw8).astype(np.int64), og.int_gemm(q8, w8))


def test_extreme_codes_matrix_core_paths(cr):
    """All codes at +-qmax over K = 32768 on the block kernels (M > 64): the
    fp6 path's float32 sums (|sum| <= 32768 * 49 < 2^24) and the int8 64 x 64
    blocks' int32 sums (127 * 127 * 32768 < 2^31) stay exact."""
    M, N, K = 130, 256, 32768                     # 130 rows: a ragged last row block
    qa = np.full((M, K), 7, np.int64)
    qa[::2] = -7
    qa[:, ::3] *= -1
    qw = np.full((N, K), -7, np.int64)
    qw[1::2] = 7
    from oracle import pack as opack
    one = dev(np.ones(1, np.float32))
    af6 = dev(opack.f6_pack(qa))
    wf6 = dev(opack.f6_pack(qw))
    raw = cr.w4a4_gemm(af6, one, 0, wf6, one, 0, M, N, K, out_type=2)
    assert np.array_equal(host(raw).astype(np.int64), og.int_gemm(qa, qw))
    q8 = np.full((M, K), 127, np.int64)
    q8[::3] = -127
    w8 = np.full((N, K), -127, np.int64)
    w8[:, 1::2] = 127
    raw8 = cr.int8_tensorwise_gemm(dev(q8.astype(np.int8)), one, dev(w8.astype(np.int8)), one, M, N, K,
                                   out_type=2)
    assert np.array_equal(host(raw8).astype(np.int64), og.int_gemm(q8, w8))


@pytest.mark.parametrize("M", [1, 2, 3])
def test_extreme_codes_int8_streaming(cr, M):
    """All codes at +-127 over K = 32768 on the weight streaming kernel (one
    to three tokens): the int32 sums stay exact (127 * 127 * 32768 < 2^31),
    float32 outputs are their scaled values."""
    N, K = 256, 32768
    say(f"int8 streaming extreme codes M {M}")
    q8 = np.full((M, K), 127, np.int64)
    q8[:, ::5] = -127
    w8 = np.full((N, K), -127, np.int64)
    w8[::3, 1::2] = 127
    w8[:, ::7] *= -1
    one = dev(np.ones(1, np.float32))
    a, w = dev(q8.astype(np.int8)), dev(w8.astype(np.int8))
    want = og.int_gemm(q8, w8)
    assert np.array_equal(host(cr.int8_tensorwise_gemm(a, one, w, one, M, N, K, out_type=2)).astype(np.int64), want)
    sa, sw = dev(np.array([0.5], np.float32)), dev(np.array([0.25], np.float32))
    yf = host(cr.int8_tensorwise_gemm(a, sa, w, sw, M, N, K, out_type=1)).astype(np.float64)
    assert np.array_equal(yf, want.astype(np.float32).astype(np.float64) * 0.125)


def test_gemm_determinism(cr):
    """Repeated calls give bit-identical outputs: the fp6 W4A4 path (4-bit
    weight tiles expanded per call), the int8-core W4A4 path, INT8 x INT8 and
    W4A8, each twice on the same inputs."""
    M, N, K = 1000, 768, 3072
    say("gemm determinism")
    xb = wl.activation(32, 0, M, K, n_outliers=3, outlier_scale=20.0)
    wb = wl.weight(32, 1, N, K)
    x, w = bf16_dev(xb), bf16_dev(wb)
    wc, ws, _, _ = cr.convrot_rotate_quantize(w, 256, 0, 0)
    wt = cr.w4_pack_weights(wc, ws, N, K)[0]
    a6, s6, _, _ = cr.convrot_rotate_quantize(x, 256, 0, 0, layout=cr.LAYOUT.F6)
    at, st, _, _ = cr.convrot_rotate_quantize(x, 256, 0, 0, layout=cr.LAYOUT.TILED)
    a8, s8, _, _ = cr.convrot_rotate_quantize(x, 256, 1, 0)
    w8, ws8, _, _ = cr.convrot_rotate_quantize(w, 256, 1, 0)
    ah, sh, _, _ = cr.convrot_rotate_quantize(x, 256, 1, 1, layout=cr.LAYOUT.F16)
    wa, wsa, wza, _ = cr.convrot_rotate_quantize(w, 256, 3, 2, 16)
    pa, psa, pza, _ = cr.w4_pack_weights(wa, wsa, N, K, 3, 2, 16, zeros=wza)
    calls = [lambda: cr.w4a4_gemm(a6, s6, 0, wt, ws, 0, M, N, K),
             lambda: cr.w4a4_gemm(at, st, 0, wt, ws, 0, M, N, K),
             lambda: cr.int8_tensorwise_gemm(a8, s8, w8, ws8, M, N, K),
             lambda: cr.w4a8_gemm(ah, sh, 1, pa, psa, pza, M, N, K)]
    for f in calls:
        y0, y1 = host(f()), host(f())
        assert np.array_equal(y0, y1)
