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


# The W4A8 float outputs come from weights dequantized to fp16(s * (q - z)) on
# the fp16 matrix cores: one rounding per weight, |delta| <= 2^-11, which for
# uncorrelated errors gives a relative L2 of about 2^-11 / sqrt(3) = 2.8e-4 on
# the float32 output. The bar for it is 1e-3; the bf16 bar stays 2e-3 and the
# exact int32 output (int8 matrix cores) stays bit-exact.
W4A8_F32_TOL = 1e-3


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
        lu = bf16_dev(l1)
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


# M <= 64: weight streaming; above: the direct-to-LDS kernel of 256 x 128
# blocks (2600 x 3072: 264 of them, a ragged last row block)
INT8_CASES = [(2, 256, 3072), (33, 384, 512), (64, 128, 256), (190, 256, 1024), (512, 384, 3072), (2600, 3072, 256)]


@pytest.mark.parametrize("case", INT8_CASES)
def test_int8_tensorwise(cr, case):
    M, N, K = case
    say(f"int8 {case}")
    xb = wl.activation(24, M + K, M, K, n_outliers=2, outlier_scale=15.0)
    wb = wl.weight(24, N + K, N, K)
    ref = ol.int8_linear(xb, wb)
    a = dev(ref["x"]["codes"])
    sa = dev(ref["x"]["scales"])
    w = dev(ref["w"]["codes"])
    sw = dev(ref["w"]["scales"])
    raw = cr.int8_tensorwise_gemm(a, sa, w, sw, M, N, K, out_type=2)
    assert np.array_equal(host(raw).astype(np.int64), ref["raw"])
    yb = cr.int8_tensorwise_gemm(a, sa, w, sw, M, N, K, out_type=0)
    yf = cr.int8_tensorwise_gemm(a, sa, w, sw, M, N, K, out_type=1)
    _check_out(yb, yf, ref["y"])


W4A8_CASES = [(1, 128, 512), (50, 256, 1024), (128, 256, 3072), (333, 384, 768)]


@pytest.mark.parametrize("case", W4A8_CASES)
def test_w4a8(cr, case):
    M, N, K = case
    say(f"w4a8 {case}")
    xb = wl.activation(25, M + K, M, K)
    wb = wl.weight(25, N + K, N, K)
    bias = wl.weight(25, 3, 1, N, std=0.5)[0]
    wp = ol.prepare_w4a8(wb)
    ref = ol.w4a8_linear(xb, wb, wprep=wp)
    ref_b = ol.w4a8_linear(xb, wb, bias_bits=bias, wprep=wp)
    a = dev(ref["x"]["codes"])
    sa = dev(ref["x"]["scales"])
    w = dev(wp["tiles"].reshape(-1))
    sw = dev(wp["scales_tiles"].reshape(-1))
    zw = dev(wp["zeros_tiles"].reshape(-1))
    ws = dev(wp["wsum16"])
    raw = cr.w4a8_gemm(a, sa, 1, w, sw, zw, M, N, K, out_type=2)
    assert np.array_equal(host(raw).astype(np.int64), ref["raw"])
    yb = cr.w4a8_gemm(a, sa, 1, w, sw, zw, M, N, K, out_type=0, w_sum=ws)
    yf = cr.w4a8_gemm(a, sa, 1, w, sw, zw, M, N, K, out_type=1, w_sum=ws)
    _check_out(yb, yf, ref["y"], f32_tol=W4A8_F32_TOL)
    ybias = cr.w4a8_gemm(a, sa, 1, w, sw, zw, M, N, K, bias=bf16_dev(bias), out_type=1, w_sum=ws)
    assert rel_l2(host(ybias), ref_b["y"]) <= W4A8_F32_TOL


@pytest.mark.parametrize("R", [32, 64])
def test_w4a8_lora_bypass(cr, R):
    """A LoRA kept as a bf16 low-rank branch beside the W4A8 weight: la from
    the rotate+quantize call on the unrotated input, the up-projection fused
    into the GEMM epilogue; the output against the oracle's linear with the
    same branch (bf16 la)."""
    M, N, K = 333, 256, 3072
    say(f"w4a8 lora R={R}")
    xb = wl.activation(29, R, M, K)
    wb = wl.weight(29, R + 1, N, K)
    l1 = wl.weight(29, R + 2, N, R, std=0.05)
    l2 = wl.weight(29, R + 3, R, K, std=0.05)
    bias = wl.weight(29, R + 4, 1, N, std=0.5)[0]
    wp = ol.prepare_w4a8(wb)
    ref = ol.w4a8_linear(xb, wb, wprep=wp, l1_bits=l1, l2_bits=l2, bias_bits=bias)
    a, sa, _, la = cr.convrot_rotate_quantize(bf16_dev(xb), 256, cr.Q.SYM_INT8, cr.GRAN.ROW, lora_down=bf16_dev(l2))
    assert np.array_equal(host(a).view(np.uint8), ref["x"]["codes"].view(np.uint8))
    args = (a, sa, 1, dev(wp["tiles"].reshape(-1)), dev(wp["scales_tiles"].reshape(-1)),
            dev(wp["zeros_tiles"].reshape(-1)), M, N, K)
    kw = dict(w_sum=dev(wp["wsum16"]), lora_act=la, lora_up=bf16_dev(l1), bias=bf16_dev(bias))
    yf = cr.w4a8_gemm(*args, out_type=1, **kw)
    yb = cr.w4a8_gemm(*args, out_type=0, **kw)
    _check_out(yb, yf, ref["y"], f32_tol=W4A8_F32_TOL)
    plain = cr.w4a8_gemm(*args, out_type=1, w_sum=kw["w_sum"], bias=kw["bias"])
    assert rel_l2(host(yf) - host(plain), ref["y"] - ol.w4a8_linear(xb, wb, wprep=wp, bias_bits=bias)["y"]) <= 1e-2


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
    yf = cr.w4a4_gemm(a, sa, 0, w, sw, 0, M, N, K, lora_act=la_ref, lora_up=bf16_dev(l1), out_type=1)
    yb = cr.w4a4_gemm(a, sa, 0, w, sw, 0, M, N, K, lora_act=la_ref, lora_up=bf16_dev(l1), out_type=0)
    _check_out(yb, yf, ref["y"])
    # end to end with the GPU's la (its bf16 rounding may differ by one ulp): bf16 bar
    ye = cr.w4a4_gemm(a, sa, 0, w, sw, 0, M, N, K, lora_act=la, lora_up=bf16_dev(l1), out_type=0)
    assert rel_l2(bf16_to_f32(host(ye)), ref["y"]) <= 2e-3


def test_w4a8_float_outputs_match_fp16_weights(cr):
    """The float outputs equal, to float32 accumulation rounding, the product
    with each weight taken as fp16(s (q - z)): a reference built from the
    oracle's codes with that one rounding, evaluated in float64."""
    M, N, K = 200, 256, 1024
    say("w4a8 fp16-weight reference")
    xb = wl.activation(26, 7, M, K)
    wb = wl.weight(26, 8, N, K)
    wp = ol.prepare_w4a8(wb)
    xa = ol.rotate_quantize(xb, 256, "int8", "row")
    w16 = oq.dequant_asym(wp["values"], wp["scales"], wp["zeros"], 16).astype(np.float16).astype(np.float64)
    ref = (np.asarray(xa["values"], np.float64) @ w16.T) * np.asarray(xa["scales"], np.float64)[:, None]
    y = cr.w4a8_gemm(dev(xa["codes"]), dev(xa["scales"]), 1, dev(wp["tiles"].reshape(-1)),
                     dev(wp["scales_tiles"].reshape(-1)), dev(wp["zeros_tiles"].reshape(-1)), M, N, K,
                     out_type=1, w_sum=dev(wp["wsum16"]))
    # float32 accumulation of (1152 + a) w: partial sums about 40x the result
    assert rel_l2(host(y), ref) <= 1e-4


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
