"""GPU parity of the fp6 matrix-core W4A4 path (CR_LAYOUT_F6) against the
CPU oracle.

The fp6 path carries the same integer codes as the int8-core path, as E2M3
values in 32 x 64 fragments (oracle.pack.f6_pack defines the layout). Bars:
codes and packed bytes bit-exact (decoded to integers for the rows the
library writes); int32 results bit-exact; float32 output within 1e-5 and bf16
within 2e-3 relative L2 of the oracle's float32 epilogue.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from oracle import linear as ol, pack as opack  # noqa: E402
from tests.gpu_helpers import bf16_dev, bytes_of, dev, host, rel_l2, bf16_to_f32, say  # noqa: E402

GR = {"tensor": 0, "row": 1, "row_group": 2}
F6 = 3


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_rotated_quantized_amd as m
    assert m.device_check() == 0
    return m


@pytest.mark.parametrize("shape", [(128, 128), (256, 512), (384, 3072), (128, 12288)])
def test_pack_weights_f6_bytes(cr, shape):
    N, K = shape
    say(f"f6 pack {shape}")
    rng = np.random.default_rng(N + K)
    q = rng.integers(-7, 8, size=(N, K))
    q[0, :8] = [7, -7, 0, 1, -1, 3, -5, 6]
    packed = cr.w4_pack_weights_f6(dev(opack.pack_int4(q)), N, K)
    assert cr.w4_packed_f6_bytes(N, K) == packed.numel()
    assert np.array_equal(bytes_of(packed), opack.f6_pack(q).reshape(-1))


RQ_SHAPES = [(64, 512), (37, 3072), (300, 768), (5, 256), (129, 12288)]


@pytest.mark.parametrize("rot", [256, 16, 64, 1024])
@pytest.mark.parametrize("gran", ["tensor", "row", "row_group"])
@pytest.mark.parametrize("shape", RQ_SHAPES)
def test_rotate_quantize_f6(cr, rot, gran, shape):
    rows, K = shape
    if K % rot:
        pytest.skip("K not a multiple of the rotation")
    say(f"rq f6 rot {rot} {gran} {shape}")
    xb = wl.activation(31, rows * 5 + K + rot, rows, K, n_outliers=max(1, K // 200), outlier_scale=25.0)
    qg = 64 if gran == "row_group" else 0
    ref = ol.rotate_quantize(xb, rot, "int4", gran, qg or None)
    codes, scales, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), rot, 0, GR[gran], qg, layout=F6)
    assert tuple(codes.shape) == ((rows + 31) // 32, K // 64, 1536)
    assert np.array_equal(opack.f6_unpack(host(codes), rows), ref["values"]), "fp6 codes differ"
    # the written rows' bytes are the oracle's encoding (+0 for zero codes)
    want = opack.f6_pack(ref["values"])
    got = host(codes)
    full = rows // 32
    assert np.array_equal(got[:full], want[:full])
    assert np.array_equal(host(scales).reshape(-1).view(np.uint32),
                          np.asarray(ref["scales"], np.float32).reshape(-1).view(np.uint32)), "scales differ"


@pytest.mark.parametrize("rot", [256, 1024])
def test_rotate_quantize_dual_f6(cr, rot):
    rows, K = 300, 3072
    say(f"rq dual f6 rot {rot}")
    xb = wl.activation(33, rot, rows, K, n_outliers=10, outlier_scale=25.0)
    r4 = ol.rotate_quantize(xb, rot, "int4", "tensor")
    r8 = ol.rotate_quantize(xb, rot, "int8", "tensor")
    c4, s4, c8, s8 = cr.convrot_rotate_quantize_dual(bf16_dev(xb), rot, layout4=F6)
    assert np.array_equal(opack.f6_unpack(host(c4), rows), r4["values"])
    assert np.array_equal(host(c8), r8["codes"])
    assert host(s4)[0] == np.float32(r4["scales"]).reshape(-1)[0]
    assert host(s8)[0] == np.float32(r8["scales"]).reshape(-1)[0]


F6_CASES = [
    # M, N, K, a_gran, w_gran
    (1, 256, 512, "tensor", "tensor"),        # small-M kernel
    (17, 384, 3072, "tensor", "row"),
    (33, 128, 1024, "row", "row"),
    (64, 256, 512, "row", "tensor"),
    (65, 256, 512, "tensor", "tensor"),       # tiled kernel from here on (64 x 64 blocks while 128 x 128
                                              # ones would number fewer than 256); one ragged 32-row block
    (77, 768, 256, "row", "tensor"),          # two 128-deep stages
    (200, 384, 3072, "tensor", "tensor"),
    (256, 384, 3072, "row", "row"),
    (300, 512, 768, "tensor", "tensor"),
    (129, 128, 12288, "tensor", "tensor"),
    (2100, 2048, 256, "row", "tensor"),       # 128 x 128 blocks (>= 256 of them, N not a multiple of 192)
    (1300, 3072, 512, "tensor", "row"),       # 256 x 192 blocks would be too few: 128 x 128
]


@pytest.mark.parametrize("case", F6_CASES)
def test_w4a4_f6_gemm(cr, case):
    M, N, K, ag, wg = case
    say(f"w4a4 f6 {case}")
    xb = wl.activation(41, M + N + K, M, K, n_outliers=3, outlier_scale=20.0)
    wb = wl.weight(41, 7 + M + N + K, N, K)
    bias = wl.weight(41, 9, 1, N, std=0.5)[0]
    wp = ol.prepare_w4a4(wb, 256, wg)
    ref = ol.w4a4_linear(xb, wb, 256, ag, wg, wprep=wp)
    ref_b = ol.w4a4_linear(xb, wb, 256, ag, wg, bias_bits=bias, wprep=wp)
    a = dev(opack.f6_pack(ref["x"]["values"]))
    w = dev(opack.f6_pack(wp["values"]))
    sa = dev(np.asarray(ref["x"]["scales"], np.float32).reshape(-1))
    sw = dev(np.asarray(wp["scales"], np.float32).reshape(-1))
    raw = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=2)
    assert np.array_equal(host(raw).astype(np.int64), ref["raw"])
    yf = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=1)
    assert rel_l2(host(yf), ref["y"]) <= 1e-5
    yb = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, out_type=0)
    assert rel_l2(bf16_to_f32(host(yb)), ref["y"]) <= 2e-3
    ybias = cr.w4a4_gemm(a, sa, GR[ag], w, sw, GR[wg], M, N, K, bias=bf16_dev(bias), out_type=1)
    assert rel_l2(host(ybias), ref_b["y"]) <= 1e-5
    # the same float32 epilogue as the int8-core path: identical outputs
    at = dev(opack.tile_pack_a(ref["x"]["codes"]))
    wt = dev(wp["tiles"].reshape(-1))
    yf8 = cr.w4a4_gemm(at, sa, GR[ag], wt, sw, GR[wg], M, N, K, out_type=1)
    assert np.array_equal(host(yf).view(np.uint32), host(yf8).view(np.uint32))
    # fp6 codes against the 4-bit tile-packed weights (expanded by the call in
    # its workspace): the same results bit for bit
    assert cr.w4a4_gemm_workspace_size(N, K, F6, 1) == (N // 32) * (K // 64) * 1536
    raw_t = cr.w4a4_gemm(a, sa, GR[ag], wt, sw, GR[wg], M, N, K, out_type=2)
    assert np.array_equal(host(raw_t).astype(np.int64), ref["raw"])
    ws = torch.full((cr.w4a4_gemm_workspace_size(N, K, F6, 1),), 0x55, dtype=torch.uint8, device="cuda")
    yb_t = cr.w4a4_gemm(a, sa, GR[ag], wt, sw, GR[wg], M, N, K, out_type=0, workspace=ws)
    assert np.array_equal(host(yb_t), host(yb))
    assert np.array_equal(bytes_of(ws), host(w).reshape(-1))      # the expansion is the fp6 weight image
    # the expansion as a call of its own: the same bytes, and the GEMM on them
    f6w = cr.w4_expand_weights_f6(wt, N, K)
    assert np.array_equal(bytes_of(f6w), host(w).reshape(-1))
    yb_e = cr.w4a4_gemm(a, sa, GR[ag], f6w, sw, GR[wg], M, N, K, out_type=0)
    assert np.array_equal(host(yb_e), host(yb))


@pytest.mark.parametrize("M", [7950, 6100])
def test_w4a4_f6_wide_blocks(cr, M):
    """256 x 256 blocks (wide outputs, at least three rounds of tiles on 256
    CUs: 7950 x 8192 gives 1024 tiles, 6100 x 8192 exactly 768, the last row
    block ragged in both): raw sums equal the exact integer product, float32
    outputs its scaled value."""
    N, K = 8192, 128
    say(f"w4a4 f6 256x256 blocks M={M}")
    rng = np.random.default_rng(11)
    qa = rng.integers(-7, 8, size=(M, K))
    qw = rng.integers(-7, 8, size=(N, K))
    ref = qa.astype(np.float64) @ qw.astype(np.float64).T          # exact: |sum| <= 128 * 49
    a, w = dev(opack.f6_pack(qa)), dev(opack.f6_pack(qw))
    sa, sw = dev(np.array([0.0123], np.float32)), dev(np.array([0.0456], np.float32))
    raw = host(cr.w4a4_gemm(a, sa, 0, w, sw, 0, M, N, K, out_type=2))
    assert np.array_equal(raw.astype(np.float64), ref)
    yf = host(cr.w4a4_gemm(a, sa, 0, w, sw, 0, M, N, K, out_type=1))
    s = float(np.float32(0.0123)) * float(np.float32(0.0456))
    assert rel_l2(yf, ref * s) <= 1e-6


@pytest.mark.parametrize("shape", [(7950, 8192, 128), (6100, 8192, 128), (4000, 3072, 256)],
                         ids=["256x256", "256x256_three_rounds", "256x192"])
def test_w4a4_f6_large_blocks_row_scales_bias(cr, shape):
    """The large blocks' epilogues with per-row scales on both sides and a
    bias: 256 x 256 blocks (7950 x 8192 and 6100 x 8192, ragged last row
    blocks, four and three rounds of tiles) and 256 x 192
    blocks (4000 x 3072: 256 tiles, ragged); bf16 rows through LDS within
    2e-3, float32 within 1e-5 of y = s_a[m] s_w[n] sum + b[n] in float64."""
    M, N, K = shape
    say(f"w4a4 f6 large blocks row scales bias {shape}")
    rng = np.random.default_rng(13)
    qa = rng.integers(-7, 8, size=(M, K))
    qw = rng.integers(-7, 8, size=(N, K))
    raw = qa.astype(np.float64) @ qw.astype(np.float64).T
    sa = (rng.random(M) * 0.02 + 0.001).astype(np.float32)
    sw = (rng.random(N) * 0.05 + 0.001).astype(np.float32)
    b = wl.bf16_bits_from_f32((rng.standard_normal(N) * 0.5).astype(np.float32))
    ref = raw * sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] + \
        wl.f32_from_bf16_bits(b).astype(np.float64)[None, :]
    a, w = dev(opack.f6_pack(qa)), dev(opack.f6_pack(qw))
    yf = host(cr.w4a4_gemm(a, dev(sa), 1, w, dev(sw), 1, M, N, K, bias=bf16_dev(b), out_type=1))
    assert rel_l2(yf, ref) <= 1e-5
    yb = bf16_to_f32(host(cr.w4a4_gemm(a, dev(sa), 1, w, dev(sw), 1, M, N, K, bias=bf16_dev(b), out_type=0)))
    assert rel_l2(yb, ref) <= 2e-3


def test_w4a4_f6_ldc_padding(cr):
    M, N, K, ldc = 150, 256, 512, 264
    say("w4a4 f6 ldc")
    rng = np.random.default_rng(5)
    qa = rng.integers(-7, 8, size=(M, K))
    qw = rng.integers(-7, 8, size=(N, K))
    out = torch.full((M, ldc), -1, dtype=torch.int32, device="cuda")
    sa = dev(np.ones(1, np.float32))
    cr.w4a4_gemm(dev(opack.f6_pack(qa)), sa, 0, dev(opack.f6_pack(qw)), sa, 0, M, N, K, out_type=2,
                 out=out[:, :N].as_strided((M, N), (ldc, 1)))
    o = host(out)
    assert np.array_equal(o[:, :N].astype(np.int64), qa @ qw.T)
    assert np.all(o[:, N:] == -1)


def test_w4a4_f6_layer_on_gpu(cr):
    """Whole layer on the GPU path: both operands rotated and quantized by
    convrot_rotate_quantize into fp6 fragments (weights also through
    w4_pack_weights_f6 from natural codes), GEMM on the fp6 cores."""
    M, N, K = 200, 384, 3072
    say("w4a4 f6 layer")
    xb = wl.activation(43, 1, M, K, n_outliers=3, outlier_scale=20.0)
    wb = wl.weight(43, 2, N, K)
    ref = ol.w4a4_linear(xb, wb, 256, "tensor", "row")
    a, sa, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, 0, 0, layout=F6)
    wf, ws, _, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, 0, 1, layout=F6)
    wn, _, _, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, 0, 1)
    wp = cr.w4_pack_weights_f6(wn, N, K)
    assert np.array_equal(bytes_of(wp), bytes_of(wf))
    raw = cr.w4a4_gemm(a, sa, 0, wf, ws, 1, M, N, K, out_type=2)
    assert np.array_equal(host(raw).astype(np.int64), ref["raw"])
    yb = cr.w4a4_gemm(a, sa, 0, wf, ws, 1, M, N, K, out_type=0)
    assert rel_l2(bf16_to_f32(host(yb)), ref["y"]) <= 2e-3
    # the stored format: 4-bit tile-packed weights (w4_pack_weights), expanded per call
    wt, _, _, _ = cr.w4_pack_weights(wn, ws, N, K, 0, 1)
    assert np.array_equal(bytes_of(wt), ref["w"]["tiles"].reshape(-1))
    assert np.array_equal(host(cr.w4a4_gemm(a, sa, 0, wt, ws, 1, M, N, K, out_type=2)), host(raw))
    assert np.array_equal(host(cr.w4a4_gemm(a, sa, 0, wt, ws, 1, M, N, K, out_type=0)), host(yb))


def test_f6_rejects_unsupported(cr):
    M, N, K = 64, 128, 256
    a = torch.zeros(((M + 31) // 32, K // 64, 1536), dtype=torch.uint8, device="cuda")
    w = torch.zeros((N // 32, K // 64, 1536), dtype=torch.uint8, device="cuda")
    s = torch.ones(M * (K // 64), dtype=torch.float32, device="cuda")
    lr = torch.zeros((M, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cr.ConvRotError, match="format not available"):
        cr.w4a4_gemm(a, s, 2, w, s, 0, M, N, K)              # 64-group scales on one side only
    with pytest.raises(cr.ConvRotError, match="format not available"):
        cr.w4a4_gemm(a, s, 0, w, s, 0, M, N, K, a_unsigned=True, a_shift=0.171875, w_sum=s)
    with pytest.raises(cr.ConvRotError, match="format not available"):
        cr.w4a4_gemm(a, s, 1, w, s, 1, M, N, K, lora_act=lr,
                     lora_up=torch.zeros((N // 128, 32, 128), dtype=torch.bfloat16, device="cuda"))
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cr.ConvRotError, match="format not available"):
        cr.convrot_rotate_quantize(x, 256, 1, 0, 0, layout=F6)  # INT8 codes


# ---------------------------------------------------------------------------
# 64-group scales without rotation (the SVDQuant-style low-rank corrected
# format): quantizer into fp6 fragments, signed or unsigned shifted codes, the
# low-rank down-projection fused; GEMM with per-group scaling on the fp6 cores.
# ---------------------------------------------------------------------------
PLAIN_SHAPES = [(64, 512), (37, 3072), (300, 768), (5, 256), (129, 4096)]


@pytest.mark.parametrize("uns", [False, True])
@pytest.mark.parametrize("rank", [0, 32, 64])
@pytest.mark.parametrize("shape", PLAIN_SHAPES)
def test_quantize_g64_f6(cr, uns, rank, shape):
    rows, K = shape
    say(f"rq g64 f6 uns {uns} rank {rank} {shape}")
    shift = 0.171875 if uns else 0.0
    xb = wl.gelu_activation(37, rows + K + rank, rows, K) if uns else wl.activation(37, rows + K + rank, rows, K)
    ref = ol.rotate_quantize(xb, 0, "uint4_shift" if uns else "int4", "row_group", 64, shift)
    qt = cr.Q.UNSIGNED_INT4_SHIFT if uns else cr.Q.SYM_INT4
    l2 = wl.weight(37, 3, rank, K) if rank else None
    kw = dict(shift=shift, lora_down=None if l2 is None else bf16_dev(l2))
    codes, scales, _, la = cr.convrot_rotate_quantize(bf16_dev(xb), 0, qt, cr.GRAN.ROW_GROUP, 64, layout=F6, **kw)
    assert tuple(codes.shape) == ((rows + 31) // 32, K // 64, 1536)
    vals = opack.f6_unpack(host(codes), rows) * (2 if uns else 1)
    assert np.array_equal(vals, ref["values"]), "fp6 codes differ"
    full = rows // 32
    assert np.array_equal(host(codes)[:full], opack.f6_pack(ref["values"], unsigned=uns)[:full])
    assert np.array_equal(host(scales).reshape(-1).view(np.uint32),
                          np.asarray(ref["scales"], np.float32).reshape(-1).view(np.uint32)), "scales differ"
    if rank:   # the same fused down-projection as the natural layout's: identical bits
        _, _, _, la_n = cr.convrot_rotate_quantize(bf16_dev(xb), 0, qt, cr.GRAN.ROW_GROUP, 64, **kw)
        assert np.array_equal(host(la), host(la_n))


F6_G64_CASES = [
    # M, N, K, unsigned, lora(None|bf16|f32), rank, bias
    (16, 256, 512, False, None, 0, False),
    (40, 384, 1024, True, None, 0, False),
    (200, 256, 3072, False, "bf16", 32, True),
    (130, 384, 1024, True, "bf16", 32, False),
    (64, 256, 512, True, "f32", 32, True),
    (257, 128, 768, False, "f32", 64, False),
    (300, 512, 1024, True, "bf16", 64, True),
    (100, 384, 128, False, None, 0, True),      # a single 128-deep stage
    (1, 128, 256, True, "bf16", 32, True),
    (1000, 384, 1152, True, "bf16", 32, True),   # ragged 128-row block, nine 128-deep stages
    (515, 256, 640, False, "f32", 64, False),    # five stages, a 3-row tail
]


@pytest.mark.parametrize("case", F6_G64_CASES)
def test_w4a4_f6_group64(cr, case):
    M, N, K, uns, lora, rank, use_bias = case
    say(f"w4a4 f6 g64 {case}")
    shift = 0.171875 if uns else 0.0
    xb = wl.gelu_activation(29, M + K, M, K) if uns else wl.activation(29, M + K, M, K)
    wb = wl.weight(29, N + K, N, K)
    l1 = l2 = None
    if lora:
        l1, l2, wb = wl.lowrank_split(wb, rank)
    bias = wl.weight(29, 5, 1, N, std=0.5)[0] if use_bias else None
    wp = ol.prepare_w4a4(wb, 0, "row_group", 64)
    ref = ol.w4a4_linear(xb, wb, 0, "row_group", "row_group", 64, shift, l1, l2,
                         act_f32=(lora == "f32"), bias_bits=bias, wprep=wp)
    a = dev(opack.f6_pack(ref["x"]["values"], unsigned=uns))
    sa = dev(np.asarray(ref["x"]["scales"], np.float32))
    w = dev(opack.f6_pack(wp["values"]))
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
    yf = cr.w4a4_gemm(a, sa, 2, w, sw, 2, M, N, K, out_type=1, **kw)
    assert rel_l2(host(yf), ref["y"]) <= 1e-5
    yb = cr.w4a4_gemm(a, sa, 2, w, sw, 2, M, N, K, out_type=0, **kw)
    assert rel_l2(bf16_to_f32(host(yb)), ref["y"]) <= 2e-3
    # the bf16 output is the float32 one rounded to nearest even
    assert np.array_equal(host(yb), host(yf.to(torch.bfloat16)))
    # the same against the 4-bit tile-packed weights, expanded by the call
    wt = dev(wp["tiles"].reshape(-1))
    assert np.array_equal(host(cr.w4a4_gemm(a, sa, 2, wt, sw, 2, M, N, K, out_type=2, **kw)), host(raw))
    yf_t = cr.w4a4_gemm(a, sa, 2, wt, sw, 2, M, N, K, out_type=1, **kw)
    assert np.array_equal(host(yf_t).view(np.uint32), host(yf).view(np.uint32))


def test_w4a4_f6_group64_ldc_padding(cr):
    M, N, K, ldc = 150, 256, 512, 264
    say("w4a4 f6 g64 ldc")
    rng = np.random.default_rng(6)
    qa = rng.integers(-7, 8, size=(M, K))
    qw = rng.integers(-7, 8, size=(N, K))
    sa = dev(np.ones(M * (K // 64), np.float32))
    sw = dev(np.ones(N * (K // 64), np.float32))
    out = torch.full((M, ldc), 7.0, dtype=torch.float32, device="cuda")
    cr.w4a4_gemm(dev(opack.f6_pack(qa)), sa, 2, dev(opack.f6_pack(qw)), sw, 2, M, N, K, out_type=1,
                 out=out[:, :N].as_strided((M, N), (ldc, 1)))
    o = host(out)
    assert np.array_equal(o[:, :N].astype(np.int64), qa @ qw.T)
    assert np.all(o[:, N:] == 7.0)
