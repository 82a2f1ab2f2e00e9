"""Full-size parity of the benchmarked path: the single MMDiT projection
(X bf16 [M, 3072] with M = 4096 and M = 32, W [3072, 3072]), run exactly as
bench.py runs it (GPU rotate+quantize into the tiled code layout, then the
W4A4 GEMM), against the oracle.

Bit-exact: every activation code and the per-tensor scale, every packed
weight byte, and the int32 results on sampled rows (all N columns). bf16
outputs: relative L2 <= 2e-3 against the oracle's float32 epilogue on the
same rows.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from oracle import quant as oq, linear as ol, gemm as og, pack as opack  # noqa: E402
from tests.gpu_helpers import bf16_dev, bf16_to_f32, bytes_of, dev, host, rel_l2, say  # noqa: E402


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_rotated_quantized_amd as m
    assert m.device_check() == 0
    return m


@pytest.fixture(scope="module")
def c2_weights(cr):
    N = K = 3072
    wb = wl.weight(2, 1, N, K)
    wp = ol.prepare_w4a4(wb)
    wc, ws, _, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR)
    assert np.array_equal(bytes_of(wc), wp["codes"].reshape(-1))
    assert host(ws)[0] == np.float32(wp["scales"]).reshape(-1)[0]
    packed, _, _, _ = cr.w4_pack_weights(wc, ws, N, K)
    assert np.array_equal(bytes_of(packed), wp["tiles"].reshape(-1))
    return wp, packed, ws


@pytest.mark.parametrize("M", [4096, 32])
def test_c2_full_pipeline(cr, c2_weights, M):
    N = K = 3072
    say(f"c2 full size M={M}")
    wp, packed, ws = c2_weights
    xb = wl.activation(2, 0 if M == 4096 else 2, M, K, n_outliers=15, outlier_scale=30.0)
    xa = ol.rotate_quantize(xb, 256, "int4", "tensor")
    codes, sa, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR,
                                                 layout=cr.LAYOUT.TILED)
    ref_tiled = opack.tile_pack_a(xa["codes"])
    got = bytes_of(codes).reshape(ref_tiled.shape)
    if M % 16:
        # rows past M in the last 16-row block are left unwritten: compare the valid rows only
        got = opack.tile_unpack_a(got, M)
        ref_tiled = xa["codes"]
    assert np.array_equal(got, ref_tiled)
    assert host(sa)[0] == np.float32(xa["scales"]).reshape(-1)[0]

    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(M, size=min(M, 192), replace=False))
    raw = host(cr.w4a4_gemm(codes, sa, 0, packed, ws, 0, M, N, K, out_type=cr.OUT.I32_RAW))
    ref_raw = og.int_gemm(xa["values"][rows], wp["values"])
    assert np.array_equal(raw[rows].astype(np.int64), ref_raw)
    y = bf16_to_f32(host(cr.w4a4_gemm(codes, sa, 0, packed, ws, 0, M, N, K)))
    ref_y = ol.epilogue_scalar(ref_raw, xa["scales"], "tensor", wp["scales"], "tensor")
    assert rel_l2(y[rows], ref_y) <= 2e-3


@pytest.mark.parametrize("M", [4096, 32])
def test_c2_full_pipeline_f6(cr, c2_weights, M):
    """The benchmarked path on the fp6 matrix cores: GPU rotate+quantize into
    fp6 fragments, weights packed to fp6 fragments, GEMM (256 x 192 blocks at
    M = 4096, the small-M kernel at 32)."""
    N = K = 3072
    say(f"c2 full size fp6 M={M}")
    wp, _, ws = c2_weights
    wc, _, _, _ = cr.convrot_rotate_quantize(bf16_dev(wl.weight(2, 1, N, K)), 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR)
    wf = cr.w4_pack_weights_f6(wc, N, K)
    assert np.array_equal(bytes_of(wf), opack.f6_pack(wp["values"]).reshape(-1))
    xb = wl.activation(2, 0 if M == 4096 else 2, M, K, n_outliers=15, outlier_scale=30.0)
    xa = ol.rotate_quantize(xb, 256, "int4", "tensor")
    codes, sa, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR,
                                                 layout=cr.LAYOUT.F6)
    assert np.array_equal(opack.f6_unpack(host(codes), M), xa["values"])
    assert host(sa)[0] == np.float32(xa["scales"]).reshape(-1)[0]
    rng = np.random.default_rng(4321)
    rows = np.sort(rng.choice(M, size=min(M, 192), replace=False))
    raw = host(cr.w4a4_gemm(codes, sa, 0, wf, ws, 0, M, N, K, out_type=cr.OUT.I32_RAW))
    ref_raw = og.int_gemm(xa["values"][rows], wp["values"])
    assert np.array_equal(raw[rows].astype(np.int64), ref_raw)
    y = bf16_to_f32(host(cr.w4a4_gemm(codes, sa, 0, wf, ws, 0, M, N, K)))
    ref_y = ol.epilogue_scalar(ref_raw, xa["scales"], "tensor", wp["scales"], "tensor")
    assert rel_l2(y[rows], ref_y) <= 2e-3


# ---------------------------------------------------------------------------
# the other workloads at full size (sampled outputs)
# ---------------------------------------------------------------------------

def _rows(M, n, seed):
    return np.sort(np.random.default_rng(seed).choice(M, size=min(M, n), replace=False))


def _cols(N, n, seed):
    return np.sort(np.random.default_rng(seed + 1).choice(N, size=min(N, n), replace=False))


def _lin(cfg, name):
    w = wl.CONFIGS[cfg]()
    return w, [l for l in w.linears if l.name == name][0]


def _chunks(M, step=1024):
    return [(r, min(M, r + step)) for r in range(0, M, step)]


def test_c3_w4a8_full(cr):
    """W4A8: X [8192, 3072] int8 per token (fp16-carried codes, the layout the
    GEMM runs on), W [12288, 3072] asym uint4 g16; every output row compared.
    The oracle's y = s_a sum_g s_w[n, g] P[m, n, g] is evaluated in row chunks
    as s_a (A @ W_hat^T) in float64, with W_hat = s_w (q - z) the oracle's
    exact dequantized weight (the same sum, grouped by k instead of by g)."""
    w, lin = _lin("c3", "mlp_up")
    M, N, K = lin.M, lin.N, lin.K
    say(f"c3 full {M}x{N}x{K}")
    xb, wb = wl.act_bits(w, lin.x_id), wl.weight_bits(w, lin)
    xa = ol.rotate_quantize(xb, 256, "int8", "row")
    wp = ol.prepare_w4a8(wb)
    a, sa, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, cr.Q.SYM_INT8, cr.GRAN.ROW, layout=cr.LAYOUT.F16)
    assert np.array_equal(host(a).astype(np.int64), xa["values"].astype(np.int64))
    assert np.array_equal(host(sa).view(np.uint32), np.asarray(xa["scales"], np.float32).view(np.uint32))
    wc, ws, wz, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, cr.Q.ASYM_UINT4, cr.GRAN.ROW_GROUP, 16)
    packed, pscales, pzeros, _ = cr.w4_pack_weights(wc, ws, N, K, cr.Q.ASYM_UINT4, cr.GRAN.ROW_GROUP, 16, zeros=wz)
    assert np.array_equal(bytes_of(packed), wp["tiles"].reshape(-1))
    assert np.array_equal(host(pscales).view(np.uint16).reshape(-1), wp["scales_tiles"].view(np.uint16).reshape(-1))
    assert np.array_equal(host(pzeros).reshape(-1), wp["zeros_tiles"].reshape(-1))
    raw = host(cr.w4a8_gemm(a, sa, cr.GRAN.ROW, packed, pscales, pzeros, M, N, K, out_type=cr.OUT.I32_RAW))
    yb = bf16_to_f32(host(cr.w4a8_gemm(a, sa, cr.GRAN.ROW, packed, pscales, pzeros, M, N, K)))
    yf = host(cr.w4a8_gemm(a, sa, cr.GRAN.ROW, packed, pscales, pzeros, M, N, K, out_type=cr.OUT.F32))
    zexp = np.repeat(wp["zeros"].astype(np.int64), 16, axis=1)
    d = (wp["values"].astype(np.int64) - zexp).astype(np.float64)
    w_hat = oq.dequant_asym(wp["values"], wp["scales"], wp["zeros"], 16).astype(np.float64)
    A = xa["values"].astype(np.float64)
    s_a = np.asarray(xa["scales"], np.float64)
    num = den = numf = 0.0
    for r0, r1 in _chunks(M):
        assert np.array_equal(raw[r0:r1].astype(np.int64), (A[r0:r1] @ d.T).astype(np.int64))
        ref = (s_a[r0:r1, None] * (A[r0:r1] @ w_hat.T)).astype(np.float32).astype(np.float64)
        num += float(np.sum((yb[r0:r1] - ref) ** 2))
        numf += float(np.sum((yf[r0:r1] - ref) ** 2))
        den += float(np.sum(ref ** 2))
    assert np.sqrt(num / den) <= 2e-3, np.sqrt(num / den)
    assert np.sqrt(numf / den) <= 1e-5, np.sqrt(numf / den)


def _int8_layer(cr, w, lin, rows_n=32):
    M, N, K = lin.M, lin.N, lin.K
    xb, wb = wl.act_bits(w, lin.x_id), wl.weight_bits(w, lin)
    xa = ol.rotate_quantize(xb, 256, "int8", "tensor")
    wq = ol.rotate_quantize(wb, 256, "int8", "tensor")
    ws_need = cr.convrot_rq_workspace_size(M, K, 256, cr.Q.SYM_INT8, cr.GRAN.TENSOR)
    a, sa, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, cr.Q.SYM_INT8, cr.GRAN.TENSOR)
    assert ws_need > 0
    assert np.array_equal(host(a), xa["codes"])
    assert host(sa)[0] == np.float32(xa["scales"]).reshape(-1)[0]
    wc, wsc, _, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, cr.Q.SYM_INT8, cr.GRAN.TENSOR)
    assert np.array_equal(host(wc), wq["codes"])
    rows = _rows(M, rows_n, 41)
    raw = host(cr.int8_tensorwise_gemm(a, sa, wc, wsc, M, N, K, out_type=cr.OUT.I32_RAW))
    ref_raw = og.int_gemm(xa["values"][rows], wq["values"])
    assert np.array_equal(raw[rows].astype(np.int64), ref_raw)
    y = bf16_to_f32(host(cr.int8_tensorwise_gemm(a, sa, wc, wsc, M, N, K)))
    ref_y = ol.epilogue_scalar(ref_raw, xa["scales"], "tensor", wq["scales"], "tensor")
    assert rel_l2(y[rows], ref_y) <= 2e-3


def _w4a4_layer(cr, w, lin, rows_n=32):
    M, N, K = lin.M, lin.N, lin.K
    xb, wb = wl.act_bits(w, lin.x_id), wl.weight_bits(w, lin)
    xa = ol.rotate_quantize(xb, 256, "int4", "tensor")
    wp = ol.prepare_w4a4(wb)
    codes, sa, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR,
                                                 layout=cr.LAYOUT.TILED)
    assert np.array_equal(opack.tile_unpack_a(bytes_of(codes).reshape((M + 15) // 16, K // 64, 512), M),
                          xa["codes"])
    assert host(sa)[0] == np.float32(xa["scales"]).reshape(-1)[0]
    wc, ws, _, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR)
    packed, _, _, _ = cr.w4_pack_weights(wc, ws, N, K)
    assert np.array_equal(bytes_of(packed), wp["tiles"].reshape(-1))
    rows = _rows(M, rows_n, 51)
    raw = host(cr.w4a4_gemm(codes, sa, 0, packed, ws, 0, M, N, K, out_type=cr.OUT.I32_RAW))
    ref_raw = og.int_gemm(xa["values"][rows], wp["values"])
    assert np.array_equal(raw[rows].astype(np.int64), ref_raw)
    y = bf16_to_f32(host(cr.w4a4_gemm(codes, sa, 0, packed, ws, 0, M, N, K)))
    ref_y = ol.epilogue_scalar(ref_raw, xa["scales"], "tensor", wp["scales"], "tensor")
    assert rel_l2(y[rows], ref_y) <= 2e-3


@pytest.mark.parametrize("name", ["img_v", "img_mod"])
def test_c4_int8_layers_full(cr, name):
    w, lin = _lin("c4", name)
    say(f"c4 full {name} {lin.M}x{lin.N}x{lin.K}")
    _int8_layer(cr, w, lin)


@pytest.mark.parametrize("name", ["img_mlp_up", "img_mlp_down", "txt_q"])
def test_c4_w4a4_layers_full(cr, name):
    w, lin = _lin("c4", name)
    say(f"c4 full {name} {lin.M}x{lin.N}x{lin.K}")
    _w4a4_layer(cr, w, lin)


def _w4a4_layer_f6(cr, w, lin, rows_n=32):
    M, N, K = lin.M, lin.N, lin.K
    xb, wb = wl.act_bits(w, lin.x_id), wl.weight_bits(w, lin)
    xa = ol.rotate_quantize(xb, 256, "int4", "tensor")
    wq = ol.rotate_quantize(wb, 256, "int4", "tensor")
    codes, sa, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR,
                                                 layout=cr.LAYOUT.F6)
    assert np.array_equal(opack.f6_unpack(host(codes), M), xa["values"])
    wf, ws, _, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR,
                                              layout=cr.LAYOUT.F6)
    assert np.array_equal(bytes_of(wf), opack.f6_pack(wq["values"]).reshape(-1))
    rows = _rows(M, rows_n, 53)
    raw = host(cr.w4a4_gemm(codes, sa, 0, wf, ws, 0, M, N, K, out_type=cr.OUT.I32_RAW))
    ref_raw = og.int_gemm(xa["values"][rows], wq["values"])
    assert np.array_equal(raw[rows].astype(np.int64), ref_raw)
    y = bf16_to_f32(host(cr.w4a4_gemm(codes, sa, 0, wf, ws, 0, M, N, K)))
    ref_y = ol.epilogue_scalar(ref_raw, xa["scales"], "tensor", wq["scales"], "tensor")
    assert rel_l2(y[rows], ref_y) <= 2e-3


@pytest.mark.parametrize("name", ["img_mlp_up", "img_mlp_down", "txt_q"])
def test_c4_w4a4_layers_full_f6(cr, name):
    w, lin = _lin("c4", name)
    say(f"c4 full fp6 {name} {lin.M}x{lin.N}x{lin.K}")
    _w4a4_layer_f6(cr, w, lin)


@pytest.mark.parametrize("name", ["qkv", "mlp_down"])
def test_c5_lowrank_g64_full(cr, name):
    """Low-rank corrected W4A4 with 64-group scales (no rotation): rank-32
    branch with the down-projection fused into the quantizer and the
    up-projection into the GEMM epilogue; MLP down takes the unsigned
    post-GELU path with the 0.171875 shift."""
    w, lin = _lin("c5", name)
    M, N, K = lin.M, lin.N, lin.K
    shift = lin.unsigned_shift
    uns = shift != 0.0
    say(f"c5 full {name} {M}x{N}x{K}")
    xb = wl.act_bits(w, lin.x_id)
    l1, l2, r = wl.lowrank_bits(w, lin)
    xa = ol.rotate_quantize(xb, 0, "uint4_shift" if uns else "int4", "row_group", 64, shift)
    la_ref = ol.lora_down(xb, l2)
    wp = ol.prepare_w4a4(r, 0, "row_group", 64)
    qt = cr.Q.UNSIGNED_INT4_SHIFT if uns else cr.Q.SYM_INT4
    codes, sa, _, la = cr.convrot_rotate_quantize(bf16_dev(xb), 0, qt, cr.GRAN.ROW_GROUP, 64, shift=shift,
                                                  lora_down=bf16_dev(l2), layout=cr.LAYOUT.TILED)
    assert np.array_equal(opack.tile_unpack_a(bytes_of(codes).reshape((M + 15) // 16, K // 64, 512), M),
                          xa["codes"])
    assert np.array_equal(host(sa).view(np.uint32), np.asarray(xa["scales"], np.float32).view(np.uint32))
    # low-rank activations: bf16 of a float32 sum taken in another order -> within one bf16 ulp
    la_ref32 = ol.lora_down(xb, l2, act_f32=True).astype(np.float64)
    mag = np.abs(wl.f32_from_bf16_bits(xb)).astype(np.float64) @ np.abs(wl.f32_from_bf16_bits(l2)).astype(np.float64).T
    got_la = wl.f32_from_bf16_bits(host(la)).astype(np.float64)
    assert np.all(np.abs(got_la - la_ref32) <= np.abs(la_ref32) * 2.0 ** -7 + mag * 2 ** -20 + 1e-30)
    wc, ws, _, _ = cr.convrot_rotate_quantize(bf16_dev(r), 0, cr.Q.SYM_INT4, cr.GRAN.ROW_GROUP, 64)
    packed, pscales, _, wsum = cr.w4_pack_weights(wc, ws, N, K, cr.Q.SYM_INT4, cr.GRAN.ROW_GROUP, 64,
                                                  want_wsum=True)
    assert np.array_equal(bytes_of(packed), wp["tiles"].reshape(-1))
    assert np.array_equal(host(pscales).reshape(-1), wp["scales_tiles"].reshape(-1))
    kw = dict(a_unsigned=uns, a_shift=shift, w_sum=wsum)
    rows, cols = _rows(M, 16, 61), _cols(N, 1024, 61)
    raw = host(cr.w4a4_gemm(codes, sa, 2, packed, pscales, 2, M, N, K, out_type=cr.OUT.I32_RAW, **kw))
    ref_raw = og.int_gemm(xa["values"][rows], wp["values"])
    assert np.array_equal(raw[rows].astype(np.int64), ref_raw)
    y = bf16_to_f32(host(cr.w4a4_gemm(codes, sa, 2, packed, pscales, 2, M, N, K, lora_act=la,
                                      lora_up=bf16_dev(l1), **kw)))
    P = og.group_partials(xa["values"][rows], wp["values"][cols], 64)
    ref_y = ol.epilogue_g64(P, np.asarray(xa["scales"])[rows], np.asarray(wp["scales"])[cols], shift,
                            np.asarray(wp["wsum"])[cols], la_ref[rows], l1[cols])
    assert rel_l2(y[np.ix_(rows, cols)], ref_y) <= 2e-3


@pytest.mark.parametrize("name", ["qkv", "mlp_down"])
def test_c5_lowrank_g64_full_f6(cr, name):
    """The same layers on the fp6 matrix cores: codes (unsigned ones as u/2)
    in fp6 fragments from the quantizer, weights through
    w4_pack_weights_f6, 64-group scales and column sums from w4_pack_weights."""
    w, lin = _lin("c5", name)
    M, N, K = lin.M, lin.N, lin.K
    shift = lin.unsigned_shift
    uns = shift != 0.0
    say(f"c5 full fp6 {name} {M}x{N}x{K}")
    xb = wl.act_bits(w, lin.x_id)
    l1, l2, r = wl.lowrank_bits(w, lin)
    xa = ol.rotate_quantize(xb, 0, "uint4_shift" if uns else "int4", "row_group", 64, shift)
    la_ref = ol.lora_down(xb, l2)
    wp = ol.prepare_w4a4(r, 0, "row_group", 64)
    qt = cr.Q.UNSIGNED_INT4_SHIFT if uns else cr.Q.SYM_INT4
    codes, sa, _, la = cr.convrot_rotate_quantize(bf16_dev(xb), 0, qt, cr.GRAN.ROW_GROUP, 64, shift=shift,
                                                  lora_down=bf16_dev(l2), layout=cr.LAYOUT.F6)
    assert np.array_equal(opack.f6_unpack(host(codes), M) * (2 if uns else 1), xa["values"])
    assert np.array_equal(host(sa).view(np.uint32), np.asarray(xa["scales"], np.float32).view(np.uint32))
    wc, ws, _, _ = cr.convrot_rotate_quantize(bf16_dev(r), 0, cr.Q.SYM_INT4, cr.GRAN.ROW_GROUP, 64)
    _, pscales, _, wsum = cr.w4_pack_weights(wc, ws, N, K, cr.Q.SYM_INT4, cr.GRAN.ROW_GROUP, 64, want_wsum=True)
    wf = cr.w4_pack_weights_f6(wc, N, K)
    assert np.array_equal(bytes_of(wf), opack.f6_pack(wp["values"]).reshape(-1))
    kw = dict(a_unsigned=uns, a_shift=shift, w_sum=wsum)
    rows, cols = _rows(M, 16, 62), _cols(N, 1024, 62)
    raw = host(cr.w4a4_gemm(codes, sa, 2, wf, pscales, 2, M, N, K, out_type=cr.OUT.I32_RAW, **kw))
    assert np.array_equal(raw[rows].astype(np.int64), og.int_gemm(xa["values"][rows], wp["values"]))
    y = bf16_to_f32(host(cr.w4a4_gemm(codes, sa, 2, wf, pscales, 2, M, N, K, lora_act=la,
                                      lora_up=bf16_dev(l1), **kw)))
    P = og.group_partials(xa["values"][rows], wp["values"][cols], 64)
    ref_y = ol.epilogue_g64(P, np.asarray(xa["scales"])[rows], np.asarray(wp["scales"])[cols], shift,
                            np.asarray(wp["wsum"])[cols], la_ref[rows], l1[cols])
    assert rel_l2(y[np.ix_(rows, cols)], ref_y) <= 2e-3
