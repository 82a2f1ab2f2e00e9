"""GPU parity of convrot_rotate_quantize and w4_pack_weights against the
CPU oracle: codes, scales, zero points and packed bytes must be bit-exact;
the LoRA-down activations (float32 matrix-core accumulation in another order)
agree to a float32-sum tolerance before and one bf16 ulp after rounding."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from oracle import hadamard as oh, linear as ol, pack as opack  # noqa: E402
from tests.gpu_helpers import bf16_dev, dev, host, bytes_of, say  # noqa: E402


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_rotated_quantized_amd as m
    assert m.device_check() == 0, "device is not gfx950"
    return m


QT = {"int4": 0, "int8": 1}
GR = {"tensor": 0, "row": 1, "row_group": 2}

ROT_SHAPES = [(64, 512), (37, 3072), (300, 768), (5, 256), (129, 12288)]


@pytest.mark.parametrize("qt", ["int4", "int8"])
@pytest.mark.parametrize("gran", ["tensor", "row", "row_group"])
@pytest.mark.parametrize("shape", ROT_SHAPES)
def test_rotate_quantize_sym(cr, qt, gran, shape):
    rows, K = shape
    say(f"rq sym {qt} {gran} {shape}")
    xb = wl.activation(11, rows * 7 + K, rows, K, n_outliers=max(1, K // 200), outlier_scale=25.0)
    qg = 64 if gran == "row_group" else 0
    ref = ol.rotate_quantize(xb, 256, qt, gran, qg or None)
    codes, scales, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, QT[qt], GR[gran], qg)
    assert np.array_equal(host(codes).reshape(ref["codes"].shape).view(np.uint8),
                          ref["codes"].view(np.uint8)), "codes differ"
    assert np.array_equal(host(scales).reshape(-1).view(np.uint32),
                          np.asarray(ref["scales"], np.float32).reshape(-1).view(np.uint32)), "scales differ"
    if qt == "int4":
        tcodes, tscales, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, 0, GR[gran], qg, layout=1)
        assert np.array_equal(opack.tile_unpack_a(host(tcodes), rows), ref["codes"]), "tiled codes differ"
        assert np.array_equal(host(tscales).reshape(-1), np.asarray(ref["scales"]).reshape(-1))
    else:
        # the same codes as fp16 values (every integer of the range is exact;
        # zero as +0): bit patterns equal the oracle's codes converted to fp16
        hcodes, hscales, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, 1, GR[gran], qg, layout=4)
        want = ref["values"].astype(np.float16).view(np.uint16)
        assert np.array_equal(host(hcodes).view(np.uint16), want), "fp16 codes differ"
        assert np.array_equal(host(hscales).reshape(-1).view(np.uint32),
                              np.asarray(ref["scales"], np.float32).reshape(-1).view(np.uint32))


# The other ConvRot group sizes of the W4A4 recipe: 16 and 64 lie inside one
# 256-element chunk of a lane segment, 1024 spans four chunks of one segment.
GROUP_SHAPES = [(64, 1024), (37, 3072), (300, 2048), (129, 12288)]


@pytest.mark.parametrize("rot", [16, 64, 1024])
@pytest.mark.parametrize("qt", ["int4", "int8"])
@pytest.mark.parametrize("gran", ["tensor", "row", "row_group"])
@pytest.mark.parametrize("shape", GROUP_SHAPES)
def test_rotate_quantize_group_sizes(cr, rot, qt, gran, shape):
    rows, K = shape
    say(f"rq rot {rot} {qt} {gran} {shape}")
    xb = wl.activation(15, rows * 3 + K + rot, rows, K, n_outliers=max(1, K // 200), outlier_scale=25.0)
    qg = 64 if gran == "row_group" else 0
    ref = ol.rotate_quantize(xb, rot, qt, gran, qg or None)
    codes, scales, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), rot, QT[qt], GR[gran], qg)
    assert np.array_equal(host(codes).reshape(ref["codes"].shape).view(np.uint8),
                          ref["codes"].view(np.uint8)), "codes differ"
    assert np.array_equal(host(scales).reshape(-1).view(np.uint32),
                          np.asarray(ref["scales"], np.float32).reshape(-1).view(np.uint32)), "scales differ"
    if qt == "int4":
        tcodes, _, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), rot, 0, GR[gran], qg, layout=1)
        assert np.array_equal(opack.tile_unpack_a(host(tcodes), rows), ref["codes"]), "tiled codes differ"


@pytest.mark.parametrize("rot", [256, 64, 1024])
@pytest.mark.parametrize("shape", [(37, 3072), (300, 1024), (129, 12288)])
def test_rotate_quantize_dual(cr, rot, shape):
    """One rotation, per-tensor INT4 (tiled) and INT8 codes: both sets and
    scales equal the oracle's separate quantizations bit for bit."""
    rows, K = shape
    say(f"rq dual rot {rot} {shape}")
    xb = wl.activation(19, rows + K + rot, rows, K, n_outliers=max(1, K // 200), outlier_scale=25.0)
    r4 = ol.rotate_quantize(xb, rot, "int4", "tensor")
    r8 = ol.rotate_quantize(xb, rot, "int8", "tensor")
    c4, s4, c8, s8 = cr.convrot_rotate_quantize_dual(bf16_dev(xb), rot, layout4=1)
    assert np.array_equal(opack.tile_unpack_a(host(c4), rows), r4["codes"])
    assert np.array_equal(host(s4).view(np.uint32), np.asarray(r4["scales"], np.float32).reshape(-1).view(np.uint32))
    assert np.array_equal(host(c8).view(np.uint8), r8["codes"].view(np.uint8))
    assert np.array_equal(host(s8).view(np.uint32), np.asarray(r8["scales"], np.float32).reshape(-1).view(np.uint32))
    n4, _, _, _ = cr.convrot_rotate_quantize_dual(bf16_dev(xb), rot, layout4=0)
    assert np.array_equal(host(n4), r4["codes"])


# Per-tensor scales on mid-size inputs (four 256-groups per lane and block,
# a grid of several hundred blocks, a ragged last 16-row block), every code
# layout and the dual output.
MID_SHAPES = [(1531, 4096), (3000, 3072), (4100, 4096)]


@pytest.mark.parametrize("rot", [256, 64, 16])
@pytest.mark.parametrize("shape", MID_SHAPES)
def test_rotate_quantize_tensor_mid(cr, rot, shape):
    rows, K = shape
    say(f"rq tensor mid rot {rot} {shape}")
    xb = wl.activation(17, rows + K + rot, rows, K, n_outliers=max(1, K // 200), outlier_scale=25.0)
    r4 = ol.rotate_quantize(xb, rot, "int4", "tensor")
    r8 = ol.rotate_quantize(xb, rot, "int8", "tensor")
    s4ref = np.asarray(r4["scales"], np.float32).reshape(-1).view(np.uint32)
    for layout in (0, 1, 3):
        codes, scales, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), rot, 0, 0, layout=layout)
        got = host(codes)
        if layout == 0:
            assert np.array_equal(got, r4["codes"]), "natural codes differ"
        elif layout == 1:
            assert np.array_equal(opack.tile_unpack_a(got, rows), r4["codes"]), "tiled codes differ"
        else:
            assert np.array_equal(opack.f6_unpack(got, rows), r4["values"]), "fp6 codes differ"
        assert np.array_equal(host(scales).view(np.uint32), s4ref)
    c8, s8, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), rot, 1, 0)
    assert np.array_equal(host(c8).view(np.uint8), r8["codes"].view(np.uint8))
    assert np.array_equal(host(s8).view(np.uint32), np.asarray(r8["scales"], np.float32).reshape(-1).view(np.uint32))
    d4, ds4, d8, ds8 = cr.convrot_rotate_quantize_dual(bf16_dev(xb), rot, layout4=3)
    assert np.array_equal(opack.f6_unpack(host(d4), rows), r4["values"])
    assert np.array_equal(host(ds4).view(np.uint32), s4ref)
    assert np.array_equal(host(d8).view(np.uint8), r8["codes"].view(np.uint8))


# Per-tensor plans on a 256-CU MI355X: at most 64 groups of 256 take one
# workgroup; grids up to one workgroup per CU (256) with one or two groups per
# segment (one for the 16 and 64 rotations) take one launch with the maxima
# exchanged through the workspace; larger inputs take two launches. Cases
# (shape, launches with the 256 rotation, with 16 and 64): (4, 4096) is 64
# groups, (4, 4352) 68; (256, 4096) is exactly 256 workgroups of one group,
# (272, 4096) one row block more; (672, 3072) is 252 workgroups of two
# groups, (688, 3072) 258.
PLAN_CASES = [((1, 256), 1, 1), ((2, 3072), 1, 1), ((4, 4096), 1, 1), ((4, 4352), 1, 1), ((256, 4096), 1, 1),
              ((272, 4096), 1, 2), ((512, 3072), 1, 2), ((672, 3072), 1, 2), ((688, 3072), 2, 2),
              ((4096, 3072), 2, 2)]


@pytest.mark.parametrize("rot", [256, 64, 16])
@pytest.mark.parametrize("case", PLAN_CASES, ids=lambda c: f"{c[0][0]}x{c[0][1]}")
def test_rotate_quantize_tensor_plans(cr, rot, case):
    """Every code layout, INT8 codes and the dual output at each plan
    boundary, bit-exact against the oracle; launch counts as planned."""
    (rows, K), l256, l_other = case
    launches = l256 if rot == 256 else l_other
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        launches = None   # the plan follows the CU count
    say(f"rq tensor plan rot {rot} {(rows, K)}")
    xb = wl.activation(29, rows + K + rot, rows, K, n_outliers=max(1, K // 200), outlier_scale=25.0)
    r4 = ol.rotate_quantize(xb, rot, "int4", "tensor")
    r8 = ol.rotate_quantize(xb, rot, "int8", "tensor")
    s4ref = np.asarray(r4["scales"], np.float32).reshape(-1).view(np.uint32)
    s8ref = np.asarray(r8["scales"], np.float32).reshape(-1).view(np.uint32)
    for layout in (0, 1, 3):
        cr.reset_counters()
        codes, scales, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), rot, 0, 0, layout=layout)
        assert launches is None or cr.get_counters()["rotate_quantize"] == launches
        got = host(codes)
        if layout == 0:
            assert np.array_equal(got, r4["codes"]), "natural codes differ"
        elif layout == 1:
            assert np.array_equal(opack.tile_unpack_a(got, rows), r4["codes"]), "tiled codes differ"
        else:
            assert np.array_equal(opack.f6_unpack(got, rows), r4["values"]), "fp6 codes differ"
        assert np.array_equal(host(scales).view(np.uint32), s4ref)
    c8, s8, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), rot, 1, 0)
    assert np.array_equal(host(c8).view(np.uint8), r8["codes"].view(np.uint8))
    assert np.array_equal(host(s8).view(np.uint32), s8ref)
    h8, hs8, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), rot, 1, 0, layout=4)
    assert np.array_equal(host(h8).view(np.uint16), r8["values"].astype(np.float16).view(np.uint16))
    assert np.array_equal(host(hs8).view(np.uint32), s8ref)
    for layout4 in (1, 3):
        cr.reset_counters()
        d4, ds4, d8, ds8 = cr.convrot_rotate_quantize_dual(bf16_dev(xb), rot, layout4=layout4)
        assert launches is None or cr.get_counters()["rotate_quantize"] == launches
        if layout4 == 1:
            assert np.array_equal(opack.tile_unpack_a(host(d4), rows), r4["codes"])
        else:
            assert np.array_equal(opack.f6_unpack(host(d4), rows), r4["values"])
        assert np.array_equal(host(ds4).view(np.uint32), s4ref)
        assert np.array_equal(host(d8).view(np.uint8), r8["codes"].view(np.uint8))
        assert np.array_equal(host(ds8).view(np.uint32), s8ref)


def test_rotate_quantize_tensor_workspace_contents(cr):
    """The one-launch exchange accepts any workspace contents and needs no
    clearing: random bytes, an int64 count-up pattern, repeated calls (the
    epoch moves on), a call with another grid size on the same workspace,
    and a workspace shifted by 16 bytes all give the oracle's codes."""
    shapes = [(300, 3072), (37, 3072), (700, 3072), (512, 3072)]
    ref = {}
    xs = {}
    for rows, K in shapes:
        xb = wl.activation(31, rows + K, rows, K, n_outliers=max(1, K // 200), outlier_scale=25.0)
        xs[(rows, K)] = bf16_dev(xb)
        r = ol.rotate_quantize(xb, 256, "int4", "tensor")
        ref[(rows, K)] = (r["codes"], np.asarray(r["scales"], np.float32).reshape(-1).view(np.uint32))
    need = max(cr.convrot_rq_workspace_size(r, K, 256, 0, 0) for r, K in shapes)
    g = torch.Generator(device="cpu").manual_seed(5)
    rnd = torch.randint(0, 256, (need + 64,), dtype=torch.uint8, generator=g).to("cuda")
    ramp = torch.arange((need + 64) // 8, dtype=torch.int64).view(torch.uint8).to("cuda")
    for ws in (rnd, ramp):
        seq = [shapes[0], shapes[0], shapes[1], shapes[0], shapes[2], shapes[1], shapes[0]]
        for off in (0, 16):
            w = ws[off:off + need]
            for shp in seq:
                say(f"rq workspace contents {shp} offset {off}")
                codes, scales, _, _ = cr.convrot_rotate_quantize(xs[shp], 256, 0, 0, workspace=w)
                assert np.array_equal(host(codes), ref[shp][0]), f"codes differ at {shp}"
                assert np.array_equal(host(scales).view(np.uint32), ref[shp][1])


def _check_lora_act(la, xb, l2, f32):
    la_ref32 = ol.lora_down(xb, l2, act_f32=True).astype(np.float64)
    mag = np.abs(wl.f32_from_bf16_bits(xb)).astype(np.float64) @ np.abs(wl.f32_from_bf16_bits(l2)).astype(np.float64).T
    got = host(la)
    if f32:
        assert np.all(np.abs(got - la_ref32) <= mag * 2 ** -20 + 1e-30)
    else:
        gotf = wl.f32_from_bf16_bits(got).astype(np.float64)
        assert np.all(np.abs(gotf - la_ref32) <= np.abs(la_ref32) * 2.0 ** -7 + mag * 2 ** -20 + 1e-30)


@pytest.mark.parametrize("R", [32, 64])
@pytest.mark.parametrize("mode", [("int4", "tensor"), ("int8", "row"), ("int4", "row_group")])
def test_rotate_quantize_with_lora_down(cr, R, mode):
    """Rotation on plus the low-rank down-projection of the unrotated input
    (the LoRA bypass): codes and scales bit-exact, la to float32-sum bounds."""
    qt, gran = mode
    rows, K = 150, 3072
    say(f"rq rot 256 + lora R={R} {mode}")
    xb = wl.activation(20, R, rows, K, n_outliers=10, outlier_scale=20.0)
    l2 = wl.weight(20, 500 + R, R, K, std=0.05)
    qg = 64 if gran == "row_group" else 0
    ref = ol.rotate_quantize(xb, 256, qt, gran, qg or None)
    for f32 in (False, True):
        codes, scales, _, la = cr.convrot_rotate_quantize(bf16_dev(xb), 256, QT[qt], GR[gran], qg,
                                                          lora_down=bf16_dev(l2), lora_act_f32=f32)
        assert np.array_equal(host(codes).reshape(ref["codes"].shape).view(np.uint8), ref["codes"].view(np.uint8))
        assert np.array_equal(host(scales).reshape(-1).view(np.uint32),
                              np.asarray(ref["scales"], np.float32).reshape(-1).view(np.uint32))
        _check_lora_act(la, xb, l2, f32)


def test_rotate_quantize_plain_lora_rank64(cr):
    rows, K = 77, 1024
    xb = wl.activation(21, 0, rows, K)
    l2 = wl.weight(21, 1, 64, K, std=0.05)
    ref = ol.rotate_quantize(xb, 0, "int4", "row_group", 64)
    codes, scales, _, la = cr.convrot_rotate_quantize(bf16_dev(xb), 0, 0, 2, 64, lora_down=bf16_dev(l2))
    assert np.array_equal(host(codes), ref["codes"])
    _check_lora_act(la, xb, l2, False)


MERGE_CASES = [("int4", "tensor", 256), ("int4", "row", 1024), ("int4", "row_group", 64), ("int8", "tensor", 256),
               ("int8", "row", 16), ("int4", "tensor", 0), ("asym_u4", "row_group", 256)]


@pytest.mark.parametrize("case", MERGE_CASES)
@pytest.mark.parametrize("R", [0, 16, 64])
def test_dequantize_weights_merge(cr, case, R):
    """Quantized weights back to bf16 in the unrotated basis plus a low-rank
    delta (a LoRA merge): bit-exact against the oracle."""
    qt, gran, rot = case
    N, K = 256, 3072
    say(f"dequantize {case} R={R}")
    wb = wl.weight(22, rot + R, N, K)
    qg = {"row_group": 16 if qt == "asym_u4" else 64}.get(gran)
    ref = ol.rotate_quantize(wb, rot, qt, gran, qg)
    QQ = {"int4": 0, "int8": 1, "asym_u4": 3}[qt]
    codes = dev(np.ascontiguousarray(ref["codes"]))
    scales = dev(np.ascontiguousarray(ref["scales"]))
    zeros = dev(ref["zeros_packed"]) if qt == "asym_u4" else None
    up = wl.weight(22, 900 + R, N, R, std=0.05) if R else None
    down = wl.weight(22, 901 + R, R, K, std=0.05) if R else None
    out = cr.convrot_dequantize_weights(codes, scales, N, K, QQ, GR[gran], qg or 0, rot, zeros=zeros,
                                        delta_up=None if up is None else bf16_dev(up),
                                        delta_down=None if down is None else bf16_dev(down))
    want = ol.dequantize_weights(ref["values"], ref["scales"], qt, gran, qg, ref.get("zeros"), rot, up, down)
    assert np.array_equal(host(out).view(np.uint16), want)


def test_lora_merge_round_trip(cr):
    """The whole merge on the GPU path: quantize (ConvRot 256, INT4 per
    tensor), dequantize + delta, quantize and pack again; codes, scale and the
    packed tiles equal the oracle's same steps."""
    N, K, R = 384, 3072, 32
    wb = wl.weight(23, 0, N, K)
    up, down = wl.weight(23, 1, N, R, std=0.05), wl.weight(23, 2, R, K, std=0.05)
    codes, scales, _, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, 0, 0)
    merged = cr.convrot_dequantize_weights(codes, scales, N, K, 0, 0, 0, 256, delta_up=bf16_dev(up),
                                           delta_down=bf16_dev(down))
    c2, s2, _, _ = cr.convrot_rotate_quantize(merged, 256, 0, 0)
    packed = cr.w4_pack_weights(c2, s2, N, K)[0]
    r0 = ol.rotate_quantize(wb, 256, "int4", "tensor")
    mb = ol.dequantize_weights(r0["values"], r0["scales"], "int4", "tensor", None, None, 256, up, down)
    r1 = ol.prepare_w4a4(mb, 256, "tensor")
    assert np.array_equal(host(merged).view(np.uint16), mb)
    assert np.array_equal(host(c2), r1["codes"])
    assert np.array_equal(host(s2).view(np.uint32), np.asarray(r1["scales"], np.float32).reshape(-1).view(np.uint32))
    assert np.array_equal(bytes_of(packed), r1["tiles"].reshape(-1))


SMOOTH_CASES = [(256, "int4", "row"), (256, "int8", "row_group"), (256, "int8", "row"), (0, "int4", "row_group"),
                (0, "uint4_shift", "row_group")]


@pytest.mark.parametrize("case", SMOOTH_CASES)
@pytest.mark.parametrize("shape", [(37, 3072), (300, 1024)])
def test_rotate_quantize_smoothing(cr, case, shape):
    """A per-channel smoothing multiplier before the rotation (and before the
    unsigned shift): codes and scales bit-exact against the oracle."""
    rot, qt, gran = case
    rows, K = shape
    say(f"rq smooth {case} {shape}")
    g = np.random.default_rng(rows + K + rot)
    m = (g.random(K) * 1.5 + 0.25).astype(np.float32)
    if qt == "uint4_shift":
        xb = wl.gelu_activation(24, rows + K, rows, K)
    else:
        xb = wl.activation(24, rows + K, rows, K, n_outliers=5, outlier_scale=20.0)
    qg = 64 if gran == "row_group" else 0
    shift = 0.171875 if qt == "uint4_shift" else 0.0
    ref = ol.rotate_quantize(xb, rot, qt, gran, qg or None, shift, smooth=m)
    QQ = {"int4": 0, "int8": 1, "uint4_shift": 2}[qt]
    codes, scales, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), rot, QQ, GR[gran], qg, shift=shift, smooth=dev(m))
    assert np.array_equal(host(codes).reshape(ref["codes"].shape).view(np.uint8), ref["codes"].view(np.uint8))
    assert np.array_equal(host(scales).reshape(-1).view(np.uint32),
                          np.asarray(ref["scales"], np.float32).reshape(-1).view(np.uint32))


def test_rotate_quantize_strided_rows_and_zero_rows(cr):
    rows, K, ldx = 40, 1024, 1024 + 64
    xb = wl.activation(12, 0, rows, ldx)
    xb[3, :] = 0          # an all-zero row: scale 0, codes 0
    xb[7, :K] = 0
    full = bf16_dev(xb)
    view = full[:, :K]
    for gran in ("row", "tensor", "row_group"):
        qg = 64 if gran == "row_group" else 0
        ref = ol.rotate_quantize(np.ascontiguousarray(xb[:, :K]), 256, "int4", gran, qg or None)
        codes, scales, _, _ = cr.convrot_rotate_quantize(view, 256, 0, GR[gran], qg)
        assert np.array_equal(host(codes), ref["codes"])
        assert np.array_equal(host(scales).reshape(-1), np.asarray(ref["scales"]).reshape(-1))


@pytest.mark.parametrize("unsigned", [False, True])
def test_rotate_quantize_plain_strided_rows_and_zero_rows(cr, unsigned):
    """Unrotated 64-group quantizer on a row-strided view (ldx = K + 64) with
    all-zero rows, through the 32-row blocks (8170 rows), every code layout
    and the fused rank-32 down-projection (identical to the contiguous run)."""
    rows, K, ldx = 8170, 256, 320
    say(f"rq plain strided unsigned={unsigned}")
    xb = (wl.gelu_activation if unsigned else wl.activation)(18, 5, rows, ldx)
    xb[3, :] = 0
    xb[rows - 1, :K] = 0
    shift = 0.171875 if unsigned else 0.0
    qt = 2 if unsigned else 0
    dense = np.ascontiguousarray(xb[:, :K])
    ref = ol.rotate_quantize(dense, 0, "uint4_shift" if unsigned else "int4", "row_group", 64, shift)
    l2 = bf16_dev(wl.weight(18, 6, 32, K, std=0.05))
    view = bf16_dev(xb)[:, :K]
    _, _, _, la_dense = cr.convrot_rotate_quantize(bf16_dev(dense), 0, qt, 2, 64, shift=shift, lora_down=l2)
    for layout in (0, 1, 3):
        codes, scales, _, la = cr.convrot_rotate_quantize(view, 0, qt, 2, 64, shift=shift, lora_down=l2, layout=layout)
        got = host(codes)
        if layout == 0:
            assert np.array_equal(got, ref["codes"])
        elif layout == 1:
            assert np.array_equal(opack.tile_unpack_a(got, rows), ref["codes"])
        else:
            assert np.array_equal(opack.f6_unpack(got, rows) * (2 if unsigned else 1), ref["values"])
        assert np.array_equal(host(scales).view(np.uint32), ref["scales"].view(np.uint32))
        assert np.array_equal(host(la), host(la_dense))


def test_rotate_quantize_subnormal_and_tiny_inputs(cr):
    rows, K = 8, 512
    g = np.random.default_rng(5)
    # inputs around the float32 normal/subnormal boundary; every scale group
    # keeps qmax / max|v| finite (the documented domain), while the stored
    # scales (max|v| / qmax / 16) fall into the subnormal range
    x = (g.standard_normal((rows, K)) * 1e-38).astype(np.float32)
    xb = wl.bf16_bits_from_f32(x)
    for qt in ("int4", "int8"):
        ref = ol.rotate_quantize(xb, 256, qt, "row")
        codes, scales, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, QT[qt], 1)
        assert np.array_equal(host(codes).view(np.uint8), ref["codes"].view(np.uint8))
        assert np.array_equal(host(scales).view(np.uint32), ref["scales"].view(np.uint32))


@pytest.mark.parametrize("shape", [(128, 512), (384, 3072), (256, 12288)])
def test_rotate_quantize_asym_weights(cr, shape):
    N, K = shape
    say(f"rq asym {shape}")
    wb = wl.weight(13, N + K, N, K)
    wb[5, 16:32] = 0      # a constant group
    ref = ol.rotate_quantize(wb, 256, "asym_u4", "row_group", 16)
    codes, scales, zeros, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, 3, 2, 16)
    assert np.array_equal(host(codes), ref["codes"])
    assert np.array_equal(host(scales).view(np.uint16), ref["scales"].view(np.uint16))
    assert np.array_equal(host(zeros), ref["zeros_packed"])


@pytest.mark.parametrize("unsigned", [False, True])
@pytest.mark.parametrize("lora", [None, "bf16", "f32"])
@pytest.mark.parametrize("shape", [(16, 256), (45, 3072), (200, 1024)])
def test_rotate_quantize_plain_g64(cr, unsigned, lora, shape):
    rows, K = shape
    say(f"rq plain unsigned={unsigned} lora={lora} {shape}")
    if unsigned:
        xb = wl.gelu_activation(14, rows + K, rows, K)
    else:
        xb = wl.activation(14, rows + K, rows, K)
    shift = 0.171875 if unsigned else 0.0
    ref = ol.rotate_quantize(xb, 0, "uint4_shift" if unsigned else "int4", "row_group", 64, shift)
    l2 = wl.weight(14, 999, 32, K, std=0.05) if lora else None
    codes, scales, _, la = cr.convrot_rotate_quantize(
        bf16_dev(xb), 0, 2 if unsigned else 0, 2, 64, shift=shift,
        lora_down=None if l2 is None else bf16_dev(l2), lora_act_f32=(lora == "f32"))
    assert np.array_equal(host(codes), ref["codes"])
    assert np.array_equal(host(scales).view(np.uint32), ref["scales"].view(np.uint32))
    tcodes, _, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 0, 2 if unsigned else 0, 2, 64, shift=shift,
                                                 layout=1)
    assert np.array_equal(opack.tile_unpack_a(host(tcodes), rows), ref["codes"])
    if lora:
        la_ref32 = ol.lora_down(xb, l2, act_f32=True).astype(np.float64)
        mag = np.abs(wl.f32_from_bf16_bits(xb)).astype(np.float64) @ np.abs(wl.f32_from_bf16_bits(l2)).astype(np.float64).T
        got = host(la)
        if lora == "f32":
            assert np.all(np.abs(got - la_ref32) <= mag * 2 ** -20 + 1e-30)
        else:
            gotf = wl.f32_from_bf16_bits(got).astype(np.float64)
            ulp = np.abs(la_ref32) * 2.0 ** -7 + mag * 2 ** -20
            assert np.all(np.abs(gotf - la_ref32) <= ulp + 1e-30)


# Tall inputs take the 32-row blocks of the unrotated quantizer (two 16-row
# tiles per block share each low-rank fragment): 8170 rows leave the last
# block's second tile empty, 8190 fill it partly, 8192 exactly.
@pytest.mark.parametrize("unsigned", [False, True])
@pytest.mark.parametrize("rows", [8170, 8190, 8192])
def test_rotate_quantize_plain_g64_tall(cr, unsigned, rows):
    K = 256 if rows != 8192 else 448
    say(f"rq plain tall unsigned={unsigned} rows={rows} K={K}")
    xb = (wl.gelu_activation if unsigned else wl.activation)(16, rows + K, rows, K)
    shift = 0.171875 if unsigned else 0.0
    ref = ol.rotate_quantize(xb, 0, "uint4_shift" if unsigned else "int4", "row_group", 64, shift)
    l2 = wl.weight(16, 77, 32, K, std=0.05)
    kw = dict(shift=shift, lora_down=bf16_dev(l2))
    qt = 2 if unsigned else 0
    codes, scales, _, la = cr.convrot_rotate_quantize(bf16_dev(xb), 0, qt, 2, 64, **kw)
    assert np.array_equal(host(codes), ref["codes"])
    assert np.array_equal(host(scales).view(np.uint32), ref["scales"].view(np.uint32))
    tcodes, tsc, _, tla = cr.convrot_rotate_quantize(bf16_dev(xb), 0, qt, 2, 64, layout=1, **kw)
    assert np.array_equal(opack.tile_unpack_a(host(tcodes), rows), ref["codes"])
    fcodes, fsc, _, fla = cr.convrot_rotate_quantize(bf16_dev(xb), 0, qt, 2, 64, layout=3, **kw)
    assert np.array_equal(opack.f6_unpack(host(fcodes), rows) * (2 if unsigned else 1), ref["values"])
    for s2 in (tsc, fsc):
        assert np.array_equal(host(s2).view(np.uint32), ref["scales"].view(np.uint32))
    la_ref32 = ol.lora_down(xb, l2, act_f32=True).astype(np.float64)
    mag = np.abs(wl.f32_from_bf16_bits(xb)).astype(np.float64) @ np.abs(wl.f32_from_bf16_bits(l2)).astype(np.float64).T
    gotf = wl.f32_from_bf16_bits(host(la)).astype(np.float64)
    assert np.all(np.abs(gotf - la_ref32) <= np.abs(la_ref32) * 2.0 ** -7 + mag * 2 ** -20 + 1e-30)
    # the three layouts run the same low-rank accumulation
    assert np.array_equal(host(la), host(tla)) and np.array_equal(host(la), host(fla))


@pytest.mark.parametrize("gran", ["tensor", "row", "row_group"])
@pytest.mark.parametrize("shape", [(128, 512), (384, 3072)])
def test_pack_w4a4(cr, gran, shape):
    N, K = shape
    say(f"pack w4a4 {gran} {shape}")
    wb = wl.weight(15, N + K, N, K)
    rot = 0 if gran == "row_group" else 256
    qg = 64 if gran == "row_group" else None
    ref = ol.prepare_w4a4(wb, rot, gran, qg)
    codes, scales, _, _ = cr.convrot_rotate_quantize(bf16_dev(wb), rot, 0, GR[gran], qg or 0)
    packed, pscales, _, wsum = cr.w4_pack_weights(codes, scales, N, K, 0, GR[gran], qg or 0, want_wsum=True)
    assert np.array_equal(bytes_of(packed), ref["tiles"].reshape(-1))
    if gran == "row_group":
        assert np.array_equal(host(pscales).reshape(-1), ref["scales_tiles"].reshape(-1))
    w = host(wsum)
    assert np.allclose(w, ref["wsum"], rtol=1e-5, atol=1e-5 * np.abs(ref["wsum"]).max())


@pytest.mark.parametrize("shape", [(128, 512), (256, 3072)])
def test_pack_w4a8(cr, shape):
    N, K = shape
    say(f"pack w4a8 {shape}")
    wb = wl.weight(16, N + K, N, K)
    ref = ol.prepare_w4a8(wb)
    codes, scales, zeros, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, 3, 2, 16)
    packed, pscales, pzeros, _ = cr.w4_pack_weights(codes, scales, N, K, 3, 2, 16, zeros=zeros)
    assert np.array_equal(bytes_of(packed), ref["tiles"].reshape(-1))
    assert np.array_equal(host(pscales).view(np.uint16).reshape(-1), ref["scales_tiles"].view(np.uint16).reshape(-1))
    assert np.array_equal(host(pzeros).reshape(-1), ref["zeros_tiles"].reshape(-1))


@pytest.mark.parametrize("shape", [(128, 32), (384, 64), (3072, 32)])
def test_pack_lora_up(cr, shape):
    """L1 [N, R] -> [N/128, R, 128] on the GPU, byte-exact against the oracle."""
    N, R = shape
    say(f"pack lora_up {shape}")
    rng = np.random.default_rng(N + R)
    up = rng.integers(0, 1 << 16, size=(N, R), dtype=np.uint16)
    got = cr.w4_pack_lora_up(bf16_dev(up))
    assert tuple(got.shape) == (N // 128, R, 128)
    assert np.array_equal(host(got).reshape(-1), opack.tile_pack_lora_up(up).reshape(-1))


def test_pack_sampled_tiles_full_size(cr):
    # full-size MLP-up weight (12288 x 3072): GPU pack vs oracle pack of sampled tiles
    N, K = 12288, 3072
    wb = wl.weight(17, 0, N, K)
    codes, scales, zeros, _ = cr.convrot_rotate_quantize(bf16_dev(wb), 256, 3, 2, 16)
    packed, _, _, _ = cr.w4_pack_weights(codes, scales, N, K, 3, 2, 16, zeros=zeros)
    tiles = bytes_of(packed).reshape(N // 128, K // 64, 4096)
    g = np.random.default_rng(0)
    for tn, kt in zip(g.integers(0, N // 128, 6), g.integers(0, K // 64, 6)):
        sub = ol.rotate_quantize(wb[128 * tn:128 * tn + 128], 256, "asym_u4", "row_group", 16)["values"]
        ref = opack.tile_pack_w4a8(np.ascontiguousarray(sub[:, 64 * kt:64 * kt + 64]))
        assert np.array_equal(tiles[tn, kt], ref[0, 0])


def test_determinism(cr):
    xb = wl.activation(18, 0, 333, 3072, n_outliers=10, outlier_scale=30.0)
    x = bf16_dev(xb)
    a = cr.convrot_rotate_quantize(x, 256, 0, 0)
    b = cr.convrot_rotate_quantize(x, 256, 0, 0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("qt,gran", [("int4", "tensor"), ("int4", "row"), ("int8", "tensor"), ("int8", "row")])
def test_rotate_quantize_constructed_ties(cr, qt, gran):
    """Round half to even through the GPU quantizer, on constructed ties: the
    input is x = H v / 256 per 256-group (H H = 256 I), so the rotation
    returns v exactly; v holds one value qmax 2^e per row (the maximum, so
    r = qmax / A = 2^-e is exact) and values (k + 1/2) 2^e, whose codes must
    come out as the even neighbour (v chosen so that x is exact in bf16)."""
    qmax = 7 if qt == "int4" else 127
    rows, K, e = 48, 512, -3
    H = oh.regular_hadamard(256).astype(np.float64)
    rng = np.random.default_rng(71 + qmax)
    V = np.zeros((rows, K))
    for r in range(rows):
        V[r, rng.integers(0, 256)] = qmax * (1 if rng.random() < 0.5 else -1)
        nt = 8 if qt == "int4" else 2          # keeps every x within bf16's 8 significant bits
        kmax = qmax if qt == "int4" else 64
        for j in rng.choice(256, nt, replace=False):
            V[r, 256 + j] = (rng.integers(0, kmax) + 0.5) * (1 if rng.random() < 0.5 else -1)
    V *= 2.0 ** e
    X = np.concatenate([V[:, :256] @ H / 256.0, V[:, 256:] @ H / 256.0], axis=1)
    xb = wl.bf16_bits_from_f32(X.astype(np.float32))
    assert np.array_equal(wl.f32_from_bf16_bits(xb).astype(np.float64), X), "input not exact in bf16"
    want = np.rint(V / 2.0 ** e).astype(np.int64)          # numpy rint: half to even
    assert np.all(np.abs(want) <= qmax) and np.any(np.abs(V / 2.0 ** e - np.trunc(V / 2.0 ** e)) == 0.5)
    ref = ol.rotate_quantize(xb, 256, qt, gran)
    assert np.array_equal(ref["values"].astype(np.int64), want)
    say(f"rq ties {qt} {gran}")
    codes, scales, _, _ = cr.convrot_rotate_quantize(bf16_dev(xb), 256, QT[qt], GR[gran], 0)
    got = host(codes)
    vals = opack.unpack_int4(got, True) if qt == "int4" else got
    assert np.array_equal(vals.astype(np.int64), want), "tie codes differ"
    assert np.all(host(scales).reshape(-1) == np.float32(2.0 ** e / 16))
