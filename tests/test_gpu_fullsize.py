"""Full-size parity of the benchmarked path, every output row compared.

Each workload runs exactly as bench.py runs it (bench_workloads.Runner: the
same rotate+quantize passes, code layouts, 4-bit weight tiles expanded per
call, kernels and launch configurations), one step on one buffer set; then
every layer is checked against the oracle:
  * activation codes and scales bit-exact (every row);
  * packed weights bit-exact;
  * the exact integer result (CR_OUT_I32_RAW of the same call, the same
    kernel configuration) bit-exact on every row;
  * the step's bf16 output within 2e-3 relative L2 of the oracle's float32
    epilogue, over all rows.
The oracle's integer products are taken in row chunks as float64 BLAS on the
integer codes (exact below 2^53); group-scaled outputs use the oracle's exact
dequantized operands (s * q in float64), the same sum as the per-group form
grouped by k instead of by group.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from oracle import quant as oq, linear as ol, pack as opack  # noqa: E402
from tests.gpu_helpers import bf16_to_f32, bytes_of, host, say  # noqa: E402


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_rotated_quantized_amd as m
    assert m.device_check() == 0
    return m


def _chunks(M, step=1024):
    return [(r, min(M, r + step)) for r in range(0, M, step)]


class _Err:
    """relative L2 error accumulated over row chunks"""
    def __init__(self):
        self.num = self.den = 0.0

    def add(self, got, ref):
        ref = np.asarray(ref, np.float64)
        self.num += float(np.sum((np.asarray(got, np.float64) - ref) ** 2))
        self.den += float(np.sum(ref ** 2))

    def rel(self):
        return float(np.sqrt(self.num / self.den))


_RUNNERS = {}


def _runner(name, fuse=False):
    """one step of the workload as the benchmark runs it (one per module and
    workload); fuse: layers sharing an input run as one call, as in bench.py"""
    import bench_workloads as bw
    key = (name, fuse)
    if key not in _RUNNERS:
        for k in list(_RUNNERS):            # one workload's buffers on the device at a time
            del _RUNNERS[k]
        torch.cuda.empty_cache()
        r = bw.Runner(name, nsets=1, schedule="chains", fuse=fuse)   # token streams on streams of their own
        r.step(0)
        torch.cuda.synchronize()
        _RUNNERS[key] = r
    return _RUNNERS[key]


_ACT = {}


def _oracle_act(w, x_id, qt, gran="tensor", rot=256, group=None, shift=0.0):
    key = (w.config_id, x_id, qt, gran, rot, group, shift)
    if key not in _ACT:
        _ACT[key] = ol.rotate_quantize(wl.act_bits(w, x_id), rot, qt, gran, group, shift)
    return _ACT[key]


def _tensorwise_layer(cr, r, lin):
    """W4A4 or INT8 tensorwise layer of a runner: codes, weights, int32, bf16."""
    w = r.w
    M, N, K = lin.M, lin.N, lin.K
    st = r.sets[0]
    key = [k for l, k in r.gemm_plan if l.name == lin.name][0]
    o, p = st["rq"][key], st["prep"][lin.name]
    qt = "int4" if lin.fmt == "w4a4" else "int8"
    xa = _oracle_act(w, lin.x_id, qt)
    wq = ol.rotate_quantize(wl.weight_bits(w, lin), 256, qt, "tensor")
    if qt == "int4":
        got = host(o["codes"])
        if r.f6_codes(M):
            assert np.array_equal(opack.f6_unpack(got, M), xa["values"]), "fp6 codes differ"
        else:
            assert np.array_equal(opack.tile_unpack_a(got, M), xa["codes"]), "tiled codes differ"
        a, sa = o["codes"], o["scales"]
        assert np.array_equal(bytes_of(p["w"]), opack.tile_pack_w4a4(wq["codes"]).reshape(-1)), "weight tiles"
        raw = host(cr.w4a4_gemm(a, sa, 0, p["w"], p["ws"], 0, M, N, K, out_type=cr.OUT.I32_RAW,
                                workspace=st["gws"]))
    else:
        a, sa = (o["codes8"], o["scales8"]) if "codes8" in o else (o["codes"], o["scales"])
        assert np.array_equal(host(a), xa["codes"]), "int8 codes differ"
        assert np.array_equal(host(p["w"]), wq["codes"]), "int8 weights differ"
        raw = host(cr.int8_tensorwise_gemm(a, sa, p["w"], p["ws"], M, N, K, out_type=cr.OUT.I32_RAW))
    assert host(sa)[0] == np.float32(xa["scales"]).reshape(-1)[0]
    assert host(p["ws"])[0] == np.float32(wq["scales"]).reshape(-1)[0]
    y = bf16_to_f32(host(st["out"][lin.name]))
    A = xa["values"].astype(np.float64)
    W = wq["values"].astype(np.float64)
    err = _Err()
    for r0, r1 in _chunks(M):
        ref_raw = np.rint(A[r0:r1] @ W.T).astype(np.int64)
        assert np.array_equal(raw[r0:r1].astype(np.int64), ref_raw), f"int32 rows {r0}..{r1}"
        err.add(y[r0:r1], ol.epilogue_scalar(ref_raw, xa["scales"], "tensor", wq["scales"], "tensor"))
    assert err.rel() <= 2e-3, err.rel()


@pytest.mark.parametrize("name", ["proj4096", "proj32"])
def test_c2_full(cr, name):
    """The single MMDiT projection, M = 4096 (fp6 codes, 4-bit weight tiles
    expanded per call, fp6 matrix cores) and M = 32 (tiled int4 codes,
    weight-streaming int8-core kernel)."""
    r = _runner("c2")
    lin = [l for l in r.w.linears if l.name == name][0]
    say(f"c2 full {name}")
    _tensorwise_layer(cr, r, lin)


C4_LAYERS = [f"{s}_{n}" for s in ("img", "txt") for n in ("q", "k", "v", "out", "mlp_up", "mlp_down", "mod")]


@pytest.mark.parametrize("name", C4_LAYERS)
def test_c4_layer_full(cr, name):
    """Every linear of the mixed MMDiT block (W4A4: q, k, mlp_up, mlp_down;
    INT8: v, out, mod; image and text streams)."""
    r = _runner("c4")
    lin = [l for l in r.w.linears if l.name == name][0]
    say(f"c4 full {name} {lin.M}x{lin.N}x{lin.K}")
    _tensorwise_layer(cr, r, lin)


@pytest.mark.parametrize("s", ["img", "txt"])
def test_c4_fused_qk_full(cr, s):
    """The Q and K projections of one token stream as the benchmark runs them:
    one call on both weights side by side along N, per-channel scales holding
    each part's own per-tensor scale. Weight tiles, int32 sums and bf16
    outputs of both parts against the oracle, every output row."""
    r = _runner("c4", fuse=True)
    lin = [l for l in r.w.linears if l.name == f"{s}_q+{s}_k"][0]
    w_def = wl.CONFIGS["c4"]()
    M, N, K = lin.M, lin.N, lin.K
    say(f"c4 fused {lin.name} {M}x{N}x{K}")
    st = r.sets[0]
    key = [k for l, k in r.gemm_plan if l.name == lin.name][0]
    o, p = st["rq"][key], st["prep"][lin.name]
    xa = _oracle_act(w_def, lin.x_id, "int4")
    raw = host(cr.w4a4_gemm(o["codes"], o["scales"], 0, p["w"], p["ws"], cr.GRAN.ROW, M, N, K,
                            out_type=cr.OUT.I32_RAW, workspace=st["gws"]))
    y = bf16_to_f32(host(st["out"][lin.name]))
    tiles, ws = bytes_of(p["w"]), host(p["ws"])
    A = xa["values"].astype(np.float64)
    n0 = off = 0
    for part in lin.parts:
        wq = ol.rotate_quantize(wl.weight_bits(w_def, part), 256, "int4", "tensor")
        t = opack.tile_pack_w4a4(wq["codes"]).reshape(-1)
        assert np.array_equal(tiles[off:off + t.size], t), f"{part.name} tiles"
        assert np.all(ws[n0:n0 + part.N] == np.float32(wq["scales"]).reshape(-1)[0]), f"{part.name} scales"
        W = wq["values"].astype(np.float64)
        err = _Err()
        for r0, r1 in _chunks(M):
            ref_raw = np.rint(A[r0:r1] @ W.T).astype(np.int64)
            assert np.array_equal(raw[r0:r1, n0:n0 + part.N].astype(np.int64), ref_raw), f"{part.name} rows {r0}"
            err.add(y[r0:r1, n0:n0 + part.N],
                    ol.epilogue_scalar(ref_raw, xa["scales"], "tensor", wq["scales"], "tensor"))
        assert err.rel() <= 2e-3, (part.name, err.rel())
        n0 += part.N
        off += t.size


def test_c3_w4a8_full(cr):
    """W4A8: X [8192, 3072] int8 per token (fp16-carried codes, the layout the
    GEMM runs on), W [12288, 3072] asym uint4 g16."""
    r = _runner("c3")
    lin = r.w.linears[0]
    M, N, K = lin.M, lin.N, lin.K
    say(f"c3 full {M}x{N}x{K}")
    st = r.sets[0]
    key = r.gemm_plan[0][1]
    o, p = st["rq"][key], st["prep"][lin.name]
    xa = _oracle_act(r.w, lin.x_id, "int8", "row")
    wp = ol.prepare_w4a8(wl.weight_bits(r.w, lin))
    assert np.array_equal(host(o["codes"]).astype(np.int64), xa["values"].astype(np.int64))
    assert np.array_equal(host(o["scales"]).view(np.uint32), np.asarray(xa["scales"], np.float32).view(np.uint32))
    assert np.array_equal(bytes_of(p["w"]), wp["tiles"].reshape(-1))
    assert np.array_equal(host(p["ws"]).view(np.uint16).reshape(-1), wp["scales_tiles"].view(np.uint16).reshape(-1))
    assert np.array_equal(host(p["wz"]).reshape(-1), wp["zeros_tiles"].reshape(-1))
    args = (o["codes"], o["scales"], cr.GRAN.ROW, p["w"], p["ws"], p["wz"], M, N, K)
    raw = host(cr.w4a8_gemm(*args, out_type=cr.OUT.I32_RAW))
    yf = host(cr.w4a8_gemm(*args, out_type=cr.OUT.F32))
    yb = bf16_to_f32(host(st["out"][lin.name]))
    zexp = np.repeat(wp["zeros"].astype(np.int64), 16, axis=1)
    d = (wp["values"].astype(np.int64) - zexp).astype(np.float64)
    w_hat = oq.dequant_asym(wp["values"], wp["scales"], wp["zeros"], 16).astype(np.float64)
    A = xa["values"].astype(np.float64)
    s_a = np.asarray(xa["scales"], np.float64)
    eb, ef = _Err(), _Err()
    for r0, r1 in _chunks(M):
        assert np.array_equal(raw[r0:r1].astype(np.int64), np.rint(A[r0:r1] @ d.T).astype(np.int64))
        ref = (s_a[r0:r1, None] * (A[r0:r1] @ w_hat.T)).astype(np.float32)
        eb.add(yb[r0:r1], ref)
        ef.add(yf[r0:r1], ref)
    assert eb.rel() <= 2e-3, eb.rel()
    assert ef.rel() <= 1e-5, ef.rel()


@pytest.mark.parametrize("name", ["qkv", "mlp_down"])
def test_c5_lowrank_g64_full(cr, name):
    """Low-rank corrected W4A4 with 64-group scales (no rotation), as the
    benchmark runs it: fp6 codes (unsigned post-GELU codes as u/2 for MLP
    down, shift 0.171875), the rank-32 down-projection fused into the
    quantizer, 4-bit weight tiles expanded per call, the up-projection fused
    into the GEMM epilogue."""
    r = _runner("c5")
    lin = [l for l in r.w.linears if l.name == name][0]
    M, N, K = lin.M, lin.N, lin.K
    shift = lin.unsigned_shift
    uns = shift != 0.0
    say(f"c5 full {name} {M}x{N}x{K}")
    st = r.sets[0]
    key = [k for l, k in r.gemm_plan if l.name == lin.name][0]
    o, p = st["rq"][key], st["prep"][lin.name]
    xb = wl.act_bits(r.w, lin.x_id)
    l1, l2, res = wl.lowrank_bits(r.w, lin)
    xa = _oracle_act(r.w, lin.x_id, "uint4_shift" if uns else "int4", "row_group", 0, 64, shift)
    wp = ol.rotate_quantize(res, 0, "int4", "row_group", 64)
    assert np.array_equal(opack.f6_unpack(host(o["codes"]), M) * (2 if uns else 1), xa["values"])
    assert np.array_equal(host(o["scales"]).view(np.uint32), np.asarray(xa["scales"], np.float32).view(np.uint32))
    assert np.array_equal(bytes_of(p["w"]), opack.tile_pack_w4a4(wp["codes"]).reshape(-1))
    assert np.array_equal(host(p["ws"]).reshape(-1), opack.tile_pack_g64_scales(wp["scales"]).reshape(-1))
    # low-rank activations: bf16 of a float32 sum taken in another order -> within one bf16 ulp
    la = host(o["la"])
    la_ref32 = ol.lora_down(xb, l2, act_f32=True).astype(np.float64)
    mag = np.abs(wl.f32_from_bf16_bits(xb)).astype(np.float64) @ np.abs(wl.f32_from_bf16_bits(l2)).astype(np.float64).T
    got_la = wl.f32_from_bf16_bits(la).astype(np.float64)
    assert np.all(np.abs(got_la - la_ref32) <= np.abs(la_ref32) * 2.0 ** -7 + mag * 2 ** -20 + 1e-30)
    kw = dict(a_unsigned=uns, a_shift=shift, w_sum=p["wsum"])
    raw = host(cr.w4a4_gemm(o["codes"], o["scales"], 2, p["w"], p["ws"], 2, M, N, K, out_type=cr.OUT.I32_RAW,
                            workspace=st["gws"], **kw))
    y = bf16_to_f32(host(st["out"][lin.name]))
    wsum = ol.weight_sum(wp["values"], wp["scales"], "row_group", 64)
    assert np.allclose(host(p["wsum"]), wsum, rtol=1e-5, atol=1e-5 * np.abs(wsum).max())
    A = xa["values"].astype(np.float64)
    W = wp["values"].astype(np.float64)
    a_hat = A * np.repeat(np.asarray(xa["scales"], np.float64), 64, axis=1)
    w_hat = W * np.repeat(np.asarray(wp["scales"], np.float64), 64, axis=1)
    ones_m, ones_n = np.ones((M, 1)), np.ones((N, 1))
    la_use = wl.f32_from_bf16_bits(la)            # the GPU's la (its own rounding is checked above)
    err = _Err()
    for r0, r1 in _chunks(M):
        assert np.array_equal(raw[r0:r1].astype(np.int64), np.rint(A[r0:r1] @ W.T).astype(np.int64))
        ydq = a_hat[r0:r1] @ w_hat.T
        ref = ol.epilogue_g64(ydq[:, :, None], ones_m[r0:r1], ones_n, shift, wsum, la_use[r0:r1], l1)
        err.add(y[r0:r1], ref)
    assert err.rel() <= 2e-3, err.rel()
