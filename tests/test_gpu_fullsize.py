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
from oracle import linear as ol, gemm as og, pack as opack  # noqa: E402
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
