"""The allocation-free rotate+quantize (convrot_rotate_quantize_noalloc),
called through the C ABI, against convrot_rotate_quantize with a caller
workspace: codes and scales bit for bit, on consecutive calls whose second
input is smaller (the fixed scratch array keeps the first call's block
maxima, which the second must not see), for per-tensor INT4 (fp6 fragments
and tiled codes) and INT8 codes, per-row scales and the 1024 rotation."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from tests.gpu_helpers import bf16_dev, host, say  # noqa: E402


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_rotated_quantized_amd as m
    assert m.device_check() == 0
    return m


def _noalloc(cr, x, rot, qt, gran, layout, codes, scales):
    rows, K = x.shape
    st = cr.lib.convrot_rotate_quantize_noalloc(
        ctypes.c_void_p(x.data_ptr()), rows, K, x.stride(0), rot, qt, gran, 0, 0.0, None, None, 0, None, 0,
        ctypes.c_void_p(codes.data_ptr()), layout, ctypes.c_void_p(scales.data_ptr()), None,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, cr.status_string(st)


# (rows, K) of the first and the second (smaller) call
PAIRS = [((4096, 3072), (37, 1024)), ((8192, 12288), (300, 3072)), ((512, 3072), (2, 3072))]


@pytest.mark.parametrize("qt,gran,layout,rot", [(0, 0, 3, 256), (0, 0, 1, 256), (1, 0, 0, 256), (1, 0, 4, 256),
                                                (0, 1, 3, 256), (0, 0, 1, 1024)])
@pytest.mark.parametrize("pair", PAIRS)
def test_noalloc_matches_workspace_call(cr, qt, gran, layout, rot, pair):
    for i, (rows, K) in enumerate(pair):
        say(f"noalloc q{qt} g{gran} layout {layout} rot {rot} call {i} {rows}x{K}")
        # the second input's values are far smaller: stale maxima would change its scale
        xb = wl.activation(44, rows + K + i, rows, K, n_outliers=2, outlier_scale=30.0 if i == 0 else 1.0)
        x = bf16_dev(xb)
        want_c, want_s, _, _ = cr.convrot_rotate_quantize(x, rot, qt, gran, layout=layout)
        codes = torch.full_like(want_c, 0x3C if want_c.dtype == torch.uint8 else 1)
        scales = torch.full_like(want_s, -1.0)
        _noalloc(cr, x, rot, qt, gran, layout, codes, scales)
        assert np.array_equal(host(scales).view(np.uint32), host(want_s).view(np.uint32)), "scales differ"
        got, want = host(codes), host(want_c)
        if layout in (1, 3):       # rows past the end of the last row block are unspecified
            blk = 16 if layout == 1 else 32
            full = rows // blk
            assert np.array_equal(got[:full], want[:full]), "codes differ"
            if rows % blk:
                # compare the decoded valid rows of the last block
                from oracle import pack as opack
                if layout == 1:
                    assert np.array_equal(opack.tile_unpack_a(got, rows), opack.tile_unpack_a(want, rows))
                else:
                    assert np.array_equal(opack.f6_unpack(got, rows), opack.f6_unpack(want, rows))
        else:
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), "codes differ"
