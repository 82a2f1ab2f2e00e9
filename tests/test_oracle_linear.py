"""Pins of oracle.linear (epilogues and the composed linears).

Closed forms and special cases:
  * unit scales give y = acc exactly;
  * a g64 epilogue whose group scales are all equal reduces to the scalar one;
  * an exactly low-rank W gives an all-zero residual and y = low-rank branch;
  * the unsigned shift correction recovers the unshifted product;
  * the quantized linears approximate the float product, ranked
    int8 < w4a8 < w4a4 by relative error as on the W4A8-ConvRot card's
    per-layer table (a ranking, not a threshold);
  * rotation of BOTH operands is what makes W4A4 survive outlier channels
    (the purpose of ConvRot, [P1] intro).
"""
import json
import os

import numpy as np
from fractions import Fraction

from oracle import linear, gemm, quant, pack
import workloads as wl

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_unit_scales_identity():
    g = np.random.default_rng(30)
    acc = g.integers(-600000, 600000, size=(7, 9))
    y = linear.epilogue_scalar(acc, np.ones(1, np.float32), "tensor", np.ones(1, np.float32), "tensor")
    assert np.array_equal(y, acc.astype(np.float32))


def test_g64_equal_scales_reduce_to_scalar():
    g = np.random.default_rng(31)
    a = g.integers(-7, 8, size=(4, 256))
    w = g.integers(-7, 8, size=(5, 256))
    P = gemm.group_partials(a, w, 64)
    sa, sw = np.float32(0.37), np.float32(0.011)
    y1 = linear.epilogue_g64(P, np.full((4, 4), sa), np.full((5, 4), sw))
    y2 = linear.epilogue_scalar(P.sum(axis=2), np.array([sa]), "tensor", np.array([sw]), "tensor")
    assert np.array_equal(y1, y2)


def test_exact_low_rank_weight():
    g = np.random.default_rng(32)
    M, N, K, R = 8, 128, 256, 4
    l1 = wl.bf16_bits_from_f32((g.standard_normal((N, R)) * 0.1).astype(np.float32))
    l2 = wl.bf16_bits_from_f32(np.eye(R, K, dtype=np.float32))           # exact low rank
    w = wl.bf16_bits_from_f32(wl.f32_from_bf16_bits(l1) @ wl.f32_from_bf16_bits(l2))
    resid = wl.bf16_bits_from_f32(wl.f32_from_bf16_bits(w) - wl.f32_from_bf16_bits(l1) @ wl.f32_from_bf16_bits(l2))
    x = wl.activation(99, 0, M, K)
    out = linear.w4a4_linear(x, resid, rot_group=0, a_gran="row_group", w_gran="row_group",
                             group=64, l1_bits=l1, l2_bits=l2)
    assert np.all(out["w"]["values"] == 0)
    lr = wl.f32_from_bf16_bits(x).astype(np.float64) @ (wl.f32_from_bf16_bits(l1).astype(np.float64)
                                                        @ wl.f32_from_bf16_bits(l2).astype(np.float64)).T
    assert _rel(out["y"], lr) < 4e-3            # only the bf16 rounding of la remains


def test_shift_correction_recovers_unshifted_product():
    shift = GOLD["post_gelu_shift"]["value"]
    M, N, K = 16, 128, 512
    x = wl.gelu_activation(98, 0, M, K)
    w = wl.weight(98, 1, N, K)
    ref = linear.float_linear(x, w)
    shifted = linear.w4a4_linear(x, w, rot_group=0, a_gran="row_group", w_gran="row_group",
                                 group=64, shift=shift)
    # without the correction the output is off by shift * rowsum(W_hat)
    assert _rel(shifted["y"], ref) < 0.2
    wsum = shifted["w"]["wsum"].astype(np.float64)
    uncorrected = shifted["y"] + shift * wsum[None, :]
    assert _rel(uncorrected, ref) > 2 * _rel(shifted["y"], ref)


def test_error_ranking_matches_pages():
    ranking = GOLD["per_layer_rel_error_median"]["value"]
    assert ranking["bf16"] < ranking["w4a8"] < ranking["w4a4"]
    M, N, K = 64, 256, 512
    x = wl.activation(97, 0, M, K)
    w = wl.weight(97, 1, N, K)
    ref = linear.float_linear(x, w)
    e8 = _rel(linear.int8_linear(x, w)["y"], ref)
    e48 = _rel(linear.w4a8_linear(x, w)["y"], ref)
    e44 = _rel(linear.w4a4_linear(x, w)["y"], ref)
    assert e8 < e48 < e44
    assert e44 < 0.5


def test_rotation_rescues_outliers():
    M, N, K = 64, 256, 512
    x = wl.activation(96, 0, M, K, n_outliers=5, outlier_scale=20.0)
    w = wl.weight(96, 1, N, K)
    ref = linear.float_linear(x, w)
    rot = _rel(linear.w4a4_linear(x, w, rot_group=256)["y"], ref)
    plain = _rel(linear.w4a4_linear(x, w, rot_group=0)["y"], ref)
    assert rot < plain


def test_raw_equals_exact_integer_product():
    M, N, K = 32, 128, 512
    x = wl.activation(95, 0, M, K)
    w = wl.weight(95, 1, N, K)
    out = linear.w4a4_linear(x, w)
    qa = pack.unpack_int4(out["x"]["codes"], True)
    qw = pack.unpack_int4(pack.tile_unpack_w4a4(out["w"]["tiles"]), True)
    assert np.array_equal(out["raw"], qa.astype(np.int64) @ qw.astype(np.int64).T)
    o8 = linear.w4a8_linear(x, w)
    z = np.repeat(o8["w"]["zeros"].astype(np.int64), 16, axis=1)
    qw8 = pack.tile_unpack_w4a8(o8["w"]["tiles"]).astype(np.int64) - z
    assert np.array_equal(o8["raw"], o8["x"]["values"].astype(np.int64) @ qw8.T)


def test_lora_down_rounding():
    x = wl.activation(94, 0, 4, 256)
    l2 = wl.weight(94, 1, 8, 256, std=0.05)
    la32 = linear.lora_down(x, l2, act_f32=True)
    la16 = linear.lora_down(x, l2, act_f32=False)
    exact = wl.f32_from_bf16_bits(x).astype(np.float64) @ wl.f32_from_bf16_bits(l2).astype(np.float64).T
    assert np.allclose(la32, exact, rtol=1e-6, atol=1e-6)
    assert np.array_equal(la16, wl.f32_from_bf16_bits(wl.bf16_bits_from_f32(la32)))


# ---------------------------------------------------------------------------
# epilogue_g16 (W4A8): y = s_a[m] * sum_g s_w[n, g] * P[m, n, g]
# ---------------------------------------------------------------------------

def _g16_case(seed, M=5, N=6, G=7):
    rng = np.random.default_rng(seed)
    P = rng.integers(-30480, 30481, (M, N, G)).astype(np.int64)
    sa = (rng.random(M) * 0.01 + 1e-4).astype(np.float32)
    return rng, P, sa


def test_epilogue_g16_equal_group_scales_reduce_to_the_scalar_epilogue():
    # s_w[n, g] = c[n] for every g: the per-group sum collapses to c[n] * sum_g P
    rng, P, sa = _g16_case(11)
    c = (rng.random(P.shape[1]) * 0.02 + 1e-3).astype(np.float16)
    w = np.repeat(c[:, None], P.shape[2], axis=1)
    got = linear.epilogue_g16(P, sa, "row", w)
    want = linear.epilogue_scalar(P.sum(axis=2), sa, "row", c.astype(np.float32), "row")
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_epilogue_g16_power_of_two_scales_are_exact():
    # distinct powers of two per (channel, group) and per token: every output
    # is an exact dyadic value, so a scale taken from the wrong group or
    # channel, or a dropped group, changes it
    rng, P, sa_unused = _g16_case(12)
    M, N, G = P.shape
    ea = rng.integers(-9, -3, M)
    ew = rng.integers(-12, -4, (N, G))
    sa = np.ldexp(1.0, ea).astype(np.float32)
    sw = np.ldexp(1.0, ew).astype(np.float16)
    got = linear.epilogue_g16(P, sa, "row", sw)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g in range(G):
                tot += Fraction(2) ** int(ew[n, g]) * int(P[m, n, g])
            tot *= Fraction(2) ** int(ea[m])
            assert got[m, n] == np.float32(float(tot))


def test_epilogue_g16_brute_force_against_codes():
    # y from the integer codes by plain loops (exact rationals), against the
    # oracle's W4A8 linear on a tiny layer: the zero point, the group of each
    # scale and the token scale all enter
    M, N, K = 3, 128, 256
    x = wl.activation(93, 0, M, K)
    w = wl.weight(93, 1, N, K)
    out = linear.w4a8_linear(x, w)
    qa = out["x"]["values"].astype(np.int64)
    sa = out["x"]["scales"]
    qw = out["w"]["values"].astype(np.int64)
    sw = out["w"]["scales"]
    z = out["w"]["zeros"].astype(np.int64)
    for m in range(M):
        for n in range(0, N, 17):
            tot = Fraction(0)
            for g in range(K // 16):
                part = sum(int(qa[m, k]) * (int(qw[n, k]) - int(z[n, g])) for k in range(16 * g, 16 * g + 16))
                tot += Fraction(float(sw[n, g])) * part
            tot *= Fraction(float(sa[m]))
            want = float(tot)
            assert abs(float(out["y"][m, n]) - want) <= abs(want) * 2.0 ** -23 + 1e-30


def test_a8w4_linear_brute_force():
    # 8-bit activations x W4A4 weights, against a float64 triple loop over the
    # oracle's own codes and scales (checks the composition: granularities,
    # which scale goes with which axis, the bias)
    xb = wl.activation(31, 0, 3, 512)
    wb = wl.weight(31, 1, 128, 512)                   # tile packing wants N % 128 == 0
    bias = wl.weight(31, 2, 1, 128, std=0.5)[0]
    r = linear.a8w4_linear(xb, wb, 256, "row", "row", bias_bits=bias)
    qa, sa = r["x"]["values"], np.asarray(r["x"]["scales"], np.float64)
    qw, sw = r["w"]["values"], np.asarray(r["w"]["scales"], np.float64)
    assert qa.min() >= -127 and qa.max() <= 127 and qw.min() >= -7 and qw.max() <= 7
    bf = (bias.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for m in range(3):
        for n in (0, 1, 77, 127):
            acc = sum(int(qa[m, k]) * int(qw[n, k]) for k in range(512))
            assert r["raw"][m, n] == acc
            assert np.isclose(r["y"][m, n], sa[m] * sw[n] * acc + bf[n], rtol=1e-6, atol=0)


# ---------------------------------------------------------------------------
# dequantize_weights (LoRA merge)
# ---------------------------------------------------------------------------

def _bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def test_dequantize_without_rotation_is_scale_times_code():
    rng = np.random.default_rng(41)
    q = rng.integers(-7, 8, (3, 256))
    out = linear.dequantize_weights(q, np.array([2.0 ** -3], np.float32), "int4", "tensor", rot_group=0)
    assert np.array_equal(_bf16_value(out), q * 2.0 ** -3)


def test_dequantize_undoes_the_rotation_exactly_on_small_integers():
    # with s = 1 and small integer codes, H q / 4 (n = 16) is exact and bf16-representable:
    # the butterflies must reproduce the explicit regular Hadamard product
    from oracle import hadamard
    rng = np.random.default_rng(42)
    q = rng.integers(-7, 8, (2, 256))
    out = linear.dequantize_weights(q, np.array([1.0], np.float32), "int4", "tensor", rot_group=16)
    H = hadamard.regular_hadamard(16)
    ref = np.concatenate([q[:, 16 * g:16 * g + 16] @ H.T for g in range(16)], axis=1) / 4.0
    assert np.array_equal(_bf16_value(out), ref)


def test_dequantize_adds_the_low_rank_delta():
    rng = np.random.default_rng(43)
    q = rng.integers(-7, 8, (4, 256))
    up = rng.integers(-3, 4, (4, 2)).astype(np.float32)
    down = rng.integers(-3, 4, (2, 256)).astype(np.float32)
    to_bits = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out = linear.dequantize_weights(q, np.array([0.5], np.float32), "int4", "tensor", rot_group=0,
                                    up_bits=to_bits(up), down_bits=to_bits(down))
    assert np.array_equal(_bf16_value(out), q * 0.5 + up.astype(np.float64) @ down.astype(np.float64))


def test_dequantize_inverts_quantization_within_its_error():
    wb = wl.weight(44, 0, 128, 1024)
    for rot in (256, 64):
        r = linear.rotate_quantize(wb, rot, "int8", "row")
        back = _bf16_value(linear.dequantize_weights(r["values"], r["scales"], "int8", "row", rot_group=rot))
        w = _bf16_value(wb)
        err = np.linalg.norm(back - w) / np.linalg.norm(w)
        assert err < 0.01, err              # int8 per-row codes: about 0.4 % relative


# ---------------------------------------------------------------------------
# smoothing vector
# ---------------------------------------------------------------------------

def test_smoothing_by_ones_changes_nothing():
    xb = wl.activation(45, 0, 16, 512)
    a = linear.rotate_quantize(xb, 256, "int4", "row")
    b = linear.rotate_quantize(xb, 256, "int4", "row", smooth=np.ones(512, np.float32))
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


def test_smoothing_by_powers_of_two_scales_each_channel():
    # a power-of-two multiplier per channel is exact: smoothing x equals
    # quantizing the bf16 tensor x * m built directly, channel by channel
    xb = wl.activation(46, 0, 8, 512)
    m = (2.0 ** np.random.default_rng(3).integers(-3, 4, 512)).astype(np.float32)
    x = linear._f32(xb) * m[None, :]
    xm = (x.view(np.uint32) >> 16).astype(np.uint16)             # exact: bf16 times 2^j
    for rot, gran, qg in ((256, "row", None), (0, "row_group", 64)):
        a = linear.rotate_quantize(xb, rot, "int4", gran, qg, smooth=m)
        b = linear.rotate_quantize(xm, rot, "int4", gran, qg)
        assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


def test_smoothing_with_inverse_on_weights_preserves_the_product():
    # (x diag(m)) (W diag(1/m))^T = x W^T: with m a power of two per channel
    # the float products are equal up to the quantization of each side
    xb = wl.activation(47, 0, 32, 512)
    wb = wl.weight(47, 1, 128, 512)
    m = (2.0 ** np.random.default_rng(4).integers(-2, 3, 512)).astype(np.float32)
    w = linear._f32(wb) / m[None, :]
    wm = (w.view(np.uint32) >> 16).astype(np.uint16)
    ref = linear.float_linear(xb, wb)
    xa = linear.rotate_quantize(xb, 256, "int8", "row", smooth=m)
    wq = linear.rotate_quantize(wm, 256, "int8", "row")
    y = linear.epilogue_scalar(gemm.int_gemm(xa["values"], wq["values"]), xa["scales"], "row",
                               wq["scales"], "row")
    # quantization error of a few percent; a multiplier on the wrong axis (or a
    # missing inverse) would leave an error of order one
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.1
