"""Pins of oracle.quant.

Fixed by the pages: signed INT4 codes ([P1] intro, [P5] Format), INT8
tensorwise ([P1] intro), dynamic activation scales ([P1] intro), asymmetric
4-bit weights in groups of 16 ([P2] file layout), unsigned post-GELU
activations with a +0.171875 shift ([P3] Kernel Engineering).
Fixed by mathematics: range, error bound of round-to-nearest, exact ties.
"""
import json
import os

import numpy as np
import pytest

from oracle import quant, hadamard

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def _scalar_sym(row, qmax):
    """Brute force per scalar, float32 arithmetic, for tiny inputs."""
    A = np.float32(0)
    for v in row:
        A = max(A, np.float32(abs(v)))
    if A == 0:
        return [0] * len(row), np.float32(0)
    r = np.float32(np.float32(qmax) / A)
    out = []
    for v in row:
        p = np.float32(np.float32(v) * r)
        q = int(np.rint(p))
        out.append(max(-qmax, min(qmax, q)))
    return out, np.float32(A / np.float32(qmax))


@pytest.mark.parametrize("qmax", [7, 127])
def test_sym_row_matches_scalar_bruteforce(qmax):
    g = np.random.default_rng(10)
    v = (g.standard_normal((6, 32)) * 3).astype(np.float32)
    q, s = quant.quantize_sym(v, qmax, "row")
    for r in range(6):
        qq, ss = _scalar_sym(v[r], qmax)
        assert list(q[r]) == qq
        assert s[r] == ss


@pytest.mark.parametrize("gran,group", [("tensor", None), ("row", None), ("row_group", 64)])
def test_sym_range_extremes_and_error_bound(gran, group):
    g = np.random.default_rng(11)
    v = (g.standard_normal((16, 256)) * np.exp(g.standard_normal((16, 256)))).astype(np.float32)
    q, s = quant.quantize_sym(v, 7, gran, group)
    assert q.min() >= -7 and q.max() <= 7           # -8 is never produced
    # the element of largest magnitude of each scale group maps to +-qmax
    view = quant._group_view(v, gran, group)
    qv = quant._group_view(q.astype(np.float32), gran, group)
    idx = np.argmax(np.abs(view), axis=1)
    top = qv[np.arange(len(idx)), idx]
    assert np.all(np.abs(top) == 7)
    # half-step error bound (relative slack for the float32 products)
    sv = np.repeat(np.asarray(s).reshape(-1), view.shape[1]).reshape(view.shape)
    err = np.abs(view.astype(np.float64) - sv.astype(np.float64) * qv)
    assert np.all(err <= sv * 0.5 * (1 + 2 ** -20) + 1e-30)


def test_round_half_to_even_ties_constructed_exactly():
    # A = 7 * 2**-3 -> r = 7 / A = 8 exactly; v = (k + 1/2) / 8 -> v*r = k + 1/2 exactly.
    e = -3
    A = np.float32(7 * 2.0 ** e)
    ks = np.arange(-6, 6)
    v = np.concatenate([[A], ((ks + 0.5) * 2.0 ** e).astype(np.float32)]).astype(np.float32)
    q, s = quant.quantize_sym(v[None, :], 7, "row")
    got = q[0, 1:]
    expect = []
    for k in ks:
        lo, hi = k, k + 1
        expect.append(lo if lo % 2 == 0 else hi)        # tie -> even neighbour
    assert list(got) == expect
    assert s[0] == np.float32(2.0 ** e)


def test_product_rounded_to_float32_before_rint():
    # Find v with fl32(v*r) == 2.5 exactly while the exact product exceeds 2.5:
    # rounding the product first gives the tie -> 2; a fused multiply-add would give 3.
    # r < 1 makes consecutive v step the product by less than the rounding
    # window around 2.5, so such a v exists; float64 holds v*r exactly.
    A = np.float32(10.3)
    r = np.float32(np.float32(7) / A)
    v = np.float32(np.float32(2.5) / r)
    for _ in range(64):
        v = np.nextafter(v, np.float32(0))
    cand = None
    for _ in range(256):
        if np.float32(v * r) == np.float32(2.5) and float(v) * float(r) > 2.5:
            cand = v
            break
        v = np.nextafter(v, np.float32(10))
    assert cand is not None
    q, _ = quant.quantize_sym(np.array([[A, cand]], np.float32), 7, "row")
    assert q[0, 1] == 2


def test_zero_groups():
    v = np.zeros((2, 128), np.float32)
    v[1, 70] = 1.0
    q, s = quant.quantize_sym(v, 7, "row_group", 64)
    assert np.all(q[0] == 0) and np.all(s[0] == 0)
    assert s[1, 0] == 0 and s[1, 1] == np.float32(1.0) / np.float32(7)
    assert q[1, 70] == 7


def test_scale_multiplier_is_codes_neutral():
    # Quantizing the unnormalised rotation with the 1/16 carried by the scale
    # gives the same codes as quantizing the orthonormal rotation directly.
    g = np.random.default_rng(12)
    x = g.standard_normal((4, 512)).astype(np.float32)
    y = hadamard.rotate(x, 256)
    q1, s1 = quant.quantize_sym(y, 7, "row", scale_mul=1 / 16)
    q2, s2 = quant.quantize_sym((y * np.float32(1 / 16)).astype(np.float32), 7, "row")
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_unsigned_shift_path():
    shift = GOLD["post_gelu_shift"]["value"]
    assert shift == 0.171875
    g = np.random.default_rng(13)
    z = g.standard_normal((8, 128))
    from scipy.special import erf
    v = (z * 0.5 * (1 + erf(z / np.sqrt(2)))).astype(np.float32)     # GELU >= -0.17
    q, s = quant.quantize_unsigned_shift(v, shift, "row_group", 64)
    assert q.min() >= 0 and q.max() <= 15
    vs = (v + np.float32(shift)).reshape(8 * 2, 64)
    top = q.reshape(16, 64)[np.arange(16), np.argmax(vs, axis=1)]
    assert np.all(top == 15)
    # reconstruction s*q - shift approximates v within half a step
    rec = np.repeat(s.reshape(-1), 64).reshape(16, 64) * q.reshape(16, 64) - shift
    assert np.all(np.abs(rec - v.reshape(16, 64)) <= np.repeat(s.reshape(-1), 64).reshape(16, 64) * 0.5 * (1 + 2 ** -20))
    # a value below -shift clamps to code 0
    w = np.full((1, 64), 1.0, np.float32)
    w[0, 3] = -0.5
    q2, _ = quant.quantize_unsigned_shift(w, shift, "row_group", 64)
    assert q2[0, 3] == 0


def test_asym_g16():
    assert GOLD["w4a8_weight_group"]["value"] == 16
    g = np.random.default_rng(14)
    v = (g.standard_normal((8, 64)) * 0.3).astype(np.float32)
    v[1, :16] = 0.0                                 # constant (zero) group
    v[2, 16:32] = np.abs(v[2, 16:32]) + 0.1         # all-positive group: lo = 0
    q, s, z = quant.quantize_asym(v, 16)
    assert q.min() >= 0 and q.max() <= 15 and z.min() >= 0 and z.max() <= 15
    assert s.dtype == np.float16
    assert np.all(q[1, :16] == 0) and z[1, 0] == 0 and s[1, 0] == 1.0
    assert z[2, 1] == 0
    deq = quant.dequant_asym(q, s, z, 16)
    sf = np.repeat(s.astype(np.float64).reshape(-1), 16).reshape(8, 64)
    # every group's range [lo, hi] fits the grid, so the error is at most half
    # a step plus the z rounding (also half a step)
    assert np.all(np.abs(deq - v) <= sf * (1.0 + 1e-6))
    # zero is representable exactly: a 0.0 input dequantizes to 0.0
    v2 = v.copy()
    v2[0, 5] = 0.0
    q2, s2, z2 = quant.quantize_asym(v2, 16)
    assert quant.dequant_asym(q2, s2, z2, 16)[0, 5] == 0.0
