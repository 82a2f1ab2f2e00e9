"""Pins of oracle.pack and oracle.gemm.

[P5] Format fixes the natural container ([rows, cols/2] bytes holding signed
INT4); [P3] Tile-Packed Weight Format fixes the outer tiling (N/128, K/64)
of 32x128-byte tiles and the (N/128, K/64, 128) group-scale layout. The
integer GEMM is pinned against a pure-Python triple loop and numpy's int64
matmul (a library routine), independently of the float64-BLAS evaluation.
"""
import json
import os

import numpy as np
import pytest

from oracle import pack, gemm

HERE = os.path.dirname(__file__)
GOLD = json.load(open(os.path.join(HERE, "golden", "pages_facts.json")))


def _read_pack_example():
    codes, byts = {}, {}
    for line in open(os.path.join(HERE, "golden", "pack_int4_example.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, vals = line.split(":")
        kind, idx = key.split()
        if kind == "codes":
            codes[int(idx)] = [int(t) for t in vals.split()]
        else:
            byts[int(idx)] = [int(t, 16) for t in vals.split()]
    return (np.array([codes[0], codes[1]]), np.array([byts[0], byts[1]], dtype=np.uint8))


def test_pack_int4_hand_example():
    codes, expect = _read_pack_example()
    got = pack.pack_int4(codes)
    assert got.shape == (2, 4)                      # [rows, cols/2]
    assert np.array_equal(got, expect)
    assert np.array_equal(pack.unpack_int4(got, signed=True), codes)


def test_pack_round_trip_signed_and_unsigned():
    g = np.random.default_rng(20)
    s = g.integers(-8, 8, size=(5, 64))
    u = g.integers(0, 16, size=(5, 64))
    assert np.array_equal(pack.unpack_int4(pack.pack_int4(s), True), s)
    assert np.array_equal(pack.unpack_int4(pack.pack_int4(u), False), u)


def test_tile_pack_w4a4_shape_position_and_round_trip():
    shape = GOLD["tile_shape_bytes"]["value"]
    assert shape[2] * shape[3] == 4096
    g = np.random.default_rng(21)
    nat = g.integers(0, 256, size=(256, 128), dtype=np.uint8)          # N=256, K=256
    t = pack.tile_pack_w4a4(nat)
    assert t.shape == (256 // 128, 256 // 64, 4096)
    assert np.array_equal(pack.tile_unpack_w4a4(t), nat)
    # hand position check: natural (row 17, byte 9) of tile (0, 0):
    # row 17 -> n-block 1, lane%16 = 1; byte 9 -> chunk 1, j = 1 -> lane 17,
    # offset 1*512 + 17*8 + 1 = 649
    assert t[0, 0, 649] == nat[17, 9]
    # natural (row 128+5, byte 32*3 + 30) -> tile (1, 3): nb 0, lane 3*16+5 = 53, j 6
    assert t[1, 3, 53 * 8 + 6] == nat[133, 126]


def test_tile_pack_w4a8_position_and_round_trip():
    g = np.random.default_rng(22)
    vals = g.integers(0, 16, size=(128, 128)).astype(np.uint8)         # N=128, K=128
    t = pack.tile_pack_w4a8(vals)
    assert t.shape == (1, 2, 4096)
    assert np.array_equal(pack.tile_unpack_w4a8(t), vals)
    # code (row 70, k 64 + 16 + 8 + 2): k-tile 1, kg 1, lane half 1, i 2;
    # row 70 -> nb 2, lane 32 + 6 = 38; byte 1024 + 512 + 38*4 + 2, low nibble;
    # its high nibble is k + 4
    b = int(t[0, 1, 1024 + 512 + 152 + 2])
    assert b & 0xF == vals[70, 90] and b >> 4 == vals[70, 94]


def test_tile_pack_a_position_and_round_trip():
    g = np.random.default_rng(26)
    nat = g.integers(0, 256, size=(37, 128), dtype=np.uint8)           # M=37 (ragged), K=256
    t = pack.tile_pack_a(nat)
    assert t.shape == (3, 4, 512)
    assert np.array_equal(pack.tile_unpack_a(t, 37), nat)
    # natural (row 21, byte 32*2 + 19): block 1, k-tile 2, chunk 2, j 3 -> lane 2*16 + 5 = 37
    assert t[1, 2, 37 * 8 + 3] == nat[21, 83]
    assert np.all(t[2, :, :] [:, [l * 8 + j for l in range(64) if 32 + l % 16 >= 37 for j in range(8)]] == 0)


def test_group_scale_tiles():
    s = np.arange(256 * 8, dtype=np.float32).reshape(256, 8)      # N=256, K=512 (g64)
    t = pack.tile_pack_g64_scales(s)
    assert t.shape == (2, 8, 128)
    assert t[1, 5, 7] == s[128 + 7, 5]
    z = np.arange(128 * 16).reshape(128, 16)                        # N=128, K=256 (g16)
    tz = pack.tile_pack_g16(z)
    assert tz.shape == (1, 4, 4, 128)
    assert tz[0, 2, 3, 9] == z[9, 11]


def test_lora_up_tiles():
    """[N/128][R][128]: one 128-channel block's rank vectors are R runs of
    128 contiguous channels (positions worked out by hand)."""
    up = np.arange(256 * 32, dtype=np.int64).reshape(256, 32)       # N=256, R=32: up[n, r] = 32 n + r
    t = pack.tile_pack_lora_up(up)
    assert t.shape == (2, 32, 128)
    flat = t.reshape(-1)
    assert flat[0] == 0 and flat[1] == 32 and flat[127] == 127 * 32      # r = 0 of channels 0..127
    assert flat[128] == 1                                                 # r = 1 of channel 0
    assert flat[32 * 128] == 128 * 32                                     # block 1 starts at channel 128
    assert flat[32 * 128 + 5 * 128 + 7] == (128 + 7) * 32 + 5            # channel 135, r = 5
    assert np.array_equal(np.sort(flat), np.arange(256 * 32))


def _triple_loop(a, b):
    M, K = len(a), len(a[0])
    N = len(b)
    return [[sum(int(a[m][k]) * int(b[n][k]) for k in range(K)) for n in range(N)] for m in range(M)]


def test_int_gemm_vs_triple_loop():
    g = np.random.default_rng(23)
    a = g.integers(-7, 8, size=(3, 40))
    b = g.integers(-7, 8, size=(5, 40))
    assert np.array_equal(gemm.int_gemm(a, b), np.array(_triple_loop(a.tolist(), b.tolist())))


def test_int_gemm_vs_numpy_int64():
    g = np.random.default_rng(24)
    a = g.integers(-127, 128, size=(33, 3072))
    b = g.integers(-127, 128, size=(70, 3072))
    assert np.array_equal(gemm.int_gemm(a, b), a.astype(np.int64) @ b.astype(np.int64).T)


def test_group_partials_sum_and_zero_points():
    g = np.random.default_rng(25)
    a = g.integers(-127, 128, size=(4, 64))
    w = g.integers(0, 16, size=(6, 64))
    z = g.integers(0, 16, size=(6, 4))
    P = gemm.group_partials(a, w, 16, z)
    assert P.shape == (4, 6, 4)
    wz = w - np.repeat(z, 16, axis=1)
    assert np.array_equal(P.sum(axis=2), a @ wz.T)
    # one entry by hand-level brute force
    m, n, gg = 2, 3, 1
    assert P[m, n, gg] == sum(int(a[m, k]) * (int(w[n, k]) - int(z[n, gg])) for k in range(16, 32))


def test_exactness_bound_guard():
    a = np.full((1, 8), 2 ** 26, dtype=np.int64)
    with pytest.raises(ValueError):
        gemm.int_gemm(a, a)


# ---------------------------------------------------------------------------
# fp6 E2M3 fragments (operand format of the fp6 matrix-core GEMM). Pins: the
# constants the OCP Microscaling FP6 (E2M3) definition fixes, and byte
# positions derived by hand from the layout definition.
# ---------------------------------------------------------------------------
def test_e2m3_format_constants():
    v = pack.e2m3_value
    assert v(0b011111) == 7.5          # largest normal: 2^2 * 1.875
    assert v(0b001000) == 1.0          # smallest normal
    assert v(0b000111) == 0.875        # largest subnormal
    assert v(0b000001) == 0.125        # smallest subnormal
    assert v(0b111111) == -7.5
    assert v(0b100000) == 0.0 and np.signbit(v(0b100000))
    vals = v(np.arange(64))
    assert len(set(vals.tolist())) == 63   # only +0 / -0 coincide
    assert np.all(np.diff(vals[:32]) > 0)  # codes 0..31 increase with their value


def test_e2m3_codes_of_int4_round_trip():
    q = np.arange(-7, 8)
    c = pack.e2m3_code_of_int(q)
    assert np.array_equal(pack.e2m3_value(c), q)
    assert c[7] == 0 and c.max() < 64      # zero as +0
    # by hand: 3 = 2^1 * 1.5 (e = 2, m = 4), 5 = 2^2 * 1.25 (e = 3, m = 2), -1 = sign | e = 1
    assert c[q.tolist().index(3)] == 0b010100
    assert c[q.tolist().index(5)] == 0b011010
    assert c[q.tolist().index(-1)] == 0b101000
    for bad in (8, -8):
        with pytest.raises(ValueError):
            pack.e2m3_code_of_int(np.array([bad]))


def test_f6_fragment_positions_by_hand():
    rows, K = 40, 128
    c = np.zeros((rows, K), dtype=np.int64)
    c[0, 0] = 1        # block 0, k-tile 0, lane 0, field 0 -> byte 0 bits 0..5
    c[33, 127] = -7    # block 1, k-tile 1, lane 32 + 1 = 33, field 31 -> lane byte 23 bits 2..7
    c[5, 70] = 3       # block 0, k-tile 1, lane 5, field 6 -> lane bits 36..41 = byte 4 bits 4..7, byte 5 bits 0..1
    fr = pack.f6_pack(c)
    assert fr.shape == (2, 2, 1536)
    nz = {(int(b), int(t), int(o)): int(fr[b, t, o]) for b, t, o in zip(*np.nonzero(fr))}
    assert nz == {(0, 0, 0): 0b001000,
                  (1, 1, 1024 + 33 * 8 + 7): 0b111110 << 2,
                  (0, 1, 5 * 16 + 4): (0b010100 << 4) & 0xFF,
                  (0, 1, 5 * 16 + 5): 0b010100 >> 4}
    assert np.array_equal(pack.f6_unpack(fr, rows), c)


def test_f6_round_trip_and_dot_products():
    rng = np.random.default_rng(11)
    a = rng.integers(-7, 8, size=(45, 192))
    w = rng.integers(-7, 8, size=(64, 192))
    av, wv = pack.f6_unpack(pack.f6_pack(a), 45), pack.f6_unpack(pack.f6_pack(w), 64)
    assert np.array_equal(av, a) and np.array_equal(wv, w)
    assert np.array_equal((av @ wv.T).astype(np.int64), gemm.int_gemm(a, w))


def test_e2m3_codes_of_unsigned_halves():
    u = np.arange(16)
    c = pack.e2m3_code_of_half(u)
    assert np.array_equal(pack.e2m3_value(c) * 2, u)
    assert c[1] == 0b000100          # 0.5 = subnormal 4/8
    assert c[15] == 0b011111         # 7.5 = 2^2 * 1.875, the largest normal
    assert c[3] == 0b001100          # 1.5 = 2^0 * 1.5
    for bad in (-1, 16):
        with pytest.raises(ValueError):
            pack.e2m3_code_of_half(np.array([bad]))
    rng = np.random.default_rng(12)
    a = rng.integers(0, 16, size=(40, 128))
    w = rng.integers(-7, 8, size=(64, 128))
    av = pack.f6_unpack(pack.f6_pack(a, unsigned=True), 40)
    assert np.array_equal(av * 2, a)
    assert np.array_equal((2 * av @ pack.f6_unpack(pack.f6_pack(w), 64).T).astype(np.int64), gemm.int_gemm(a, w))
