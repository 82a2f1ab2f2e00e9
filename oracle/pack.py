"""Int4 packing: the natural two-per-byte layout and the tile-packed layouts.

Sources:
  [P5] Format: a quantized layer stores its weight as an INT8 container of
       shape [rows, cols/2] holding signed INT4 values.
  [P1] intro: packed signed INT4 weights, two per byte.
  [P3] Key Technical Optimizations, tile-packed weight format: weights are
       reorganised from the natural layout into tiles of 128 output rows by
       64 input channels, (N/128, K/64, 32, 128) bytes, with group scales laid
       out (N/128, K/64, 128).

Readings where the pages are silent:
  * nibble order: byte j of a row holds element 2j in its low nibble and
    element 2j+1 in its high nibble, each as a 4-bit two's-complement value
    (unsigned 0..15 for unsigned / asymmetric codes);
  * the outer tiling is the pages' [N/128][K/64] grid of 4096-byte tiles; the
    byte order INSIDE a tile is this project's own choice, made so that one
    64-lane matrix-core operand fragment is 512 (or 256) contiguous bytes:

    W4A4 tile (symmetric int4, k-chunks of 16 values):
        tile byte  nb*512 + l*8 + j,  nb in [0,8), l in [0,64), j in [0,8)
        <- natural byte (row 16*nb + l%16 of the tile, byte 8*(l//16) + j of
           the tile's 32-byte k slice)
    W4A8 tile (asymmetric uint4, k-groups of 16):
        tile byte  kg*1024 + nb*256 + l*4 + i,  kg, nb in [0,4), l in [0,64), i in [0,4)
        = code (row, k0+i) | code (row, k0+4+i) << 4, row 32*nb + l%32 of the
          tile, k0 = 16*kg + 8*(l//32) in the tile (so a lane's low nibbles
          are 4 consecutive k and its high nibbles the next 4)

  * activation codes may also be stored tiled: [ceil(M/16)][K/64][512 B],
    byte l*8 + j <- natural byte (row 16*b + l%16, byte 8*(l//16) + j of the
    32-byte k-tile slice), i.e. the weight tile's fragment order;
  * per-group scales of the W4A4 g64 format: float32 [N/128][K/64][128]
    (the pages' wscales layout); W4A8 g16 scales (fp16) and zero points
    (one byte each) : [N/128][K/64][4][128].
  * the low-rank up-projection L1 [N, R] (bf16) in the pages' tiled layout
    [N/128][R][128]: for every block of 128 output channels, rank index r
    major and the 128 channels contiguous.
"""
from __future__ import annotations

import numpy as np


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """codes int [rows, K] (signed in [-8,7] or unsigned in [0,15]) -> uint8 [rows, K/2]."""
    c = np.asarray(codes).astype(np.int64)
    rows, K = c.shape
    if K % 2:
        raise ValueError("K must be even")
    lo = c[:, 0::2] & 0xF
    hi = c[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray, signed: bool = True) -> np.ndarray:
    """uint8 [rows, K/2] -> int8/uint8 [rows, K] (inverse of pack_int4)."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    rows, half = p.shape
    out = np.empty((rows, 2 * half), dtype=np.int64)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = (p >> 4) & 0xF
    if signed:
        out = np.where(out >= 8, out - 16, out)
        return out.astype(np.int8)
    return out.astype(np.uint8)


def _check_tiles(N: int, K: int):
    if N % 128 or K % 64:
        raise ValueError("tile packing needs N % 128 == 0 and K % 64 == 0")


def tile_pack_w4a4(packed: np.ndarray) -> np.ndarray:
    """natural uint8 [N, K/2] -> tile-packed uint8 [N/128, K/64, 4096]."""
    packed = np.asarray(packed, dtype=np.uint8)
    N, half = packed.shape
    K = 2 * half
    _check_tiles(N, K)
    out = np.empty((N // 128, K // 64, 4096), dtype=np.uint8)
    for tn in range(N // 128):
        for kt in range(K // 64):
            tile = packed[128 * tn:128 * tn + 128, 32 * kt:32 * kt + 32]   # [128 rows, 32 bytes]
            for nb in range(8):
                for lane in range(64):
                    row = 16 * nb + lane % 16
                    col = 8 * (lane // 16)
                    o = nb * 512 + lane * 8
                    out[tn, kt, o:o + 8] = tile[row, col:col + 8]
    return out


def tile_unpack_w4a4(tiles: np.ndarray) -> np.ndarray:
    """Inverse of tile_pack_w4a4."""
    tiles = np.asarray(tiles, dtype=np.uint8)
    TN, TK, _ = tiles.shape
    out = np.empty((TN * 128, TK * 32), dtype=np.uint8)
    for tn in range(TN):
        for kt in range(TK):
            for nb in range(8):
                for lane in range(64):
                    row = 128 * tn + 16 * nb + lane % 16
                    col = 32 * kt + 8 * (lane // 16)
                    o = nb * 512 + lane * 8
                    out[row, col:col + 8] = tiles[tn, kt, o:o + 8]
    return out


def tile_pack_w4a8(values: np.ndarray) -> np.ndarray:
    """uint4 codes [N, K] (values 0..15) -> tile-packed uint8 [N/128, K/64, 4096].
    Byte kg*1024 + nb*256 + lane*4 + i of tile (tn, kt) holds code
    (row, k0 + i) in its low nibble and (row, k0 + 4 + i) in its high nibble,
    with row = 128*tn + 32*nb + lane%32 and k0 = 64*kt + 16*kg + 8*(lane//32)."""
    v = np.asarray(values).astype(np.int64)
    N, K = v.shape
    _check_tiles(N, K)
    out = np.empty((N // 128, K // 64, 4096), dtype=np.uint8)
    for tn in range(N // 128):
        for kt in range(K // 64):
            for kg in range(4):
                for nb in range(4):
                    for lane in range(64):
                        row = 128 * tn + 32 * nb + lane % 32
                        k0 = 64 * kt + 16 * kg + 8 * (lane // 32)
                        o = kg * 1024 + nb * 256 + lane * 4
                        for i in range(4):
                            out[tn, kt, o + i] = (v[row, k0 + i] & 0xF) | ((v[row, k0 + 4 + i] & 0xF) << 4)
    return out


def tile_unpack_w4a8(tiles: np.ndarray) -> np.ndarray:
    """Inverse of tile_pack_w4a8: uint8 codes [N, K]."""
    tiles = np.asarray(tiles, dtype=np.uint8)
    TN, TK, _ = tiles.shape
    out = np.empty((TN * 128, TK * 64), dtype=np.uint8)
    for tn in range(TN):
        for kt in range(TK):
            for kg in range(4):
                for nb in range(4):
                    for lane in range(64):
                        row = 128 * tn + 32 * nb + lane % 32
                        k0 = 64 * kt + 16 * kg + 8 * (lane // 32)
                        o = kg * 1024 + nb * 256 + lane * 4
                        for i in range(4):
                            b = int(tiles[tn, kt, o + i])
                            out[row, k0 + i] = b & 0xF
                            out[row, k0 + 4 + i] = b >> 4
    return out


def tile_pack_a(packed: np.ndarray) -> np.ndarray:
    """Activation codes, natural uint8 [M, K/2] -> tiled uint8 [ceil(M/16), K/64, 512]:
    byte l*8 + j of block (b, kt) <- natural byte (row 16*b + l%16, 32*kt + 8*(l//16) + j),
    the 16-row analogue of the W4A4 weight tile (one operand fragment per
    512 bytes). Rows past M in the last block are zero here (the library
    leaves them unwritten)."""
    packed = np.asarray(packed, dtype=np.uint8)
    M, half = packed.shape
    K = 2 * half
    if K % 64:
        raise ValueError("K % 64 != 0")
    MB = (M + 15) // 16
    out = np.zeros((MB, K // 64, 512), dtype=np.uint8)
    for b in range(MB):
        for kt in range(K // 64):
            for lane in range(64):
                row = 16 * b + lane % 16
                if row >= M:
                    continue
                col = 32 * kt + 8 * (lane // 16)
                out[b, kt, lane * 8:lane * 8 + 8] = packed[row, col:col + 8]
    return out


def tile_unpack_a(tiles: np.ndarray, M: int) -> np.ndarray:
    """Inverse of tile_pack_a (first M rows)."""
    tiles = np.asarray(tiles, dtype=np.uint8)
    MB, KT, _ = tiles.shape
    out = np.zeros((MB * 16, KT * 32), dtype=np.uint8)
    for b in range(MB):
        for kt in range(KT):
            for lane in range(64):
                row = 16 * b + lane % 16
                col = 32 * kt + 8 * (lane // 16)
                out[row, col:col + 8] = tiles[b, kt, lane * 8:lane * 8 + 8]
    return out[:M]


def tile_pack_g64_scales(scales: np.ndarray) -> np.ndarray:
    """float32 [N, K/64] -> [N/128, K/64, 128]: element (tn, kt, i) is the
    scale of row 128*tn + i for k-group kt."""
    s = np.asarray(scales, dtype=np.float32)
    N, G = s.shape
    return np.ascontiguousarray(s.reshape(N // 128, 128, G).transpose(0, 2, 1))


def tile_pack_g16(per_group: np.ndarray) -> np.ndarray:
    """[N, K/16] per-(row, 16-group) values -> [N/128, K/64, 4, 128]:
    element (tn, kt, kg, i) belongs to row 128*tn + i and group 4*kt + kg."""
    a = np.asarray(per_group)
    N, G = a.shape
    return np.ascontiguousarray(a.reshape(N // 128, 128, G // 4, 4).transpose(0, 2, 3, 1))


def tile_pack_lora_up(up: np.ndarray) -> np.ndarray:
    """L1 [N, R] -> [N/128, R, 128] ([P3] Tile-Packed Weight Format, LoRA-up):
    element (tn, r, i) is L1[128*tn + i, r]."""
    a = np.asarray(up)
    N, R = a.shape
    return np.ascontiguousarray(a.reshape(N // 128, 128, R).transpose(0, 2, 1))


def pack_zeros_u4(zeros: np.ndarray) -> np.ndarray:
    """uint4 zero points [N, K/16] -> natural two-per-byte [N, K/32]."""
    return pack_int4(zeros.astype(np.int64))


# ---------------------------------------------------------------------------
# fp6 E2M3 fragments: the operand layout of the fp6 matrix-core W4A4 GEMM.
#
# Not from the pages: E2M3 is the OCP Microscaling (MX) FP6 format -- sign bit
# 5, exponent bits 4:3 with bias 1, mantissa bits 2:0; a normal value
# (e >= 1) is (-1)^s 2^(e-1) (1 + m/8), a subnormal (e = 0) is (-1)^s m/8, and
# there is no Inf or NaN. Every integer in [-7, 7] (a symmetric INT4 code) is
# an E2M3 value, so the format carries the codes exactly.
#
# Layout (this project's choice, one 64-lane operand fragment of the
# 32x32x64 matrix-core instruction per 1536 bytes): [ceil(rows/32)][K/64][1536 B];
# lane l of fragment (b, kt) holds row 32b + l%32 and columns
# 64kt + 32(l//32) + i, i = 0..31, as 32 six-bit fields, field i at bits
# 6i..6i+5 of a 24-byte little-endian string; bytes 0..15 of it are stored at
# l*16, bytes 16..23 at 1024 + l*8. Rows past `rows` are zero here (the
# library leaves them unwritten).
# ---------------------------------------------------------------------------
def e2m3_value(code) -> np.ndarray:
    """The real value of E2M3 codes (uint, 0..63), by the format's definition."""
    c = np.asarray(code).astype(np.int64)
    s = np.where((c >> 5) & 1, -1.0, 1.0)
    e = (c >> 3) & 3
    m = c & 7
    mag = np.where(e == 0, m / 8.0, np.ldexp(1.0 + m / 8.0, e - 1))
    return s * mag


def e2m3_code_of_int(q) -> np.ndarray:
    """The E2M3 code of integers in [-7, 7] (zero as +0)."""
    q = np.asarray(q).astype(np.int64)
    if np.any(np.abs(q) > 7):
        raise ValueError("integer outside [-7, 7] has no exact E2M3 code")
    a = np.abs(q)
    e = np.zeros_like(a)
    nz = a > 0
    e[nz] = np.floor(np.log2(a[nz])).astype(np.int64) + 1      # a = 2^(e-1) (1 + m/8)
    m = np.zeros_like(a)
    m[nz] = (a[nz] * 8) // (1 << (e[nz] - 1)) - 8
    code = (e << 3) | m
    return np.where(q < 0, code | 32, code).astype(np.uint8)


def e2m3_code_of_half(u) -> np.ndarray:
    """The E2M3 code of u/2 for unsigned codes u in [0, 15]: every half-integer
    0, 0.5, ..., 7.5 is an E2M3 value (0.5 a subnormal, 7.5 the largest normal)."""
    u = np.asarray(u).astype(np.int64)
    if np.any((u < 0) | (u > 15)):
        raise ValueError("unsigned code outside [0, 15]")
    out = np.zeros(u.shape, dtype=np.uint8)
    for code in range(32):                     # the non-negative codes, by value
        v = e2m3_value(code)
        hit = (u == int(round(2 * v))) & (2 * v == np.round(2 * v))
        out[hit & (out == 0)] = code
    return out


def f6_pack(codes: np.ndarray, unsigned: bool = False) -> np.ndarray:
    """Int4 codes int [rows, K] -> uint8 [ceil(rows/32), K/64, 1536] fp6
    E2M3 fragments (layout above). Signed codes (values in [-7, 7]) are
    stored as themselves; unsigned codes u in [0, 15] (the shifted post-GELU
    path) as the E2M3 value u/2, so a product sum over them is half the
    integer one (exact)."""
    c = np.asarray(codes).astype(np.int64)
    rows, K = c.shape
    if K % 64:
        raise ValueError("K % 64 != 0")
    MB, KT = (rows + 31) // 32, K // 64
    f = np.zeros((MB * 32, K), dtype=np.int64)
    f[:rows] = e2m3_code_of_half(c) if unsigned else e2m3_code_of_int(c)
    # [b, r, kt, h, i] -> [b, kt, lane = 32 h + r, i]
    f = f.reshape(MB, 32, KT, 2, 32).transpose(0, 2, 3, 1, 4).reshape(MB, KT, 64, 32)
    # four 6-bit fields -> three bytes, little-endian
    g = f.reshape(MB, KT, 64, 8, 4)
    v = g[..., 0] | (g[..., 1] << 6) | (g[..., 2] << 12) | (g[..., 3] << 18)
    lane_bytes = np.stack([v & 0xFF, (v >> 8) & 0xFF, (v >> 16) & 0xFF], axis=-1).reshape(MB, KT, 64, 24)
    out = np.zeros((MB, KT, 1536), dtype=np.uint8)
    out[:, :, :1024] = lane_bytes[..., :16].reshape(MB, KT, 1024)
    out[:, :, 1024:] = lane_bytes[..., 16:].reshape(MB, KT, 512)
    return out


def f6_unpack(frags: np.ndarray, rows: int) -> np.ndarray:
    """Inverse of f6_pack: uint8 [MB, K/64, 1536] -> the real values of the
    first `rows` rows, float64 [rows, K] (the signed codes, or u/2 for
    unsigned codes)."""
    fr = np.asarray(frags, dtype=np.uint8)
    MB, KT, _ = fr.shape
    lane_bytes = np.concatenate([fr[:, :, :1024].reshape(MB, KT, 64, 16),
                                 fr[:, :, 1024:].reshape(MB, KT, 64, 8)], axis=-1).astype(np.int64)
    t = lane_bytes.reshape(MB, KT, 64, 8, 3)
    v = t[..., 0] | (t[..., 1] << 8) | (t[..., 2] << 16)
    f = np.stack([(v >> (6 * j)) & 63 for j in range(4)], axis=-1).reshape(MB, KT, 64, 32)
    val = e2m3_value(f).reshape(MB, KT, 2, 32, 32).transpose(0, 3, 1, 2, 4).reshape(MB * 32, KT * 64)
    return val[:rows]
