"""Host-side byte layouts of the library's operands, written from their
definitions in include/w4a4.h (test helpers: pure permutations, no
arithmetic of the layer)."""
import numpy as np


def pad16(n):
    return (n + 15) // 16 * 16


def i8_from_codes(q):
    """Codes [M, K] -> the W4A4_CODES_I8 byte layout: inside every group of 8
    channels, channels 0,2,4,6 then 1,3,5,7 (the documented order)."""
    M, K = q.shape
    g = q.reshape(M, K // 8, 8)
    return np.concatenate([g[:, :, 0::2], g[:, :, 1::2]], axis=2).reshape(M, K).astype(np.int8)


def codes_from_i8(b):
    M, K = b.shape
    g = b.view(np.int8).reshape(M, K // 8, 8)
    out = np.empty_like(g)
    out[:, :, 0::2] = g[:, :, :4]
    out[:, :, 1::2] = g[:, :, 4:]
    return out.reshape(M, K)


def tile_codes_i8(i8, rng=None):
    """[M, K] W4A4_CODES_I8 bytes -> W4A4_CODES_I8_TILED ([pad16(M), K]):
    tile (blk, t) holds, at ((4h + g) 16 + r) 16, codes [128t + 32g + 16h,
    +16) of row 16 blk + r.  Padding rows get random bytes."""
    M, K = i8.shape
    Mp = pad16(M)
    full = np.empty((Mp, K), np.uint8)
    full[:M] = i8.view(np.uint8)
    full[M:] = (rng or np.random.default_rng(0)).integers(0, 256, (Mp - M, K), dtype=np.uint8)
    t = full.reshape(Mp // 16, 16, K // 128, 4, 2, 16).transpose(0, 2, 4, 3, 1, 5)
    return np.ascontiguousarray(t).reshape(Mp, K)


def untile_codes_i8(tiled, M):
    Mp, K = tiled.shape
    t = tiled.reshape(Mp // 16, K // 128, 2, 4, 16, 16).transpose(0, 4, 1, 3, 2, 5)
    return np.ascontiguousarray(t).reshape(Mp, K)[:M]


def tile_weights(packed, rng=None):
    """[N, K/2] packed codes -> W4A4_WEIGHTS_TILED ([pad16(N), K/2]): tile
    (blk, t) holds, at (16g + r) 16, bytes [64t + 16g, +16) of row 16 blk + r."""
    N, H = packed.shape
    Np = pad16(N)
    full = np.empty((Np, H), np.uint8)
    full[:N] = packed
    full[N:] = (rng or np.random.default_rng(1)).integers(0, 256, (Np - N, H), dtype=np.uint8)
    t = full.reshape(Np // 16, 16, H // 64, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(t).reshape(Np, H)


def untile_weights(tiled, N):
    Np, H = tiled.shape
    t = tiled.reshape(Np // 16, H // 64, 4, 16, 16).transpose(0, 3, 1, 2, 4)
    return np.ascontiguousarray(t).reshape(Np, H)[:N]


def tile_weights_residual(packed, packed_res, rng=None):
    """Residual-extended tiled weights: every 16-row block holds the K/128
    tiles of packed [N, K/2] followed by the r_pad/128 tiles of packed_res
    [N, r_pad/2], each in the W4A4_WEIGHTS_TILED tile layout."""
    main = tile_weights(packed, rng)
    res = tile_weights(packed_res, rng)
    Np = main.shape[0]
    m = main.reshape(Np // 16, -1, 1024)
    r = res.reshape(Np // 16, -1, 1024)
    return np.ascontiguousarray(np.concatenate([m, r], axis=1)).reshape(Np, -1)


def untile_weights_residual(ext, N, K):
    """Inverse of tile_weights_residual: (packed [N, K/2], packed_res [N, r_pad/2])."""
    Np, H = ext.shape
    t = ext.reshape(Np // 16, H // 64, 1024)
    nk = K // 128
    main = np.ascontiguousarray(t[:, :nk]).reshape(Np, K // 2)
    res = np.ascontiguousarray(t[:, nk:]).reshape(Np, H - K // 2)
    return untile_weights(main, N), untile_weights(res, N)


def tile_mx_scales(s, rng=None):
    """[M, K/32] E8M0 bytes -> the tiled scale array: byte (g 16 + r) of the
    64-byte tile (b, t) is the scale of block 4 t + g of row 16 b + r.
    Padding rows get random bytes."""
    M, KB = s.shape
    Mp = pad16(M)
    full = np.empty((Mp, KB), np.uint8)
    full[:M] = s
    full[M:] = (rng or np.random.default_rng(2)).integers(0, 256, (Mp - M, KB), dtype=np.uint8)
    t = full.reshape(Mp // 16, 16, KB // 4, 4).transpose(0, 2, 3, 1)
    return np.ascontiguousarray(t).reshape(-1)


def untile_mx_scales(flat, M, K):
    Mp = pad16(M)
    t = np.asarray(flat)[:Mp * K // 32].reshape(Mp // 16, K // 128, 4, 16).transpose(0, 3, 1, 2)
    return np.ascontiguousarray(t).reshape(Mp, K // 32)[:M]


def ob_weights(tiled, N, K):
    """W4A4_WEIGHTS_TILED bytes [pad16(N), K/2] -> the flat
    W4A4_WEIGHTS_TILED_OB buffer: every byte with its nibbles swapped and the
    new low nibble XOR 8, then one int32 per padded row, the sum of the row's
    codes at even channels (0 for padding rows here)."""
    t = np.asarray(tiled, np.uint8)
    conv = (((t & 0x0F) << 4) | (((t >> 4) & 0x0F) ^ 0x08)).astype(np.uint8)
    lo = (untile_weights(t, N) & 0x0F).astype(np.int32)
    sums = np.zeros(pad16(N), np.int32)
    sums[:N] = np.where(lo >= 8, lo - 16, lo).sum(axis=1)
    return np.concatenate([conv.reshape(-1), sums.view(np.uint8)])


def ob_codes(tiled, M, K):
    """W4A4_CODES_PACKED_TILED bytes [pad16(M), K/2] -> the flat
    W4A4_CODES_PACKED_TILED_OB buffer: every byte XOR 0x08, then one int32
    per padded row, the sum of the row's codes at odd channels."""
    t = np.asarray(tiled, np.uint8)
    hi = (untile_weights(t, M) >> 4).astype(np.int32)
    sums = np.zeros(pad16(M), np.int32)
    sums[:M] = np.where(hi >= 8, hi - 16, hi).sum(axis=1)
    return np.concatenate([(t ^ 0x08).reshape(-1), sums.view(np.uint8)])


def split_ob(flat, rows, K):
    """Flat offset-binary buffer -> (tile bytes [pad16(rows), K/2], int32 sums [rows])."""
    Rp = pad16(rows)
    nb = Rp * (K // 2)
    return flat[:nb].reshape(Rp, K // 2), flat[nb:nb + 4 * Rp].view(np.int32)[:rows]


# FP6 E2M3 (OCP microscaling formats): sign bit 5, exponent bits 4:3 with
# bias 1, mantissa bits 2:0; exponent 0 is subnormal (m / 8).
def e2m3_value(c):
    """Value of each 6-bit E2M3 code (any of the 64)."""
    c = np.asarray(c, np.int64)
    e, m = (c >> 3) & 3, (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0, (1.0 + m / 8.0) * np.exp2(e - 1.0))
    return np.where(c & 32, -mag, mag)


def e2m3_code(q):
    """The E2M3 code of each integer q in [-7, 7] (0 as +0), found by search
    over the 32 non-negative codes."""
    q = np.asarray(q, np.int64)
    table = {int(v): c for c, v in enumerate(e2m3_value(np.arange(32))) if float(v).is_integer()}
    mag = np.vectorize(lambda a: table[int(a)])(np.abs(q)) if q.size else np.zeros(q.shape, np.int64)
    return np.where(q < 0, mag | 32, mag).astype(np.uint8)


def _f6_lane_fields(codes32):
    """[..., 32] codes of one instruction lane -> [..., 32] fields in field
    order: field 2u is code u, field 2u + 1 code 16 + u."""
    f = np.empty_like(codes32)
    f[..., 0::2] = codes32[..., :16]
    f[..., 1::2] = codes32[..., 16:]
    return f


def _fields_to_lane_bytes(fields):
    """[..., 32] 6-bit fields -> [..., 24] bytes: field p at bits [6p, 6p + 6)
    of the lane's 192-bit little-endian value (three 64-bit words)."""
    f = fields.astype(np.uint64)
    words = np.zeros(f.shape[:-1] + (3,), np.uint64)
    for p in range(32):
        bit = 6 * p
        w, off = bit // 64, bit % 64
        words[..., w] |= (f[..., p] << np.uint64(off)) & np.uint64(0xFFFFFFFFFFFFFFFF)
        if off > 58:   # the field continues in the next word
            words[..., w + 1] |= f[..., p] >> np.uint64(64 - off)
    return words.astype("<u8").view(np.uint8).reshape(f.shape[:-1] + (24,))


def _lane_bytes_to_fields(lane_bytes):
    """Inverse of _fields_to_lane_bytes: [..., 24] bytes -> [..., 32] fields."""
    words = np.ascontiguousarray(lane_bytes).view("<u8").astype(np.uint64)
    out = np.empty(words.shape[:-1] + (32,), np.uint8)
    for p in range(32):
        bit = 6 * p
        w, off = bit // 64, bit % 64
        v = words[..., w] >> np.uint64(off)
        if off > 58:
            v |= words[..., w + 1] << np.uint64(64 - off)
        out[..., p] = (v & np.uint64(63)).astype(np.uint8)
    return out


def tile_f6(q, rng=None):
    """Codes [R, K] in [-7, 7] -> the FP6 tiled layout [pad16(R), 3K/4]
    (W4A4_CODES_F6_TILED / W4A4_WEIGHTS_TILED_F6).  Padding rows get random
    6-bit codes."""
    R, K = q.shape
    Rp = pad16(R)
    c = np.empty((Rp, K), np.uint8)
    c[:R] = e2m3_code(q)
    c[R:] = (rng or np.random.default_rng(3)).integers(0, 64, (Rp - R, K), dtype=np.uint8)
    # [blk, r, t, g, 32] -> [blk, t, g, r, 32] = tile (blk, t), lane 16 g + r
    lanes = c.reshape(Rp // 16, 16, K // 128, 4, 32).transpose(0, 2, 3, 1, 4)
    fields = _f6_lane_fields(lanes.reshape(Rp // 16, K // 128, 64, 32))
    lane_bytes = _fields_to_lane_bytes(fields)
    tile = np.concatenate([lane_bytes[..., :16].reshape(Rp // 16, K // 128, 1024),
                           lane_bytes[..., 16:].reshape(Rp // 16, K // 128, 512)], axis=-1)
    return np.ascontiguousarray(tile).reshape(Rp, 3 * K // 4)


def untile_f6_codes(tiled, R, K):
    """FP6 tiled bytes [pad16(R), 3K/4] -> the 6-bit codes [R, K] row-major."""
    Rp = pad16(R)
    t = np.asarray(tiled, np.uint8).reshape(Rp // 16, K // 128, 1536)
    lane_bytes = np.concatenate([t[..., :1024].reshape(Rp // 16, K // 128, 64, 16),
                                 t[..., 1024:].reshape(Rp // 16, K // 128, 64, 8)], axis=-1)
    fields = _lane_bytes_to_fields(lane_bytes)
    codes32 = np.concatenate([fields[..., 0::2], fields[..., 1::2]], axis=-1)
    c = codes32.reshape(Rp // 16, K // 128, 4, 16, 32).transpose(0, 3, 1, 2, 4)
    return np.ascontiguousarray(c).reshape(Rp, K)[:R]


def untile_f6(tiled, R, K):
    """FP6 tiled bytes -> the integer codes [R, K] (int8); every code must be
    an integer in [-7, 7]."""
    v = e2m3_value(np.arange(64))
    ok = (v == np.round(v)) & (np.abs(v) <= 7)
    table = np.where(ok, v, 99).astype(np.int8)   # 99: not a code
    q = table[untile_f6_codes(tiled, R, K)]
    assert not np.any(q == 99)
    return q


def workspace_codes(ws, off, M, K, layout):
    """The activation codes a layer call left in its workspace (flat uint8
    bytes, codes at byte offset `off`, stored in `layout`), rearranged row-major:
    ("packed", [M, K/2] uint8 packed bytes) or ("i8", [M, K] int8 codes; FP6
    tiles are decoded to their integer values)."""
    ws = np.asarray(ws, np.uint8)
    Mp = pad16(M)
    if layout in ("packed_tiled", "packed_tiled_ob"):
        t = ws[off:off + Mp * (K // 2)].reshape(Mp, K // 2)
        if layout == "packed_tiled_ob":
            t = t ^ 0x08
        return "packed", untile_weights(t, M)
    if layout == "packed":
        return "packed", ws[off:off + M * (K // 2)].reshape(M, K // 2)
    if layout == "i8":
        return "i8", codes_from_i8(ws[off:off + M * K].reshape(M, K))
    if layout == "i8_tiled":
        return "i8", codes_from_i8(untile_codes_i8(ws[off:off + Mp * K].reshape(Mp, K), M))
    if layout == "f6_tiled":
        return "i8", untile_f6(ws[off:off + Mp * (3 * K // 4)].reshape(Mp, 3 * K // 4), M, K)
    raise ValueError(layout)
