"""The layout helpers the GPU parity tests use are inverse permutations and
put bytes where include/w4a4.h says they go."""
import numpy as np

from layouts import (codes_from_i8, i8_from_codes, tile_codes_i8, tile_weights, untile_codes_i8,
                     tile_weights_residual, untile_weights_residual, tile_mx_scales,
                     untile_mx_scales, ob_codes, ob_weights, split_ob,
                     untile_weights)
from oracle import w4a4_oracle as O


def test_i8_order_is_even_then_odd_channels():
    q = np.arange(16, dtype=np.int8).reshape(1, 16) - 8
    b = i8_from_codes(q)
    assert b[0].tolist() == [-8, -6, -4, -2, -7, -5, -3, -1, 0, 2, 4, 6, 1, 3, 5, 7]
    assert np.array_equal(codes_from_i8(b.view(np.uint8)), q)


def test_tiling_helpers_are_inverse_permutations():
    rng = np.random.default_rng(5)
    a = rng.integers(0, 256, (37, 384), dtype=np.uint8)
    assert np.array_equal(untile_codes_i8(tile_codes_i8(a), 37), a)
    wq = rng.integers(0, 256, (21, 192), dtype=np.uint8)
    assert np.array_equal(untile_weights(tile_weights(wq), 21), wq)
    # every byte sits at the offset the header documents
    t = tile_codes_i8(a).reshape(-1)
    K = a.shape[1]
    for m in range(a.shape[0]):
        for k in range(K):
            blk, r, tt = m // 16, m % 16, k // 128
            g, h = (k % 128) // 32, (k % 32) // 16
            assert t[(blk * (K // 128) + tt) * 2048 + ((4 * h + g) * 16 + r) * 16 + k % 16] == a[m, k]
    tw = tile_weights(wq).reshape(-1)
    H = wq.shape[1]
    for n in range(wq.shape[0]):
        for j in range(H):
            off = ((n // 16) * (H // 64) + j // 64) * 1024 + (16 * ((j % 64) // 16) + n % 16) * 16 + j % 16
            assert tw[off] == wq[n, j]


def test_residual_extended_tiling():
    # every row block holds its K/128 code tiles, then its residual tiles
    rng = np.random.default_rng(6)
    N, K, rp = 21, 384, 256
    main = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    res = rng.integers(0, 256, (N, rp // 2), dtype=np.uint8)
    ext = tile_weights_residual(main, res)
    assert ext.shape == (32, (K + rp) // 2)
    m2, r2 = untile_weights_residual(ext, N, K)
    assert np.array_equal(m2, main) and np.array_equal(r2, res)
    flat = ext.reshape(-1)
    nt = (K + rp) // 128
    for n in range(N):
        for jj in range(rp // 2):
            t = K // 128 + jj // 64
            off = ((n // 16) * nt + t) * 1024 + (16 * ((jj % 64) // 16) + n % 16) * 16 + jj % 16
            assert flat[off] == res[n, jj]


def test_mx_scale_tiling():
    rng = np.random.default_rng(7)
    M, K = 21, 384
    s = rng.integers(0, 256, (M, K // 32), dtype=np.uint8)
    flat = tile_mx_scales(s)
    assert flat.size == 32 * K // 32
    assert np.array_equal(untile_mx_scales(flat, M, K), s)
    for m in range(M):
        for blk in range(K // 32):
            t, g = blk // 4, blk % 4
            assert flat[((m // 16) * (K // 128) + t) * 64 + g * 16 + m % 16] == s[m, blk]


def test_offset_binary_pairing_gives_the_corrected_integer_product():
    # The nibble pairing the offset-binary GEMM uses, emulated byte by byte on
    # the encoded operands: signed high nibble (times 16) of one side with the
    # offset low nibble of the other, both ways, summed over the bytes of a
    # row pair, equals 16 qx.qw + 128 (row sum + column sum).
    rng = np.random.default_rng(11)
    M, N, K = 19, 23, 256
    qx = rng.integers(-8, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qx[0] = -8
    qw[0] = 7
    ta, sa = split_ob(ob_codes(tile_weights(O.pack_int4(qx)), M, K), M, K)
    tb, sb = split_ob(ob_weights(tile_weights(O.pack_int4(qw)), N, K), N, K)
    A = untile_weights(ta, M).astype(np.int64)
    B = untile_weights(tb, N).astype(np.int64)

    def hi(v):
        h = v >> 4
        return np.where(h >= 8, h - 16, h)

    acc = 16 * (hi(A) @ (B & 15).T + (A & 15) @ hi(B).T)
    ref = O.int_gemm(qx, qw).astype(np.int64)
    assert np.array_equal(acc, 16 * ref + 128 * (sa[:, None].astype(np.int64) + sb[None, :]))
    # the sums are those of the odd (activations) and even (weights) channels
    assert np.array_equal(sa, qx[:, 1::2].sum(axis=1))
    assert np.array_equal(sb, qw[:, 0::2].sum(axis=1))


def test_e2m3_values_from_the_format_definition():
    from layouts import e2m3_value, e2m3_code
    # sign bit 5, exponent bits 4:3 (bias 1), mantissa 2:0; exponent 0 subnormal
    cases = {0b000000: 0.0, 0b000001: 0.125, 0b000111: 0.875, 0b001000: 1.0, 0b010000: 2.0,
             0b010100: 3.0, 0b011000: 4.0, 0b011010: 5.0, 0b011100: 6.0, 0b011110: 7.0,
             0b011111: 7.5, 0b111110: -7.0, 0b101100: -1.5}
    for c, v in cases.items():
        assert e2m3_value(c) == v, c
    assert np.signbit(e2m3_value(0b100000))  # -0
    q = np.arange(-7, 8)
    assert np.array_equal(e2m3_value(e2m3_code(q)), q)
    assert e2m3_code(np.array([3]))[0] == 0b010100 and e2m3_code(np.array([-7]))[0] == 0b111110


def test_f6_tiles_put_fields_where_the_header_says():
    from layouts import tile_f6, untile_f6, untile_f6_codes, e2m3_code
    rng = np.random.default_rng(11)
    R, K = 21, 256
    q = rng.integers(-7, 8, (R, K)).astype(np.int8)
    t = tile_f6(q)
    assert t.shape == (32, 3 * K // 4)
    assert np.array_equal(untile_f6(t, R, K), q)
    flat = t.reshape(-1)
    for m in range(R):
        for k in range(0, K, 7):
            b, r, tt, g, u = m // 16, m % 16, k // 128, (k % 128) // 32, k % 32
            p = 2 * u if u < 16 else 2 * (u - 16) + 1
            lane = 16 * g + r
            tile = (b * (K // 128) + tt) * 1536
            val = 0
            for j in range(6):
                bit = 6 * p + j
                off = tile + 16 * lane + bit // 8 if bit < 128 else tile + 1024 + 8 * lane + (bit - 128) // 8
                val |= ((int(flat[off]) >> (bit % 8)) & 1) << j
            assert val == e2m3_code(q[m:m + 1, k])[0], (m, k)
    # zero codes are +0 (code 0) in every field
    assert np.array_equal(untile_f6_codes(tile_f6(np.zeros((R, K), np.int8)), R, K),
                          np.zeros((R, K)))
