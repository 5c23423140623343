"""Pins of the oracle's MXFP4 path (SERQ page, "Metodología" item 2: the
4-bit path in INT4 or MXFP4), read as the OCP microscaling format: blocks of
32 elements sharing a power-of-two scale, FP4 E2M1 elements."""
import numpy as np
import pytest

from oracle import w4a4_oracle as O


def test_e2m1_rounding_table():
    # every representable magnitude, every midpoint (ties to the even
    # encoding), points just beside the midpoints, and saturation
    pts = [(0.0, 0), (0.5, 1), (1.0, 2), (1.5, 3), (2.0, 4), (3.0, 5), (4.0, 6), (6.0, 7),
           (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
           (0.2500001, 1), (0.7499999, 1), (1.2500001, 3), (1.7499999, 3), (2.5000001, 5),
           (3.4999999, 5), (5.0000001, 7), (6.5, 7), (7.99, 7), (0.1, 0)]
    for v, code in pts:
        assert O.e2m1_code(np.array([v]))[0] == code, v
        assert O.e2m1_code(np.array([-v]))[0] == code | 8, -v      # the sign is kept, -0 included
    assert O.e2m1_code(np.array([0.0]))[0] == 0
    assert np.array_equal(O.e2m1_value(np.arange(16)),
                          [0, .5, 1, 1.5, 2, 3, 4, 6, 0, -.5, -1, -1.5, -2, -3, -4, -6])


def test_codes_are_the_nearest_value():
    rng = np.random.default_rng(1)
    p = rng.uniform(-6, 6, 20000)
    c = O.e2m1_code(p)
    vals = O.e2m1_value(np.arange(8))
    best = np.abs(np.abs(p)[:, None] - vals[None, :]).min(axis=1)
    assert np.allclose(np.abs(np.abs(p) - np.abs(O.e2m1_value(c))), best)


@pytest.mark.parametrize("amax,e", [(6.0, 0), (4.0, 0), (7.99, 0), (3.99, -1), (1.0, -2), (8.0, 1),
                                    (2.0 ** -124, -126), (2.0 ** -125, -127), (2.0 ** -140, -127),
                                    (0.0, -127), (2.0 ** 127, 125)])
def test_block_exponent(amax, e):
    assert O.mx_block_exponent(np.array([amax]))[0] == e


def test_block_scale_puts_the_maximum_in_4_to_8():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((6, 256)) * np.exp2(rng.integers(-20, 20, (6, 1)))).astype(np.float32)
    codes, e = O.quantize_mxfp4(v)
    amax = np.abs(v.reshape(6, 8, 32)).max(axis=2)
    q = amax / np.exp2(e)
    assert np.all((q >= 4) & (q < 8))
    deq = O.mxfp4_values(codes, e)
    err = np.abs(v - deq).reshape(6, 8, 32)
    assert np.all(err <= np.exp2(e)[:, :, None] * 2)          # saturation (6, 8) costs < 2 steps
    inside = np.abs(v.reshape(6, 8, 32)) <= 6 * np.exp2(e)[:, :, None]
    assert np.all(err[inside] <= np.broadcast_to(np.exp2(e)[:, :, None], err.shape)[inside])


def test_zero_and_grid_blocks():
    v = np.zeros((2, 64), np.float32)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6] * 4, np.float32)
    v[1, 32:] = -grid * 2.0 ** -3
    codes, e = O.quantize_mxfp4(v)
    assert e[0, 0] == -127 and not codes[0].any()
    assert e[1, 1] == -3
    assert np.array_equal(O.mxfp4_values(codes, e)[1, 32:], v[1, 32:])   # lossless on the grid


def test_gemm_matches_a_literal_loop():
    rng = np.random.default_rng(3)
    M, N, K = 3, 4, 96
    cx = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
    ex = rng.integers(-10, 10, (M, K // 32))
    ew = rng.integers(-10, 10, (N, K // 32))
    y = O.mxfp4_gemm(cx, ex, cw, ew)
    for m in range(M):
        for n in range(N):
            ref = 0.0
            for k in range(K):
                vx = float(O.e2m1_value(cx[m, k])) * 2.0 ** int(ex[m, k // 32])
                vw = float(O.e2m1_value(cw[n, k])) * 2.0 ** int(ew[n, k // 32])
                ref += vx * vw
            assert y[m, n] == ref


@pytest.mark.parametrize("b", [16, 256])
def test_mxfp4_lossless_grid_gives_exact_product(b):
    # Rotated activations and weights already MXFP4-representable (each
    # block holds a 4 or a 6 times its scale): the MXFP4 forward is exact,
    # Y = X~ W~^T.  b is a power of four, so the rotations are exact.
    rng = np.random.default_rng(4)
    M, N, K = 5, 6, 512
    def grid(R, top):
        c = rng.integers(0, 16, (R, K)).astype(np.uint8)
        c[:, ::32] = top
        e = rng.integers(-8, 4, (R, K // 32))
        return O.mxfp4_values(c, e)
    xt, wt = grid(M, 7), grid(N, 6)
    X = O.rotate64(xt, b).astype(np.float32)
    Wm = O.rotate64(wt, b).astype(np.float32)
    assert np.array_equal(O.rotate64(X, b), xt)
    y = O.qlinear_forward_mxfp4(X, Wm, b)
    assert np.array_equal(y, (xt @ wt.T).astype(np.float32))


def test_sign_of_zero_leaves_the_product_unchanged():
    # A negative quotient that rounds to zero keeps its sign bit (code 8, an
    # IEEE-style -0); -0 and +0 both have the value 0, so the product and the
    # layer's output do not depend on which of the two encodings is chosen.
    v = np.array([[-1e-9, 1e-9, -0.0, 0.0] + [6.0] * 28], np.float32)
    codes, e = O.quantize_mxfp4(v)
    assert codes[0, :4].tolist() == [8, 0, 8, 0]
    rng = np.random.default_rng(6)
    M, N, K = 4, 5, 128
    cx = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
    ex = rng.integers(-6, 6, (M, K // 32))
    ew = rng.integers(-6, 6, (N, K // 32))
    flip = lambda c: np.where((c & 7) == 0, c ^ 8, c).astype(np.uint8)   # +0 <-> -0
    y = O.mxfp4_gemm(cx, ex, cw, ew)
    assert np.array_equal(O.mxfp4_gemm(flip(cx), ex, cw, ew), y)
    assert np.array_equal(O.mxfp4_gemm(cx, ex, flip(cw), ew), y)
