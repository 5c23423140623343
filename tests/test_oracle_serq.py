"""Pins of the oracle's in-GEMM residual of salient channels (SERQ page,
"Metodología" items 2-3): the quantization error of the first r (salient,
offline-permuted) weight channels, quantized to 4 bits on the step s/8 and
multiplied by the same 4-bit activation codes of those channels."""
import numpy as np
import pytest

from oracle import w4a4_oracle as O


def test_residual_codes_bound_the_error_of_salient_channels():
    rng = np.random.default_rng(1)
    w = (0.02 * rng.standard_normal((40, 512))).astype(np.float32)
    w[:, 3] *= 30
    for sd in ("float16", "float32"):
        q, s, qr = O.quantize_weight_residual(w, 96, sd)
        s64 = s.astype(np.float64)[:, None]
        err_plain = np.abs(w[:, :96] - s64 * q[:, :96])
        err_res = np.abs(w[:, :96] - s64 * (q[:, :96] + qr / 8.0))
        assert np.all(np.abs(qr) <= 4)                       # |e| <= s/2 is never clamped
        assert np.all(err_res <= s64 / 16 * (1 + 1e-5) + 1e-12)
        assert err_res.max() < err_plain.max() / 4
        q0, s0 = O.quantize_weight(w, 0, sd)                 # the main codes are untouched
        assert np.array_equal(q, q0) and np.array_equal(s, s0)


def test_residual_codes_are_nearest_on_the_step_grid():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((8, 256)).astype(np.float32)
    q, s, qr = O.quantize_weight_residual(w, 128, "float32")
    s32 = s.astype(np.float32)
    e = (w[:, :128] - (s32[:, None] * q[:, :128].astype(np.float32)).astype(np.float32))
    t = (s32 / 8).astype(np.float64)[:, None]
    levels = np.arange(-8, 8)
    best = levels[np.argmin(np.abs(e[:, :, None] / t[:, :, None] - levels), axis=2)]
    quot = e / t
    untied = np.abs(np.abs(quot - np.floor(quot)) - 0.5) > 1e-6
    assert np.array_equal(qr[untied], best[untied])


def test_zero_rank_is_the_plain_layer():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((6, 256)).astype(np.float32)
    W = (0.02 * rng.standard_normal((10, 256))).astype(np.float32)
    wq, ws, _, qr = O.prepare_weight_residual(W, 64, 0, "float32")
    assert qr.shape == (10, 0)
    y0 = O.qlinear_forward(X, wq, ws, 64, 0)
    assert np.array_equal(O.qlinear_forward_residual(X, wq, ws, qr, 64), y0)


def test_residual_product_matches_a_literal_loop():
    rng = np.random.default_rng(4)
    M, N, K, r = 3, 4, 64, 20
    qx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qr = rng.integers(-8, 8, (N, r)).astype(np.int8)
    sx = rng.uniform(0.1, 1, M).astype(np.float32)
    sw = rng.uniform(0.01, 0.1, N).astype(np.float32)
    acc = O.residual_int_gemm(qx, qw, qr)
    y = O.residual_from_codes(qx, sx, qw, sw, qr)
    for m in range(M):
        for n in range(N):
            main = sum(int(qx[m, k]) * int(qw[n, k]) for k in range(K))
            res = sum(int(qx[m, k]) * int(qr[n, k]) for k in range(r))
            assert acc[m, n] == 8 * main + res
            ref = float(sx[m]) * float(sw[n]) * (main + res / 8)
            assert abs(float(y[m, n]) - ref) <= 1e-6 * max(abs(ref), 1e-30)


@pytest.mark.parametrize("b,r", [(16, 48), (256, 128), (64, 200)])
def test_residual_lossless_grid_gives_exact_product(b, r):
    # Rotated weights on the grid s (q + c/8) in the salient channels and on
    # s q elsewhere (a code 7 in a plain channel fixes s), rotated
    # activations on the int4 grid: the residual forward is exact,
    # Y = X~ W~^T.  b is a power of four, so the rotations are exact.
    rng = np.random.default_rng(5)
    M, N, K = 5, 7, 512
    sx = np.float32(2.0 ** -7)
    qx = rng.integers(-7, 8, (M, K))
    qx[:, 1] = 7
    sw = np.float32(2.0 ** -6)
    qw = rng.integers(-7, 8, (N, K))
    qw[:, :r] = rng.integers(-6, 7, (N, r))   # |q + c/8| < 7: a plain channel sets the scale
    qw[:, K - 1] = 7
    c = rng.integers(-4, 4, (N, r))
    wt = sw * qw.astype(np.float64)
    wt[:, :r] += sw * c / 8.0
    xt = sx * qx.astype(np.float64)
    X = O.rotate64(xt, b)
    W = O.rotate64(wt, b)
    wq, ws, q, qr = O.prepare_weight_residual(W.astype(np.float32), b, r, "float32")
    assert np.array_equal(ws, np.full(N, sw, np.float32))
    assert np.array_equal(sw * (q[:, :r] + qr / 8.0), wt[:, :r])
    y = O.qlinear_forward_residual(X.astype(np.float32), wq, ws, qr, b)
    assert np.array_equal(y, (xt @ wt.T).astype(np.float32))
    # without the residual the same layer is not exact
    y_plain = O.qlinear_forward(X.astype(np.float32), wq, ws, b, 0)
    assert not np.array_equal(y_plain, y)


def test_residual_cuts_the_weight_error_from_outlier_channels():
    # Sanity (not a pin of a printed value): activation outliers in the
    # salient channels make the weight error of those channels dominate the
    # weight-side error of Y; the residual removes most of it.  Measured
    # against the product of the quantized activations with the exact
    # weights, so that only the weight error counts.
    rng = np.random.default_rng(6)
    M, N, K, r = 32, 64, 512, 32
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, :8] *= 200
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    wq, ws, _, qr = O.prepare_weight_residual(W, 1, r, "float32")
    _, sx, qx, _ = O.quantize_activation(X, 1)
    ref = (sx[:, None] * qx.astype(np.float64)) @ W.astype(np.float64).T
    e_res = np.linalg.norm(O.qlinear_forward_residual(X, wq, ws, qr, 1) - ref)
    e_plain = np.linalg.norm(O.qlinear_forward(X, wq, ws, 1, 0) - ref)
    assert e_res < 0.25 * e_plain
