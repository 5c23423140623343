"""Pins of the oracle's W4A8 layer: 8-bit per-token activations (qmax 127)
beside the 4-bit weights, the precision a phase-aware policy keeps for
sensitive layers (DynamicPTQ page, "Metodología" §2)."""
import numpy as np
import pytest

from oracle import w4a4_oracle as O

Q8 = 127


def test_ties_round_to_even_across_the_int8_range():
    s = np.float32(2.0 ** -4)
    row = np.array([127 * s] + [(n + 0.5) * s for n in (0, 1, 2, 61, 62, 125)] +
                   [-(n + 0.5) * s for n in (0, 3, 126)], np.float32)
    q, sx = O.quantize_act(row[None, :], Q8)
    assert sx[0] == s
    assert q[0].tolist() == [127, 0, 2, 2, 62, 62, 126, 0, -4, -126]


def test_absmax_maps_to_127_with_sign():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 300)).astype(np.float32)
    x[3, 17] = -50.0
    q, s = O.quantize_act(x, Q8)
    assert np.all(np.abs(q).max(axis=1) == Q8)
    assert q[3, 17] == -Q8
    assert np.all(s == (np.abs(x).max(axis=1) / np.float32(Q8)).astype(np.float32))


def test_codes_are_the_nearest_of_all_255_levels():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((4, 257)) * 3).astype(np.float32)
    q, s = O.quantize_act(x, Q8)
    levels = np.arange(-Q8, Q8 + 1, dtype=np.float64)
    for m in range(x.shape[0]):
        quot = (x[m] / s[m]).astype(np.float32).astype(np.float64)
        dist = np.abs(quot[:, None] - levels[None, :])
        best = levels[np.argmin(dist, axis=1)]
        # away from exact ties the nearest level is unique
        untied = np.abs(np.abs(quot - np.floor(quot)) - 0.5) > 1e-6
        assert np.array_equal(q[m][untied].astype(np.float64), best[untied])
        assert np.all(np.abs(x[m].astype(np.float64) - s[m] * q[m]) <= 0.5 * s[m] * (1 + 1e-6))


def test_zero_row_gives_zero_scale_and_codes():
    x = np.zeros((2, 64), np.float32)
    x[1, 5] = 1.0
    q, s = O.quantize_act(x, Q8)
    assert s[0] == 0 and not q[0].any()
    assert q[1, 5] == Q8


@pytest.mark.parametrize("b", [16, 64, 256])
def test_w4a8_lossless_grid_gives_exact_product(b):
    # Rotated activations already on the int8 grid (power-of-two scale, every
    # row reaching +-127) and weights on the int4 grid: the W4A8 forward is
    # exact, Y = X~ W~^T.  b is a power of four so X = X~ H / sqrt(b) is exact.
    rng = np.random.default_rng(12)
    M, N, K = 5, 7, 512
    qx = rng.integers(-Q8, Q8 + 1, (M, K)).astype(np.int16)
    qx[:, 3] = -Q8
    sx = np.float32(2.0 ** -7)
    qw = rng.integers(-7, 8, (N, K)).astype(np.int8)
    qw[:, 0] = 7
    sw = np.float32(2.0 ** -6)
    xt = sx * qx.astype(np.float64)
    wt = sw * qw.astype(np.float64)
    X = O.rotate64(xt, b)
    W = O.rotate64(wt, b)
    wq, ws, qw_back = O.prepare_weight(W.astype(np.float32), b, 0, "float32")
    assert np.array_equal(qw_back, qw)
    y = O.qlinear_forward(X.astype(np.float32), wq, ws, b, 0, act_bits=8)
    assert np.array_equal(y, (xt @ wt.T).astype(np.float32))


def test_eight_bit_activations_cut_the_activation_error():
    # Sanity (not a pin of a printed value): on outlier-bearing inputs the
    # 8-bit activation error is far below the 4-bit one.
    from bit_gemm_block_amd import synth
    w = synth.small("a8", 32, 1024, 8, n_outlier=2, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xr = O.rotate(X, 128)
    err = {}
    for qmax in (7, Q8):
        q, s = O.quantize_act(xr, qmax)
        err[qmax] = np.linalg.norm(xr - s[:, None] * q) / np.linalg.norm(xr)
    assert err[Q8] < err[7] / 10
