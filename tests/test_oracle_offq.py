"""Pins of the oracle's asymmetric group-wise activation path (OffQ page,
"Metodología" steps 2-3): the all-ones Hadamard row turns a group's outlier
into a constant offset, and the zero point of a per-group asymmetric
quantizer absorbs it."""
import numpy as np
import pytest

from oracle import w4a4_oracle as O


def test_min_and_max_map_to_the_ends_of_the_code_range():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((5, 256)) * 2 + 3).astype(np.float32)
    q, s, z = O.quantize_act_asym(x, 128)
    assert q.min() >= 0 and q.max() <= 15
    xg = x.reshape(5, 2, 128)
    qg = q.reshape(5, 2, 128)
    for m in range(5):
        for g in range(2):
            assert qg[m, g, np.argmin(xg[m, g])] == 0
            assert qg[m, g, np.argmax(xg[m, g])] == 15


def test_an_offset_of_whole_steps_is_absorbed_by_the_zero_point():
    # On a power-of-two grid, adding n steps to a whole group leaves every
    # code unchanged and moves only the zero point by -n, also past the ends
    # of the code range (the whole offset is absorbed).
    rng = np.random.default_rng(2)
    s = np.float32(2.0 ** -3)
    q0 = rng.integers(0, 16, (3, 128))
    q0[:, 0], q0[:, 1] = 0, 15
    z0 = 9
    x = (s * (q0 - z0)).astype(np.float32)
    qa, sa, za = O.quantize_act_asym(x, 128)
    assert np.all(sa == s) and np.all(za == z0) and np.array_equal(qa, q0)
    for n in (-30, -6, -2, 3, 9, 20):
        qb, sb, zb = O.quantize_act_asym((x + n * s).astype(np.float32), 128)
        assert np.array_equal(qb, qa)
        assert np.all(sb == s) and np.all(zb == z0 - n)


def test_offsets_cost_far_less_than_with_the_symmetric_quantizer():
    rng = np.random.default_rng(3)
    x = (100.0 + rng.standard_normal((8, 128))).astype(np.float32)
    q, s, z = O.quantize_act_asym(x, 128)
    err_asym = np.abs(x - s[:, :1] * (q.astype(np.float64) - z[:, :1])).max()
    qs, ss = O.quantize_act(x)
    err_sym = np.abs(x - ss[:, None] * qs).max()
    assert err_asym < err_sym / 10


def test_hadamard_offset_of_a_single_channel_outlier():
    # A single-channel outlier becomes a constant offset over its block after
    # the rotation (all-ones first row); the asymmetric codes then keep the
    # other channels' detail that the symmetric ones lose.
    rng = np.random.default_rng(4)
    b = 128
    x = rng.standard_normal((4, b)).astype(np.float32)
    x[:, 0] = 500.0
    xr = O.rotate(x, b)
    assert np.allclose(xr.mean(axis=1), 500 / np.sqrt(b), atol=0.5)
    qa, sa, za = O.quantize_act_asym(xr, b)
    ea = np.linalg.norm(xr - sa * (qa.astype(np.float64) - za))
    qs, ss = O.quantize_act(xr)
    es = np.linalg.norm(xr - ss[:, None] * qs)
    assert np.all(za < 0)
    assert ea < es / 8


def test_codes_are_the_nearest_level_unless_clamped():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((6, 256)) * 3).astype(np.float32)
    q, s, z = O.quantize_act_asym(x, 64)
    G = 256 // 64
    for m in range(6):
        for g in range(G):
            sl = slice(64 * g, 64 * g + 64)
            t = (x[m, sl] / s[m, g]).astype(np.float32).astype(np.float64) + z[m, g]
            levels = np.arange(16.0)
            best = levels[np.argmin(np.abs(t[:, None] - levels[None, :]), axis=1)]
            untied = np.abs(np.abs(t - np.floor(t)) - 0.5) > 1e-6
            assert np.array_equal(q[m, sl][untied].astype(np.float64), best[untied])
            inside = (t >= -0.5) & (t <= 15.5)
            rec = s[m, g] * (q[m, sl].astype(np.float64) - z[m, g])
            assert np.all(np.abs(x[m, sl][inside] - rec[inside]) <= 0.5 * s[m, g] * (1 + 1e-6))


def test_constant_groups_are_coded_as_their_value():
    # A group with no spread takes the range between its value and zero; the
    # zero group has scale 0 and all-zero codes and zero point.
    x = np.zeros((3, 128), np.float32)
    x[1] = 3.0
    x[2] = -3.0
    q, s, z = O.quantize_act_asym(x, 128)
    assert s[0, 0] == 0 and not q[0].any() and z[0, 0] == 0
    s3 = np.float32(np.float32(3.0) / np.float32(15))
    assert s[1, 0] == s3 and s[2, 0] == s3
    assert np.all(q[1] == 15) and z[1, 0] == 0
    assert np.all(q[2] == 0) and z[2, 0] == 15
    for m in (1, 2):
        rec = s[m, 0] * (q[m].astype(np.float64) - z[m, 0])
        assert np.all(np.abs(rec - x[m]) <= 0.5 * s[m, 0])


def test_zero_point_epilogue_matches_a_literal_loop():
    rng = np.random.default_rng(6)
    M, N, K, g = 3, 4, 128, 64
    qx = rng.integers(0, 16, (M, K)).astype(np.uint8)
    zx = rng.integers(0, 16, (M, K // g))
    sx = rng.uniform(0.1, 1.0, (M, K // g)).astype(np.float32)
    qw = rng.integers(-7, 8, (N, K)).astype(np.int8)
    sw = rng.uniform(0.01, 0.1, N).astype(np.float32)
    y = O.asym_from_codes(qx, sx, zx, qw, sw, g)
    for m in range(M):
        for n in range(N):
            ref = 0.0
            for j in range(K // g):
                acc = sum((int(qx[m, k]) - int(zx[m, j])) * int(qw[n, k]) for k in range(j * g, (j + 1) * g))
                ref += float(sx[m, j]) * acc
            assert abs(float(y[m, n]) - ref * float(sw[n])) <= 1e-6 * max(1.0, abs(ref * float(sw[n])))


@pytest.mark.parametrize("b", [256, 1024])
def test_asymmetric_lossless_grid_gives_exact_product(b):
    # Rotated activations already on per-group asymmetric grids (power-of-two
    # step, codes 0 and 15 in every group, zero points inside and far outside
    # [0, 15]) and weights on the int4 grid: the forward is exact,
    # Y = X~ W~^T.  b is a power of four, so X = X~ H / sqrt(b) is exact.
    rng = np.random.default_rng(7)
    M, N, K = 4, 6, 1024
    G = K // b
    s = np.float32(2.0 ** -4)
    q = rng.integers(0, 16, (M, K))
    q[:, ::b] = 0
    q[:, 1::b] = 15
    z = rng.integers(-40, 56, (M, G))
    xt = s * (q - np.repeat(z, b, axis=1)).astype(np.float64)
    qw = rng.integers(-7, 8, (N, K)).astype(np.int8)
    qw[:, 0] = 7
    sw = np.float32(2.0 ** -6)
    wt = sw * qw.astype(np.float64)
    X = O.rotate64(xt, b)
    W = O.rotate64(wt, b)
    qa, sa, za = O.quantize_act_asym(O.rotate(X.astype(np.float32), b), b)
    assert np.array_equal(qa, q) and np.all(sa == s) and np.array_equal(za, z)
    wq, ws, qw_back = O.prepare_weight(W.astype(np.float32), b, 0, "float32")
    assert np.array_equal(qw_back, qw)
    y = O.qlinear_forward_asym(X.astype(np.float32), wq, ws, b)
    assert np.array_equal(y, (xt @ wt.T).astype(np.float32))


def test_weight_group_sums():
    rng = np.random.default_rng(8)
    qw = rng.integers(-8, 8, (5, 256)).astype(np.int8)
    ws = O.weight_group_sums(qw, 128)
    for n in range(5):
        for j in range(2):
            assert ws[n, j] == sum(int(v) for v in qw[n, 128 * j:128 * j + 128])
