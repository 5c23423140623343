"""Pins of the oracle's block rotation against closed forms and invariants.

The pages fix: the rotation is an orthogonal Hadamard-type transform (SERQ
page, "Resumen técnico" §1; DynamicPTQ page, "Perspectiva Teórica"), its
first row is all ones so that one outlier channel becomes a constant offset
over its group (OffQ page, "Metodología" step 2), and it acts on groups of
channels independently (OffQ page, step 3).
"""
import numpy as np
import pytest

from oracle import w4a4_oracle as O

POW2 = [1 << p for p in range(0, 13)]  # 1 .. 4096


def fwht_textbook(v):
    """Iterative in-place Walsh-Hadamard butterflies (natural order), float64."""
    v = np.array(v, dtype=np.float64)
    n = v.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            a = v[..., i:i + h].copy()
            b = v[..., i + h:i + 2 * h].copy()
            v[..., i:i + h] = a + b
            v[..., i + h:i + 2 * h] = a - b
        h *= 2
    return v


@pytest.mark.parametrize("b", POW2)
def test_hadamard_gram_is_b_identity(b):
    H = O.hadamard_matrix(b)
    assert H.shape == (b, b)
    assert np.array_equal(np.abs(H), np.ones((b, b)))
    assert np.array_equal(H @ H.T, b * np.eye(b))
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("b", POW2)
def test_first_row_and_column_all_ones(b):
    H = O.hadamard_matrix(b)
    assert np.all(H[0, :] == 1.0)
    assert np.all(H[:, 0] == 1.0)


@pytest.mark.parametrize("b", [1, 2, 4, 8, 64, 512])
def test_sylvester_doubling(b):
    # Independent construction: H_2b = [[H_b, H_b], [H_b, -H_b]].
    Hb = O.hadamard_matrix(b)
    H2 = O.hadamard_matrix(2 * b)
    assert np.array_equal(H2, np.block([[Hb, Hb], [Hb, -Hb]]))


@pytest.mark.parametrize("b,K", [(2, 8), (8, 64), (128, 512), (4096, 4096), (128, 14336 // 28)])
def test_matches_independent_fwht(b, K):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, K))
    ref = fwht_textbook(x.reshape(5, K // b, b)).reshape(5, K) / np.sqrt(b)
    got = O.rotate64(x, b)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("b", [2, 16, 128, 4096])
def test_involution(b):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 2 * b if b < 4096 else b)) * 10
    back = O.rotate64(O.rotate64(x, b), b)
    assert np.max(np.abs(back - x)) <= 1e-12 * np.max(np.abs(x))


@pytest.mark.parametrize("b", [4, 128, 4096])
def test_norm_preserved_per_row_and_block(b):
    rng = np.random.default_rng(3)
    K = 4096
    x = rng.standard_normal((4, K))
    x[:, 7] *= 100
    y = O.rotate64(x, b)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12, atol=0)
    xb = x.reshape(4, K // b, b)
    yb = y.reshape(4, K // b, b)
    assert np.allclose(np.linalg.norm(yb, axis=2), np.linalg.norm(xb, axis=2), rtol=1e-12, atol=0)


@pytest.mark.parametrize("b,K,j", [(4, 16, 2), (128, 512, 1), (4096, 8192, 1)])
def test_first_channel_outlier_becomes_constant_offset(b, K, j):
    # OffQ, step 2: an outlier on the first channel of a group is spread
    # evenly over that group as a constant offset; other groups stay untouched.
    v = 300.0
    x = np.zeros((1, K))
    x[0, j * b] = v
    y = O.rotate64(x, b)
    blk = y[0, j * b:(j + 1) * b]
    assert np.allclose(blk, v / np.sqrt(b), rtol=1e-15, atol=0)
    rest = np.delete(y[0], np.arange(j * b, (j + 1) * b))
    assert np.all(rest == 0.0)


@pytest.mark.parametrize("b,c", [(8, 5), (128, 77), (4096, 1234)])
def test_single_channel_spreads_with_hadamard_signs(b, c):
    v = -42.0
    x = np.zeros((1, b))
    x[0, c] = v
    y = O.rotate64(x, b)[0]
    assert np.allclose(np.abs(y), abs(v) / np.sqrt(b), rtol=1e-15, atol=0)
    H = O.hadamard_matrix(b)
    assert np.array_equal(np.sign(y), np.sign(v) * H[c % b, :])


def test_outlier_plus_noise_is_offset_plus_rotated_noise():
    # Linearity: the constant offset adds on top of the rotated remainder.
    b = 128
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, b))
    base = O.rotate64(x, b)
    x2 = x.copy()
    x2[0, 0] += 1000.0
    y2 = O.rotate64(x2, b)
    assert np.allclose(y2 - base, 1000.0 / np.sqrt(b), rtol=1e-12, atol=1e-9)


def test_blocks_are_independent():
    b, K = 64, 512
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, K))
    y = O.rotate64(x, b)
    x2 = x.copy()
    x2[:, 3 * b:4 * b] = rng.standard_normal((2, b))
    y2 = O.rotate64(x2, b)
    untouched = np.r_[0:3 * b, 4 * b:K]
    assert np.array_equal(y[:, untouched], y2[:, untouched])


def test_rotate_rounds_once_to_fp32():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 256)).astype(np.float16)
    assert O.rotate(x, 256).dtype == np.float32
    assert np.array_equal(O.rotate(x, 256), O.rotate64(x, 256).astype(np.float32))


def test_block_one_is_identity():
    x = np.arange(12, dtype=np.float64).reshape(2, 6)
    assert np.array_equal(O.rotate64(x, 1), x)


def test_rejects_bad_block():
    with pytest.raises(ValueError):
        O.hadamard_matrix(12)
    with pytest.raises(ValueError):
        O.rotate64(np.zeros((1, 12)), 8)
