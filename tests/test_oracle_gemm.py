"""Pins of the oracle's integer GEMM, low-rank term, epilogue and whole layer.

SERQ page, "Resumen técnico" §1-3: a 4-bit x 4-bit matrix product in the
linear layer plus one low-rank compensation term; OffQ page, "Metodología",
steps 2-3 for the rotation in front.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def triple_loop(a, b):
    M, K = a.shape
    N = b.shape[0]
    out = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        for n in range(N):
            t = 0
            for k in range(K):
                t += int(a[m, k]) * int(b[n, k])
            out[m, n] = t
    return out


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (8, 4, 64), (13, 9, 33)])
def test_int_gemm_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    a = rng.integers(-8, 8, (M, K)).astype(np.int8)
    b = rng.integers(-8, 8, (N, K)).astype(np.int8)
    want = triple_loop(a, b)
    assert np.array_equal(O.int_gemm(a, b), want)
    assert np.array_equal(a.astype(np.int64) @ b.astype(np.int64).T, want)


def test_int_gemm_k1_exhaustive_table():
    v = np.arange(-8, 8, dtype=np.int8)
    a = v.reshape(16, 1)
    acc = O.int_gemm(a, a)
    assert np.array_equal(acc, np.outer(v.astype(np.int64), v.astype(np.int64)))


def test_int_gemm_extremes_and_bound():
    K = 14336
    neg8 = np.full((1, K), -8, np.int8)
    assert O.int_gemm(neg8, neg8)[0, 0] == 64 * K
    seven = np.full((1, K), 7, np.int8)
    assert O.int_gemm(seven, -seven)[0, 0] == -49 * K
    rng = np.random.default_rng(7)
    a = rng.integers(-7, 8, (4, 4096)).astype(np.int8)
    b = rng.integers(-7, 8, (4, 4096)).astype(np.int8)
    assert np.all(np.abs(O.int_gemm(a, b)) <= 49 * 4096)


def test_groups_sum_to_full():
    rng = np.random.default_rng(8)
    a = rng.integers(-7, 8, (5, 512)).astype(np.int8)
    b = rng.integers(-7, 8, (6, 512)).astype(np.int8)
    g = O.int_gemm_groups(a, b, 128)
    assert g.shape == (4, 5, 6)
    assert np.array_equal(g.sum(axis=0), O.int_gemm(a, b))
    assert np.array_equal(g[2], triple_loop(a[:, 256:384], b[:, 256:384]))


def test_lowrank_alone_when_weight_codes_are_zero():
    # With all-zero weight codes the layer reduces to X @ A @ B (torch fp64).
    rng = np.random.default_rng(9)
    M, K, N, r = 6, 128, 40, 8
    X = rng.standard_normal((M, K)).astype(np.float16)
    A = (0.01 * rng.standard_normal((K, r))).astype(np.float16)
    B = (0.01 * rng.standard_normal((r, N))).astype(np.float16)
    wq = np.zeros((N, K // 2), np.uint8)
    ws = np.ones(N, np.float16)
    y = O.qlinear_forward(X, wq, ws, 128, 0, A, B)
    want = (torch.from_numpy(X).double() @ torch.from_numpy(A).double()
            @ torch.from_numpy(B).double()).float().numpy()
    assert np.array_equal(y, want)


def test_without_lowrank_term():
    rng = np.random.default_rng(10)
    X = rng.standard_normal((4, 64)).astype(np.float32)
    W = (0.02 * rng.standard_normal((8, 64))).astype(np.float32)
    wq, ws, qw = O.prepare_weight(W, 64, 0, "float32")
    y = O.qlinear_forward(X, wq, ws, 64, 0)
    _, sx, qx, _ = O.quantize_activation(X, 64)
    want = (sx[:, None].astype(np.float64) * ws[None, :].astype(np.float64)
            * (qx.astype(np.int64) @ qw.astype(np.int64).T)).astype(np.float32)
    assert np.array_equal(y, want)


@pytest.mark.parametrize("b,g,sd", [(64, 0, "float32"), (16, 128, "float16"), (256, 64, "float16")])
def test_lossless_grid_gives_exact_product(b, g, sd):
    # Closed form: if the rotated activations and weights already sit on the
    # int4 grid (power-of-two scales, every row/group reaching +-7), the whole
    # pipeline is exact and Y equals the float64 product X~ W~^T.  b is a
    # power of four so that 1/sqrt(b) is a power of two and X = X~ H / sqrt(b)
    # is exactly representable in float32.
    rng = np.random.default_rng(11)
    M, N, K = 7, 9, 512
    gg = K if g == 0 else g
    qx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    qx[:, 0] = 7
    sx = np.float32(2.0 ** -3)
    qw = rng.integers(-7, 8, (N, K)).astype(np.int8)
    qw[:, ::gg] = -7
    sw = np.float32(2.0 ** -6)
    xt = sx * qx.astype(np.float64)
    wt = sw * qw.astype(np.float64)
    X = O.rotate64(xt, b)            # the rotation is an involution
    W = O.rotate64(wt, b)
    wq, ws, qw_back = O.prepare_weight(W.astype(np.float32), b, g, sd)
    assert np.array_equal(qw_back, qw)
    y = O.qlinear_forward(X.astype(np.float32), wq, ws, b, g)
    assert np.array_equal(y, (xt @ wt.T).astype(np.float32))


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_k4_example.json")) as f:
        gd = json.load(f)
    X = np.array(gd["X"], np.float32)
    W = np.array(gd["W"], np.float32)
    b = gd["had_block"]
    xp, sx, qx, xr = O.quantize_activation(X, b)
    assert np.allclose(xr, gd["x_rot"], rtol=1e-6, atol=1e-7)
    assert qx.tolist() == gd["x_codes"]
    assert xp.tolist() == gd["x_packed"]
    assert np.allclose(sx, gd["x_scale"], rtol=1e-6)
    wq, ws, qw = O.prepare_weight(W, b, 0, "float32")
    assert qw.tolist() == gd["w_codes"]
    assert np.allclose(ws, gd["w_scale"], rtol=1e-6)
    assert O.int_gemm(qx, qw).tolist() == gd["acc"]
    y = O.qlinear_forward(X, wq, ws, b, 0)
    assert np.allclose(y, gd["y"], rtol=1e-6, atol=1e-6)
    A = np.array(gd["A"], np.float32)
    B = np.array(gd["B"], np.float32)
    assert np.allclose(O.lowrank(X, A, B), gd["lowrank"], rtol=0, atol=0)
    y2 = O.qlinear_forward(X, wq, ws, b, 0, A, B)
    assert np.allclose(y2, np.array(gd["y"]) + np.array(gd["lowrank"]), rtol=1e-6, atol=1e-6)


def test_rotation_reduces_error_on_outlier_inputs():
    # Sanity of the method's premise (OffQ page, "Declaración del problema";
    # DynamicPTQ page, "Planteamiento"): with massive channels the rotated
    # W4A4 product is closer to X W^T than the unrotated one on ordinary rows.
    w = synth.small("t", 64, 1024, 256, n_outlier=4, bos_factor=500.0)
    d = synth.make_inputs(w)
    X, W = d["X"], d["W"]
    exact = X.astype(np.float64) @ W.astype(np.float64).T

    def rel_err(b):
        wq, ws, _ = O.prepare_weight(W, b, 0, "float16")
        y = O.qlinear_forward(X, wq, ws, b, 0)
        return np.linalg.norm(y[1:] - exact[1:]) / np.linalg.norm(exact[1:])

    assert rel_err(128) < 0.9 * rel_err(1)
    assert rel_err(1024) < 0.9 * rel_err(1)


def literal_layer(qx, sx, qw, sw, group, X=None, A=None, B=None):
    """The layer's output written out element by element from its definition
    (SERQ page, "Resumen técnico" §2-3): for every output, the activation
    scale times the sum over K-groups of the group's weight scale times the
    group's integer dot product, plus the low-rank term sum_r (X A)[m,r] B[r,n];
    float64 sums, rounded once to float32."""
    M, K = qx.shape
    N = qw.shape[0]
    g = K if group == 0 else group
    sw2 = np.asarray(sw, np.float64).reshape(N, -1)
    y = np.zeros((M, N), np.float32)
    for m in range(M):
        t = None
        if A is not None:
            t = [sum(float(X[m, k]) * float(A[k, r]) for k in range(K)) for r in range(A.shape[1])]
        for n in range(N):
            acc = 0.0
            for j in range(K // g):
                dot = sum(int(qx[m, k]) * int(qw[n, k]) for k in range(j * g, (j + 1) * g))
                acc += float(sx[m]) * float(sw2[n, j]) * dot
            if t is not None:
                acc += sum(t[r] * float(B[r, n]) for r in range(len(t)))
            y[m, n] = np.float32(acc)
    return y


@pytest.mark.parametrize("g,rank", [(0, 0), (0, 4), (64, 0), (128, 4), (64, 4)])
def test_qlinear_from_codes_matches_a_literal_loop(g, rank):
    # Brute force on tiny shapes, with scales that differ from group to group
    # so that a dropped group index, a single scale per row or a missing
    # low-rank term cannot pass.
    rng = np.random.default_rng(20 + g + rank)
    M, N, K = 3, 5, 256
    qx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    sx = rng.uniform(0.5, 2.0, M).astype(np.float32)
    G = 1 if g == 0 else K // g
    sw = rng.uniform(0.01, 0.05, (N, G)).astype(np.float16)
    sw = sw[:, 0] if g == 0 else sw
    X = A = B = None
    if rank:
        X = rng.standard_normal((M, K)).astype(np.float16)
        A = (0.1 * rng.standard_normal((K, rank))).astype(np.float16)
        B = (0.1 * rng.standard_normal((rank, N))).astype(np.float16)
    got = O.qlinear_from_codes(qx, sx, O.pack_int4(qw), sw, g, X, A, B)
    want = literal_layer(qx, sx, qw, sw, g, X, A, B)
    # float64 sums in another order: equal up to the final rounding to float32
    assert np.all(np.abs(got.astype(np.float64) - want) <= 2.0 ** -23 * np.abs(want))


@pytest.mark.parametrize("b,g,rank,dt", [(64, 0, 0, "float32"), (128, 64, 8, "float16"),
                                        (256, 128, 8, "float16"), (128, 128, 0, "float16"),
                                        (256, 0, 16, "float16")])
def test_qlinear_from_codes_on_the_oracle_codes_is_the_forward(b, g, rank, dt):
    # Fed the oracle's own codes and scales, the epilogue the GPU results are
    # judged by is the oracle's forward, bit for bit.
    w = synth.small("fc", 9, 512, 40, x_dtype=dt, had_block=b, w_group=g, rank=rank,
                    w_scale_dtype="float16" if dt == "float16" else "float32")
    d = synth.make_inputs(w)
    wq, ws, _ = O.prepare_weight(d["W"], b, g, w.w_scale_dtype)
    _, sx, qx, _ = O.quantize_activation(d["X"], b)
    got = O.qlinear_from_codes(qx, sx, wq, ws, g, d["X"], d["A"], d["B"])
    assert np.array_equal(got, O.qlinear_forward(d["X"], wq, ws, b, g, d["A"], d["B"]))
