"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Bars (oracle readings, see the oracle module header):
* integer and byte results (codes, packed bytes, int32 accumulators) and the
  scales of the quantizer when both sides start from the same float32 input
  (the oracle's rotated activations, had_block 0): bit-exact;
* the float32 fast Walsh-Hadamard rotation against the float64 dense one:
  per block, max |delta| <= 2 (log2 b + 2) 2^-24 ||x~_block||_2 (first-order
  error bound of log2 b rounded butterfly stages plus the final scaling);
* the fused rotate+quantize path: at most 0.01% of codes differ, each by
  exactly one step, scales within 1e-6 relative;
* the float32 output: max |Y_gpu - epilogue(GPU codes and scales)| <=
  1e-3 * RMS(Y_oracle); the distance to the oracle's own Y is reported.
"""
import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth
from bit_gemm_block_amd import w4a4 as W
from layouts import (codes_from_i8, i8_from_codes, tile_codes_i8, tile_weights, untile_codes_i8,
                     untile_weights, workspace_codes)
from bars import check_y

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def np_dtype(name):
    return np.float16 if name == "float16" else np.float32


def rotation_bound(x, b):
    ref = O.rotate64(x, b)
    M, K = ref.shape
    blk = np.linalg.norm(ref.reshape(M, K // b, b), axis=2)
    lb = int(np.log2(b))
    bound = 2 * (lb + 2) * 2.0 ** -24 * blk
    return ref, np.repeat(bound, b, axis=1).reshape(M, K)


# --------------------------------------------------------------------------
# Rotation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,b,dt", [
    (16, 256, 256, "float32"), (5, 4096, 4096, "float16"), (33, 4096, 128, "float16"),
    (9, 14336, 128, "float16"), (3, 14336, 2048, "float16"), (7, 192, 64, "float32"),
    (4, 1024, 2, "float16"), (2, 512, 512, "float32"), (8, 2048, 2048, "float16"),
    (12, 8192, 4096, "float16"), (64, 4096, 1024, "float32"), (65, 4096, 4096, "float16"),
    (1, 4096, 4096, "float32")])
def test_hadamard_rotate_within_bound(M, K, b, dt):
    w = synth.small("r", M, K, 8, x_dtype=dt, n_outlier=2, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    got = host(W.hadamard_rotate(dev(X), b))
    ref, bound = rotation_bound(X, b)
    assert np.all(np.abs(got - ref) <= bound)


# --------------------------------------------------------------------------
# Quantizers: exact on the oracle's rotated input
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,b,dt", [
    (16, 256, 256, "float32"), (37, 4096, 4096, "float16"), (20, 14336, 128, "float16"),
    (3, 192, 64, "float32"), (1, 64, 2, "float16")])
def test_quantize_act_exact_on_oracle_rotation(M, K, b, dt):
    w = synth.small("q", M, K, 8, x_dtype=dt, n_outlier=3, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xr = O.rotate(X, b)
    xq, sx = W.quantize_act_int4(dev(xr), 0)
    pq, ps, _, _ = O.quantize_activation(xr, 0)
    assert np.array_equal(host(sx), ps)
    assert np.array_equal(host(xq), pq)


@pytest.mark.parametrize("M,K,b,dt", [(37, 4096, 4096, "float16"), (20, 14336, 128, "float16"),
                                      (3, 192, 64, "float32"), (1, 64, 2, "float16")])
def test_quantize_act_i8_layout_exact(M, K, b, dt):
    w = synth.small("q8", M, K, 8, x_dtype=dt, n_outlier=3, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xr = O.rotate(X, b)
    xq, sx = W.quantize_act_int4(dev(xr), 0, layout="i8")
    _, ps, pc, _ = O.quantize_activation(xr, 0)
    assert np.array_equal(host(sx), ps)
    assert np.array_equal(codes_from_i8(host(xq)), pc)
    assert np.array_equal(host(xq).view(np.int8), i8_from_codes(pc))


@pytest.mark.parametrize("M,K,b,dt", [(37, 4096, 4096, "float16"), (20, 14336, 128, "float16"),
                                      (3, 256, 64, "float32"), (16, 128, 2, "float16"),
                                      (1, 128, 128, "float32")])
def test_quantize_act_i8_tiled_exact(M, K, b, dt):
    w = synth.small("qt", M, K, 8, x_dtype=dt, n_outlier=3, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xr = O.rotate(X, b)
    xq, sx = W.quantize_act_int4(dev(xr), 0, layout="i8_tiled")
    assert tuple(xq.shape) == (W.pad16(M), K)
    _, ps, pc, _ = O.quantize_activation(xr, 0)
    assert np.array_equal(host(sx), ps)
    got = host(xq)
    assert np.array_equal(untile_codes_i8(got, M).view(np.int8), i8_from_codes(pc))
    # the host tiling of the same bytes agrees on every real row
    ref = tile_codes_i8(i8_from_codes(pc))
    real = untile_codes_i8(ref, M)
    assert np.array_equal(real, untile_codes_i8(got, M))


@pytest.mark.parametrize("M,K,b,dt", [(37, 4096, 4096, "float16"), (20, 14336, 128, "float16"),
                                      (3, 256, 64, "float32"), (100, 1024, 1024, "float16")])
def test_quantize_act_packed_tiled_exact(M, K, b, dt):
    w = synth.small("qpt", M, K, 8, x_dtype=dt, n_outlier=3, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xr = O.rotate(X, b)
    xq, sx = W.quantize_act_int4(dev(xr), 0, layout="packed_tiled")
    assert tuple(xq.shape) == (W.pad16(M), K // 2)
    pq, ps, _, _ = O.quantize_activation(xr, 0)
    assert np.array_equal(host(sx), ps)
    assert np.array_equal(untile_weights(host(xq), M), pq)


def test_quantize_act_exact_unrotated_fp16_and_edge_rows():
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((6, 512)) * 3).astype(np.float16)
    X[1] = 0                                # zero row
    X[2, :] = 0
    X[2, 17] = np.float16(-2.0)             # single element
    X[3] = np.float16(6e-8)                 # fp16 subnormals
    X[4, ::2] = np.float16(1.5)             # ties after scaling
    X[4, 1::2] = np.float16(-10.5)
    xq, sx = W.quantize_act_int4(dev(X), 1)
    pq, ps, _, _ = O.quantize_activation(X.astype(np.float32), 0)
    assert np.array_equal(host(sx), ps)
    assert np.array_equal(host(xq), pq)


def test_quantize_act_tie_breaking_matches_division():
    # Rows built on the boundary cases where x*(1/s) and x/s round apart.
    f = np.float32
    rows = []
    for a in (3.0, 1.0, 0.3, 5.0, 11.0):
        s = f(f(a) / f(7))
        r = f(f(1) / s)
        row = [f(a)]
        for n in range(7):
            xv = f((n + 0.5) * float(s))
            for _ in range(9):
                row.append(xv)
                row.append(-xv)
                xv = np.nextafter(xv, f(np.inf), dtype=np.float32)
        row = (row + [f(0)] * 256)[:256]
        rows.append(row)
    X = np.array(rows, np.float32)
    xq, sx = W.quantize_act_int4(dev(X), 0)
    pq, ps, _, _ = O.quantize_activation(X, 0)
    assert np.array_equal(host(sx), ps)
    assert np.array_equal(host(xq), pq)


@pytest.mark.parametrize("e", [-125, -110, -98, -60, 0, 60, 98, 110, 121])
def test_quantize_act_exact_extreme_scales(e):
    # Rows of fp32 values scaled by 2^e: scales on both sides of the range in
    # which the quotient is refined from a reciprocal.
    rng = np.random.default_rng(1000 + e)
    X = (rng.standard_normal((48, 512)) * np.float64(2.0) ** e).astype(np.float32)
    X[5] = 0
    xq, sx = W.quantize_act_int4(dev(X), 0)
    pq, ps, _, _ = O.quantize_activation(X, 0)
    assert np.array_equal(host(sx), ps)
    assert np.array_equal(host(xq), pq)


def test_quantize_act_exact_random_near_ties():
    # Every element sits within a few ulps of a half-integer multiple of its
    # row's scale: the cases where a reciprocal-based quotient can round the
    # other way.
    rng = np.random.default_rng(11)
    f = np.float32
    M, K = 64, 1024
    X = np.empty((M, K), np.float32)
    for m in range(M):
        amax = f(rng.uniform(0.5, 2.0) * 2.0 ** rng.integers(-20, 20))
        s = f(amax / f(7))
        n = rng.integers(-7, 7, K).astype(np.float64) + 0.5
        base = (n * np.float64(s)).astype(np.float32)
        ulps = rng.integers(-3, 4, K)
        row = base.copy()
        for _ in range(3):
            row = np.where(ulps > 0, np.nextafter(row, f(np.inf)), row)
            row = np.where(ulps < 0, np.nextafter(row, f(-np.inf)), row)
            ulps = ulps - np.sign(ulps)
        row[0] = amax
        row = np.clip(row, -amax, amax)
        X[m] = row
    xq, sx = W.quantize_act_int4(dev(X), 0, layout="i8")
    _, ps, pc, _ = O.quantize_activation(X, 0)
    assert np.array_equal(host(sx), ps)
    assert np.array_equal(codes_from_i8(host(xq)), pc)


@pytest.mark.parametrize("N,K,g,sd", [(64, 256, 0, "float32"), (96, 4096, 0, "float16"),
                                      (40, 14336, 128, "float16"), (24, 512, 64, "float16"),
                                      (8, 4096, 4096, "float32")])
def test_quantize_weight_exact_on_oracle_rotation(N, K, g, sd):
    rng = np.random.default_rng(N + K)
    Wt = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    Wt[:, 5] *= 30
    wr = O.rotate(Wt, 128)
    wq, ws = W.quantize_weight_int4(dev(wr), 0, g, torch.float16 if sd == "float16" else torch.float32)
    oq, os_ = O.quantize_weight(wr, g, sd)
    assert np.array_equal(host(ws), os_)
    assert np.array_equal(host(wq), O.pack_int4(oq))


@pytest.mark.parametrize("g", [0, 64])
def test_quantize_weight_exact_float16_scales_normal_subnormal_zero(g):
    # Row n is scaled by 2^-n, so the float16 scales run from normal through
    # subnormal (where rounding the scale can push a quotient past 7.5 and
    # the clamp decides the code) down to zero.
    rng = np.random.default_rng(77 + g)
    N, K = 48, 512
    Wt = (0.5 * rng.standard_normal((N, K))).astype(np.float32)
    Wt *= (2.0 ** -np.arange(N, dtype=np.float64))[:, None].astype(np.float32)
    wq, ws = W.quantize_weight_int4(dev(Wt), 0, g, torch.float16)
    oq, os_ = O.quantize_weight(Wt, g, "float16")
    assert np.array_equal(host(ws), os_)
    assert np.array_equal(host(wq), O.pack_int4(oq))
    s = os_.astype(np.float32).reshape(-1)
    assert np.any((s > 0) & (s < 2.0 ** -14)) and np.any(s == 0) and np.any(s >= 2.0 ** -14)


@pytest.mark.parametrize("N,K,g,sd", [(64, 256, 0, "float32"), (100, 4096, 0, "float16"),
                                      (40, 14336, 128, "float16"), (8, 4096, 4096, "float32")])
def test_quantize_weight_tiled_exact(N, K, g, sd):
    rng = np.random.default_rng(N + K + 3)
    Wt = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    Wt[:, 9] *= 30
    wr = O.rotate(Wt, 128)
    wq, ws = W.quantize_weight_int4(dev(wr), 0, g, torch.float16 if sd == "float16" else torch.float32,
                                    layout="tiled")
    assert tuple(wq.shape) == (W.pad16(N), K // 2)
    oq, os_ = O.quantize_weight(wr, g, sd)
    assert np.array_equal(host(ws), os_)
    assert np.array_equal(untile_weights(host(wq), N), O.pack_int4(oq))


@pytest.mark.parametrize("N,K,b,g", [(64, 4096, 4096, 0), (48, 14336, 128, 128), (32, 256, 256, 0)])
def test_quantize_weight_fused_rotation(N, K, b, g):
    rng = np.random.default_rng(7)
    Wt = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    wq, ws = W.quantize_weight_int4(dev(Wt), b, g, torch.float16)
    _, os_, oq = O.prepare_weight(Wt, b, g, "float16")
    gq = O.unpack_int4(host(wq))
    diff = gq.astype(np.int16) - oq
    assert np.all(np.abs(diff) <= 1)
    assert np.count_nonzero(diff) <= 1e-4 * diff.size
    rel = np.abs(host(ws).astype(np.float64) - os_.astype(np.float64)) / os_.astype(np.float64)
    assert np.all(rel <= 1e-3)   # fp16 storage: equal or one fp16 ulp apart


@pytest.mark.parametrize("M,K,b,dt", [(16, 256, 256, "float32"), (64, 4096, 4096, "float16"),
                                      (48, 14336, 128, "float16"), (8, 8192, 4096, "float16"),
                                      (5, 2048, 2048, "float16"), (100, 4096, 4096, "float16")])
def test_quantize_act_fused_rotation(M, K, b, dt):
    w = synth.small("f", M, K, 8, x_dtype=dt, n_outlier=4, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xq, sx = W.quantize_act_int4(dev(X), b)
    _, ps, pc, _ = O.quantize_activation(X, b)
    gc = O.unpack_int4(host(xq)).astype(np.int16)
    diff = gc - pc
    assert np.all(np.abs(diff) <= 1)
    assert np.count_nonzero(diff) <= 1e-4 * diff.size
    assert np.all(np.abs(host(sx).astype(np.float64) - ps) <= 1e-6 * ps)


@pytest.mark.parametrize("M,K,b,dt", [(64, 4096, 4096, "float16"), (33, 4096, 1024, "float16"),
                                      (20, 4096, 2048, "float16"), (16, 512, 256, "float32"),
                                      (9, 1024, 128, "float32"), (300, 4096, 4096, "float16"),
                                      (4100, 4096, 128, "float16"), (4100, 4096, 4096, "float16"),
                                      (2500, 14336, 128, "float16"), (9000, 1024, 256, "float16")])
def test_quantize_act_fused_equals_rotate_then_quantize(M, K, b, dt):
    # The fused kernel quantizes x~ = RN(y / sqrt(b)) from the same butterflies
    # as the rotation kernel; when 1 / sqrt(b) is a power of two it divides y by
    # s sqrt(b) instead.  Either way its codes and scales equal those of the
    # exact quantizer applied to the rotation kernel's output.  The larger
    # fp16 cases run several row groups per workgroup (the last one ragged).
    w = synth.small("fr", M, K, 8, x_dtype=dt, n_outlier=4, bos_factor=500.0)
    X = dev(synth.make_inputs(w)["X"])
    xq, sx = W.quantize_act_int4(X, b)
    rq, rs = W.quantize_act_int4(W.hadamard_rotate(X, b), 0)
    assert np.array_equal(host(sx), host(rs))
    assert np.array_equal(host(xq), host(rq))


# --------------------------------------------------------------------------
# Integer GEMM
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (7, 33, 192), (130, 260, 384), (16, 256, 256),
                                   (257, 129, 4096), (64, 64, 14336), (8, 4096, 4096),
                                   (17, 300, 14336), (32, 64, 192), (1000, 6500, 256),
                                   (2048, 4096, 256)])
def test_qgemm_int32_exact(M, N, K):
    rng = np.random.default_rng(M * N + K)
    qx = rng.integers(-8, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qx[0, :] = -8
    qw[0, :] = -8
    _, acc = W.qgemm_w4a4(dev(O.pack_int4(qx)), None, dev(O.pack_int4(qw)), None, 0,
                          want_y=False, want_acc=True)
    assert np.array_equal(host(acc), O.int_gemm(qx, qw))


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (7, 33, 192), (130, 260, 384), (16, 4096, 4096),
                                   (32, 64, 192), (300, 129, 320), (1000, 6500, 256),
                                   (2048, 4096, 4096)])
def test_qgemm_i8_codes_int32_exact(M, N, K):
    rng = np.random.default_rng(M * N + K + 1)
    qx = rng.integers(-8, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qx[0, :] = -8
    qw[0, :] = -8
    _, acc = W.qgemm_w4a4(dev(i8_from_codes(qx).view(np.uint8)), None, dev(O.pack_int4(qw)), None, 0,
                          want_y=False, want_acc=True, layout="i8")
    assert np.array_equal(host(acc), O.int_gemm(qx, qw))


@pytest.mark.parametrize("M,N,K,g,sd", [(33, 70, 256, 0, "float32"), (128, 256, 4096, 0, "float16"),
                                        (40, 96, 1024, 128, "float16"), (17, 50, 384, 64, "float32"),
                                        (64, 128, 14336, 128, "float16"), (8, 4096, 4096, 0, "float16"),
                                        (16, 200, 14336, 128, "float16"), (24, 100, 512, 256, "float32"),
                                        (1000, 6500, 256, 128, "float16"), (5, 40, 1024, 64, "float16")])
@pytest.mark.parametrize("layout", ["packed", "i8"])
def test_qgemm_dequant(M, N, K, g, sd, layout):
    rng = np.random.default_rng(M + N + K + g)
    qx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, (N, K)).astype(np.int8)
    sx = rng.uniform(0.01, 2.0, M).astype(np.float32)
    shape = (N,) if g == 0 else (N, K // g)
    sw = rng.uniform(1e-3, 0.05, shape).astype(np_dtype(sd))
    xin = O.pack_int4(qx) if layout == "packed" else i8_from_codes(qx).view(np.uint8)
    y, acc = W.qgemm_w4a4(dev(xin), dev(sx), dev(O.pack_int4(qw)), dev(sw), g,
                          want_y=True, want_acc=True, layout=layout)
    assert np.array_equal(host(acc), O.int_gemm(qx, qw))
    accs = O.int_gemm(qx, qw) if g == 0 else O.int_gemm_groups(qx, qw, g)
    ref = O.epilogue(accs, sx, sw.astype(np.float32), None).astype(np.float64)
    # float32 epilogue: a few roundings per group term
    G = 1 if g == 0 else K // g
    mag = np.abs(sx)[:, None] * (np.abs(sw.astype(np.float64)).reshape(N, -1).max(axis=1)[None, :]) * 49 * K
    assert np.all(np.abs(host(y) - ref) <= (G + 3) * 2.0 ** -23 * mag)


@pytest.mark.parametrize("M,N,K,g", [(1, 1, 128, 0), (8, 4096, 4096, 0), (16, 300, 14336, 128),
                                     (17, 33, 256, 0), (32, 4096, 4096, 128), (33, 70, 384, 128),
                                     (130, 260, 384, 0), (300, 129, 1024, 256),
                                     (1000, 6500, 256, 128), (2048, 4096, 4096, 0),
                                     (2100, 4100, 1024, 0)])
@pytest.mark.parametrize("codes", ["i8_tiled", "packed_tiled"])
def test_qgemm_tiled_exact_and_dequant(M, N, K, g, codes):
    rng = np.random.default_rng(M * 7 + N + K + g)
    qx = rng.integers(-8, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qx[0, :] = -8
    qw[0, :] = -8
    sx = rng.uniform(0.01, 2.0, M).astype(np.float32)
    shape = (N,) if g == 0 else (N, K // g)
    sw = rng.uniform(1e-3, 0.05, shape).astype(np.float16)
    xin = (tile_codes_i8(i8_from_codes(qx), rng) if codes == "i8_tiled"
           else tile_weights(O.pack_int4(qx), rng))
    y, acc = W.qgemm_w4a4(dev(xin), dev(sx), dev(tile_weights(O.pack_int4(qw), rng)), dev(sw), g,
                          want_y=True, want_acc=True, layout=codes, w_layout="tiled")
    assert np.array_equal(host(acc), O.int_gemm(qx, qw))
    accs = O.int_gemm(qx, qw) if g == 0 else O.int_gemm_groups(qx, qw, g)
    ref = O.epilogue(accs, sx, sw.astype(np.float32), None).astype(np.float64)
    G = 1 if g == 0 else K // g
    mag = np.abs(sx)[:, None] * (np.abs(sw.astype(np.float64)).reshape(N, -1).max(axis=1)[None, :]) * 64 * K
    assert np.all(np.abs(host(y) - ref) <= (G + 3) * 2.0 ** -23 * mag)


# --------------------------------------------------------------------------
# Low-rank projection
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,r,dt", [(16, 256, 8, "float32"), (8, 4096, 64, "float16"),
                                      (100, 4096, 32, "float16"), (5, 192, 256, "float16"),
                                      (1, 64, 8, "float16"), (16, 14336, 40, "float16"),
                                      (11, 2112, 24, "float16"), (17, 4096, 64, "float16"),
                                      # the staged prefill kernel: ragged rows, one to 28 stages,
                                      # ranks below 16 and 32
                                      (1030, 4096, 32, "float16"), (1024, 14336, 32, "float16"),
                                      (2048, 1024, 16, "float16"), (1100, 512, 24, "float16"),
                                      (1024, 2560, 8, "float16"), (4096, 4096, 32, "float16")])
def test_lowrank_project(M, K, r, dt):
    w = synth.small("l", M, K, 8, x_dtype=dt, rank=r)
    d = synth.make_inputs(w)
    t = host(W.lowrank_project(dev(d["X"]), dev(d["A"].T)))
    X64, A64 = d["X"].astype(np.float64), d["A"].astype(np.float64)
    ref = X64 @ A64
    bound = K * 2.0 ** -23 * (np.abs(X64) @ np.abs(A64))
    assert np.all(np.abs(t - ref) <= bound)


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def forward_codes(w, Xd, wqd, wsd, Ad, Bd, w_layout, act_bits=4):
    """Runs qlinear_forward with an explicit workspace and returns Y and the
    activation codes [M, K] and scales [M] the call left in that workspace."""
    ws_buf = W.qlinear_workspace(w.M, w.N, w.K, w.rank, DEV)
    y = host(W.qlinear_forward(Xd, wqd, wsd, w.had_block, w.w_group, Ad, Bd, workspace=ws_buf,
                               w_layout=w_layout, act_bits=act_bits))
    wsb = host(ws_buf)
    co, cl, so = W.qlinear_workspace_layout(w.M, w.N, w.K, w.rank, w_layout, w.w_group, act_bits)
    kind, codes = workspace_codes(wsb, co, w.M, w.K, cl)
    gc = (O.unpack_int4(codes) if kind == "packed" else codes).astype(np.int16)
    return y, gc, wsb[so:so + 4 * w.M].view(np.float32).copy()


def run_layer(w, rows=None, w_layout="rowmajor"):
    """GPU qlinear_forward vs the oracle on one workload; returns stats.  The
    reference epilogue is evaluated on the codes and scales the call left in
    its workspace."""
    d = synth.make_inputs(w, rows)
    X, Wt, A, B = d["X"], d["W"], d["A"], d["B"]
    wq, ws, _ = O.prepare_weight(Wt, w.had_block, w.w_group, w.w_scale_dtype)
    Xd, wsd = dev(X), dev(ws)
    wqd = dev(tile_weights(wq) if w_layout == "tiled" else wq)
    Ad = dev(A.T) if A is not None else None   # the ABI takes At [r, K], Bt [N, r]
    Bd = dev(B.T) if B is not None else None
    y, gc, gsx = forward_codes(w, Xd, wqd, wsd, Ad, Bd, w_layout)
    _, ps, pc, _ = O.quantize_activation(X, w.had_block)
    y_on_gpu_codes = O.qlinear_from_codes(gc, gsx, wq, ws, w.w_group, X, A, B)
    y_oracle = O.qlinear_forward(X, wq, ws, w.had_block, w.w_group, A, B)
    rms = float(np.sqrt(np.mean(y_oracle.astype(np.float64) ** 2)))
    diff = gc - pc
    return dict(y=y, y_codes=y_on_gpu_codes, y_oracle=y_oracle, rms=rms, diff=diff,
                gsx=gsx, psx=ps)


def check_layer(st):
    assert np.all(np.abs(st["diff"]) <= 1)
    assert np.count_nonzero(st["diff"]) <= 1e-4 * st["diff"].size
    assert np.all(np.abs(st["gsx"].astype(np.float64) - st["psx"]) <= 1e-6 * st["psx"])
    check_y(st["y"], st["y_codes"], st["y_oracle"])


@pytest.mark.parametrize("wl", ["rowmajor", "tiled"])
@pytest.mark.parametrize("w", [synth.TINY, synth.DECODE], ids=lambda w: w.name)
def test_qlinear_full_size(w, wl):
    st = run_layer(w, w_layout=wl)
    check_layer(st)
    print(w.name, wl, "max|Y-Y_oracle|/RMS =",
          float(np.max(np.abs(st["y"] - st["y_oracle"])) / st["rms"]))


@pytest.mark.parametrize("wl", ["rowmajor", "tiled"])
def test_qlinear_prefill_full_size(wl):
    st = run_layer(synth.PREFILL, w_layout=wl)
    check_layer(st)
    print("prefill", wl, "max|Y-Y_oracle|/RMS =",
          float(np.max(np.abs(st["y"] - st["y_oracle"])) / st["rms"]))


@pytest.mark.parametrize("M,K,N,b,g,r,dt", [
    (1, 256, 64, 256, 0, 0, "float16"), (130, 1024, 260, 128, 128, 16, "float16"),
    (33, 4096, 100, 4096, 0, 64, "float16"), (65, 14336, 96, 128, 128, 32, "float16"),
    (20, 4096, 520, 128, 128, 24, "float16"), (300, 1024, 1030, 256, 0, 40, "float16"),
    (40, 384, 100, 128, 0, 0, "float32"), (16, 512, 48, 1, 0, 8, "float16")])
def test_qlinear_tiled_weights_ragged(M, K, N, b, g, r, dt):
    w = synth.small("ragt", M, K, N, x_dtype=dt, had_block=b, w_group=g, rank=r,
                    w_scale_dtype="float16" if dt == "float16" else "float32")
    check_layer(run_layer(w, w_layout="tiled"))


@pytest.mark.parametrize("M,K,N,b,g,r,dt", [
    (1, 256, 64, 256, 0, 0, "float16"), (7, 192, 33, 64, 64, 4, "float32"),
    (130, 1024, 260, 128, 128, 16, "float16"), (33, 4096, 100, 4096, 0, 64, "float16"),
    (65, 14336, 96, 128, 128, 32, "float16"), (16, 512, 48, 1, 0, 8, "float16"),
    (20, 4096, 520, 128, 128, 24, "float16"), (300, 1024, 1030, 256, 0, 40, "float16"),
    (520, 4096, 700, 4096, 0, 8, "float16"), (9, 384, 50, 128, 0, 256, "float16"),
    (300, 320, 200, 64, 64, 8, "float16"), (40, 192, 100, 64, 0, 0, "float32")])
def test_qlinear_ragged_shapes(M, K, N, b, g, r, dt):
    w = synth.small("rag", M, K, N, x_dtype=dt, had_block=b, w_group=g, rank=r,
                    w_scale_dtype="float16" if dt == "float16" else "float32")
    check_layer(run_layer(w))


@pytest.mark.parametrize("wl", ["rowmajor", "tiled"])
@pytest.mark.parametrize("M,K", [(8, 6144), (8, 12288), (8, 5632), (16, 2816), (3, 6144)])
def test_qlinear_decode_fused_projection_narrow_plans(M, K, wl):
    # Decode-sized fp16 calls fold T = X . A into the rotation launch; for
    # these K the rotation plan has fewer than 256 threads per workgroup, and
    # the projection workgroups must still run with all 256.
    w = synth.small("dnp", M, K, 520, had_block=128, rank=64)
    check_layer(run_layer(w, w_layout=wl))


def test_qlinear_empty_is_noop():
    y = torch.full((0, 16), 3.0, device=DEV)
    out = W.qlinear_forward(torch.empty((0, 256), dtype=torch.float16, device=DEV),
                            torch.zeros((16, 128), dtype=torch.uint8, device=DEV),
                            torch.ones(16, dtype=torch.float16, device=DEV), 256, 0, y=y,
                            workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert out.shape == (0, 16)


# --------------------------------------------------------------------------
# W4A8 layers: 8-bit activations (qmax 127) beside the 4-bit weights
# --------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["i8", "i8_tiled"])
@pytest.mark.parametrize("M,K,b,dt", [(37, 4096, 4096, "float16"), (20, 14336, 128, "float16"),
                                      (3, 256, 64, "float32"), (130, 1024, 1024, "float16")])
def test_quantize_act_int8_exact_on_oracle_rotation(M, K, b, dt, layout):
    w = synth.small("q8b", M, K, 8, x_dtype=dt, n_outlier=3, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xr = O.rotate(X, b)
    xq, sx = W.quantize_act_int8(dev(xr), 0, layout=layout)
    _, ps, pc, _ = O.quantize_activation(xr, 0, qmax=127)
    assert np.array_equal(host(sx), ps)
    got = host(xq)
    if layout == "i8_tiled":
        got = untile_codes_i8(got, M)
    assert np.array_equal(codes_from_i8(got), pc)


def test_quantize_act_int8_ties_and_extremes():
    f = np.float32
    rows = []
    for a in (127.0, 3.0, 1e-30, 5e30):
        s = f(f(a) / f(127))
        row = [f(a)]
        for n in (0, 1, 2, 61, 62, 125, 126):
            xv = f((n + 0.5) * float(s))
            for _ in range(3):
                row += [xv, -xv]
                xv = np.nextafter(xv, f(np.inf), dtype=np.float32)
        rows.append((row + [f(0)] * 256)[:256])
    X = np.array(rows, np.float32)
    xq, sx = W.quantize_act_int8(dev(X), 0)
    _, ps, pc, _ = O.quantize_activation(X, 0, qmax=127)
    assert np.array_equal(host(sx), ps)
    assert np.array_equal(codes_from_i8(host(xq)), pc)


@pytest.mark.parametrize("M,K,b,layout", [(64, 4096, 4096, "i8"), (48, 14336, 128, "i8"), (8, 4096, 4096, "i8"),
                                          (130, 4096, 4096, "i8_tiled"), (2048, 4096, 4096, "i8_tiled"),
                                          (300, 6144, 128, "i8_tiled"), (97, 8192, 1024, "i8_tiled")])
def test_quantize_act_int8_fused_rotation(M, K, b, layout):
    # fp32 FWHT against the float64 rotation: every flip is one step and at
    # most 0.01% of the codes flip (the 4-bit bar; measured ~4e-6 here).  The
    # tiled cases of fp16 rows take the rotation on the matrix
    # instruction.
    w = synth.small("f8", M, K, 8, n_outlier=4, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xq, sx = W.quantize_act_int8(dev(X), b, layout=layout)
    _, ps, pc, _ = O.quantize_activation(X, b, qmax=127)
    got = host(xq) if layout == "i8" else untile_codes_i8(host(xq), M)
    diff = codes_from_i8(got).astype(np.int16) - pc
    print("int8 fused rotation: fraction of codes one step off =", np.count_nonzero(diff) / diff.size)
    assert np.all(np.abs(diff) <= 1)
    assert np.count_nonzero(diff) <= 1e-4 * diff.size
    assert np.all(np.abs(host(sx).astype(np.float64) - ps) <= 1e-6 * ps)


@pytest.mark.parametrize("layout", ["i8", "i8_tiled"])
@pytest.mark.parametrize("M,N,K", [(7, 33, 256), (130, 260, 1024), (2048, 4096, 4096), (16, 300, 14336)])
def test_qgemm_int8_codes_exact(M, N, K, layout):
    rng = np.random.default_rng(M + N + K + 5)
    qx = rng.integers(-127, 128, (M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qx[0, :] = -127
    qw[0, :] = -8
    if layout == "i8":
        xin, win, wl = i8_from_codes(qx).view(np.uint8), O.pack_int4(qw), "rowmajor"
    else:
        xin, win, wl = tile_codes_i8(i8_from_codes(qx), rng), tile_weights(O.pack_int4(qw), rng), "tiled"
    _, acc = W.qgemm_w4a4(dev(xin), None, dev(win), None, 0, want_y=False, want_acc=True,
                          layout=layout, w_layout=wl, M=M, N=N)
    assert np.array_equal(host(acc), O.int_gemm(qx, qw))


def run_layer_w4a8(w, w_layout):
    d = synth.make_inputs(w)
    X, Wt, A, B = d["X"], d["W"], d["A"], d["B"]
    wq, ws, _ = O.prepare_weight(Wt, w.had_block, w.w_group, w.w_scale_dtype)
    Xd = dev(X)
    wqd = dev(tile_weights(wq) if w_layout == "tiled" else wq)
    Ad = dev(A.T) if A is not None else None
    Bd = dev(B.T) if B is not None else None
    y, gc, gsx = forward_codes(w, Xd, wqd, dev(ws), Ad, Bd, w_layout, act_bits=8)
    y_codes = O.qlinear_from_codes(gc, gsx, wq, ws, w.w_group, X, A, B)
    y_or = O.qlinear_forward(X, wq, ws, w.had_block, w.w_group, A, B, act_bits=8)
    rms = float(np.sqrt(np.mean(y_or.astype(np.float64) ** 2)))
    return y, y_codes, y_or, rms


@pytest.mark.parametrize("wl", ["rowmajor", "tiled"])
@pytest.mark.parametrize("w", [synth.PREFILL, synth.DECODE, synth.TINY,
                               synth.small("w8r", 300, 1024, 1030, had_block=256, rank=40),
                               synth.small("w8g", 65, 14336, 96, had_block=128, w_group=128, rank=32)],
                         ids=lambda w: w.name)
def test_w4a8_layer(w, wl):
    if wl == "tiled" and w.K % 128:
        pytest.skip("tiled weights need K % 128 == 0")
    y, y_codes, y_or, rms = run_layer_w4a8(w, wl)
    check_y(y, y_codes, y_or)
    print(w.name, wl, "W4A8 max|Y-Y_oracle|/RMS =", float(np.max(np.abs(y - y_or)) / rms))
