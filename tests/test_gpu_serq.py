"""Parity of the in-GEMM residual of salient channels (SERQ page,
"Metodología" items 2-3) against the CPU oracle, through the C ABI.

Bars:
* weight codes, scales and residual codes on the oracle's rotation
  (had_block 0): bit-exact, including the zero residual tiles past r;
* with the fused rotation: weight codes within one step on at most 0.01%,
  and the combined value 8 q + q_r within one step on at most 0.1% of the
  salient elements (the residual grid is 8 times finer);
* the integer 8 sum_k q_x q_w + sum_{k<r} q_x q_r: bit-exact;
* y = s_x s_w acc / 8 in float32: |y - y_oracle| <= 2^-21 |y_oracle| + tiny
  (the int32 -> float conversion, the scale product and the final product);
* the layer: codes as for the plain layer (one step on at most 0.01%),
  max |Y - epilogue(GPU codes)| <= 1e-3 RMS(Y_oracle).
"""
import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth
from bit_gemm_block_amd import w4a4 as W
from bars import check_y
from layouts import tile_weights, tile_weights_residual, untile_weights_residual, workspace_codes

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def ext_weights(q, qr, rng=None):
    """Host residual-extended tiled weights from codes and residual codes."""
    N, K = q.shape
    rp = W.res_pad(qr.shape[1])
    res = np.zeros((N, rp), np.int8)
    res[:, :qr.shape[1]] = qr
    return tile_weights_residual(O.pack_int4(q), O.pack_int4(res), rng)


def split_codes(ext, N, K, r):
    main, res = untile_weights_residual(ext, N, K)
    rc = O.unpack_int4(res)
    return O.unpack_int4(main), rc[:, :r], rc[:, r:]


# --------------------------------------------------------------------------
# Weight preparation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,r,sd", [(64, 256, 32, "float32"), (100, 4096, 64, "float16"),
                                      (48, 14336, 200, "float16"), (17, 1024, 1024, "float16"),
                                      (33, 384, 1, "float32"), (16, 512, 0, "float16")])
def test_quantize_weight_residual_exact_on_oracle_rotation(N, K, r, sd):
    rng = np.random.default_rng(N + K + r)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    w[:, 5] *= 40
    print("residual weights", N, K, r, sd, flush=True)
    wq, ws = W.quantize_weight_residual_int4(dev(w), 0, r, torch.float16 if sd == "float16" else torch.float32)
    q, s, qr = O.quantize_weight_residual(w, r, sd)
    gq, gqr, gpad = split_codes(host(wq), N, K, r)
    assert np.array_equal(host(ws), s)
    assert np.array_equal(gq, q)
    assert np.array_equal(gqr, qr)
    assert not gpad.any()


@pytest.mark.parametrize("N,K,b,r", [(96, 4096, 4096, 64), (64, 14336, 128, 128), (40, 1024, 256, 100)])
def test_quantize_weight_residual_fused_rotation(N, K, b, r):
    rng = np.random.default_rng(7)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    wq, ws = W.quantize_weight_residual_int4(dev(w), b, r, torch.float16)
    q, s, qr = O.quantize_weight_residual(O.rotate(w, b), r, "float16")
    gq, gqr, gpad = split_codes(host(wq), N, K, r)
    d = gq.astype(np.int16) - q
    assert np.all(np.abs(d) <= 1) and np.count_nonzero(d) <= 1e-4 * d.size
    comb = (8 * gq[:, :r].astype(np.int32) + gqr) - (8 * q[:, :r].astype(np.int32) + qr)
    assert np.all(np.abs(comb) <= 1) and np.count_nonzero(comb) <= 1e-3 * comb.size
    assert not gpad.any()


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K,r", [(1, 1, 128, 1), (7, 33, 256, 32), (130, 260, 1024, 128),
                                     (2048, 4096, 4096, 32), (300, 129, 14336, 200),
                                     (2100, 4100, 1024, 256), (16, 300, 4096, 4096),
                                     (65, 70, 2048, 0), (30, 70, 2048, 100), (8, 4096, 4096, 64),
                                     (17, 33, 1024, 0)])
def test_qgemm_residual_exact_and_dequant(M, N, K, r):
    rng = np.random.default_rng(M + N + K + r)
    qx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    qx[0] = -7
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qw[0] = -8
    qr = rng.integers(-8, 8, (N, r)).astype(np.int8)
    if r:
        qr[0] = -8
    sx = rng.uniform(0.01, 2.0, M).astype(np.float32)
    sw = rng.uniform(1e-3, 0.05, N).astype(np.float16)
    xin = tile_weights(O.pack_int4(qx), rng)
    print("qgemm_residual", M, N, K, r, flush=True)
    y, acc = W.qgemm_residual(dev(xin), dev(sx), dev(ext_weights(qw, qr, rng)), dev(sw), r, M, N, K,
                              want_acc=True)
    ref_acc = O.residual_int_gemm(qx, qw, qr)
    assert np.array_equal(host(acc).astype(np.int64), ref_acc)
    ref = O.residual_from_codes(qx, sx, qw, sw.astype(np.float32), qr).astype(np.float64)
    assert np.all(np.abs(host(y) - ref) <= 2.0 ** -21 * np.abs(ref) + 1e-30)


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def run_residual_layer(w, r, sample_rows=None):
    d = synth.make_inputs(w)
    X, Wt = d["X"], d["W"]
    b = w.had_block
    wq, ws, q, qr = O.prepare_weight_residual(Wt, b, r, w.w_scale_dtype)
    wqd = dev(ext_weights(q, qr))
    Xd = dev(X)
    print("residual layer", w.name, w.M, w.K, w.N, b, r, flush=True)
    ws_buf = W.qlinear_workspace(w.M, w.N, w.K, 0, DEV)
    y = host(W.qlinear_forward_residual(Xd, wqd, dev(ws), r, b, workspace=ws_buf))
    # the codes and scales the layer left in its workspace
    wsb = host(ws_buf)
    co, cl, so = W.qlinear_workspace_layout(w.M, w.N, w.K, 0, "tiled", 0)
    assert cl == "packed_tiled"
    _, packed = workspace_codes(wsb, co, w.M, w.K, cl)
    gc, gs = O.unpack_int4(packed), wsb[so:so + 4 * w.M].view(np.float32)
    rows = np.arange(w.M) if sample_rows is None else sample_rows
    _, ps, pc, _ = O.quantize_activation(X[rows], b)
    diff = gc[rows].astype(np.int16) - pc
    assert np.all(np.abs(diff) <= 1) and np.count_nonzero(diff) <= 1e-4 * diff.size
    assert np.all(np.abs(gs[rows].astype(np.float64) - ps) <= 1e-6 * ps)
    y_codes = O.residual_from_codes(gc[rows], gs[rows], q, ws.astype(np.float32), qr)
    y_oracle = O.qlinear_forward_residual(X[rows], wq, ws, qr, b)
    rms = float(np.sqrt(np.mean(y_oracle.astype(np.float64) ** 2)))
    check_y(y[rows], y_codes, y_oracle)
    return float(np.max(np.abs(y[rows] - y_oracle)) / rms)


@pytest.mark.parametrize("M,K,N,b,r,dt", [
    (1, 256, 64, 256, 32, "float16"), (130, 1024, 260, 128, 128, "float16"),
    (33, 4096, 100, 4096, 64, "float16"), (65, 14336, 96, 128, 200, "float16"),
    (40, 384, 100, 128, 5, "float32"), (300, 1024, 1030, 256, 0, "float16"),
    (8, 4096, 96, 4096, 40, "float16"), (17, 2048, 100, 128, 72, "float16")])
def test_qlinear_residual_ragged(M, K, N, b, r, dt):
    w = synth.small("res", M, K, N, x_dtype=dt, had_block=b,
                    w_scale_dtype="float16" if dt == "float16" else "float32")
    run_residual_layer(w, r)


@pytest.mark.parametrize("name,r", [("prefill_2048x4096x4096", 64), ("llama3_8b_o_4096x4096x4096", 32)])
def test_qlinear_residual_full_size(name, r):
    w = synth.by_name(name)
    rows = np.unique(np.r_[0, 1, np.random.default_rng(3).integers(0, w.M, 40), w.M - 1])
    print(name, "residual max|Y-Y_oracle|/RMS =", run_residual_layer(w, r, rows))


def test_residual_weights_from_gpu_prep_drive_the_layer():
    # The GPU weight preparation and the GPU layer together, against the
    # oracle's layer on the same weights (rotation 128, fp16 scales).
    w = synth.small("resprep", 64, 2048, 300, had_block=128)
    d = synth.make_inputs(w)
    r = 96
    wq, ws = W.quantize_weight_residual_int4(dev(d["W"]), 128, r, torch.float16)
    N, K = w.N, w.K
    gq, gqr, _ = split_codes(host(wq), N, K, r)
    gws = host(ws)
    y = host(W.qlinear_forward_residual(dev(d["X"]), wq, ws, r, 128))
    gxq, gsx = W.quantize_act_int4(dev(d["X"]), 128)
    y_codes = O.residual_from_codes(O.unpack_int4(host(gxq)), host(gsx), gq, gws.astype(np.float32), gqr)
    owq, ows, _, oqr = O.prepare_weight_residual(d["W"], 128, r, "float16")
    y_or = O.qlinear_forward_residual(d["X"], owq, ows, oqr, 128)
    rms = float(np.sqrt(np.mean(y_or.astype(np.float64) ** 2)))
    assert np.max(np.abs(y - y_codes)) <= 1e-3 * rms
