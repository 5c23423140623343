"""Parity of the FP6 tiled operands (include/w4a4.h "FP6 tiled layouts": the
same int4 codes stored as E2M3 numbers for the FP6 matrix instruction)
against the CPU oracle, through the C ABI.

Bars:
* activation codes on the oracle's rotation (had_block 0): the decoded tiles
  are the oracle's codes and the scales the oracle's, bit-exact; with the
  fused rotation, the decoded tiles equal the packed codes of the same call
  in the packed layout (same kernel and arithmetic), bit-exact;
* weights: the decoded tiles equal the tiled int4 weights of the same call,
  and the scales are equal, bit-exact (per channel and grouped);
* GEMM: the product (float32 sums of exact integers) equals the oracle's
  int64 product bit for bit; y within the bound of the int8 GEMM's test
  (per channel), or within a bound for float32 group sums (grouped);
* layer: codes within one step on at most 0.01% of the oracle's, y within
  the layer bars of tests/bars.py, and equal bit for bit to the layer on
  offset-binary (per channel) or plain tiled (grouped) weights of the same
  codes: the same integer sums scaled by the same float32 operations.
"""
import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth
from bit_gemm_block_amd import w4a4 as W
from layouts import (ob_weights, tile_f6, tile_weights, untile_f6, untile_weights,
                     workspace_codes)
from bars import check_y

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# M <= 64 rows take the wide rotation shapes (16 codes per lane: two lanes per
# FP6 chunk); K = 128 the smallest segment; the others 32 or 64 per lane.
@pytest.mark.parametrize("M,K,b,dt", [(37, 4096, 4096, "float16"), (20, 14336, 128, "float16"),
                                      (3, 256, 64, "float32"), (100, 1024, 1024, "float16"),
                                      (2048, 4096, 4096, "float16"), (1, 128, 128, "float16"),
                                      (65, 14336, 128, "float32")])
def test_quantize_act_f6_exact(M, K, b, dt):
    w = synth.small("qf6", M, K, 8, x_dtype=dt, n_outlier=3, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xr = O.rotate(X, b)
    print("quantize_act f6", M, K, b, dt, flush=True)
    xq, sx = W.quantize_act_int4(dev(xr), 0, layout="f6_tiled")
    assert tuple(xq.shape) == (W.pad16(M), 3 * K // 4)
    _, ps, pc, _ = O.quantize_activation(xr, 0)
    assert np.array_equal(host(sx), ps)
    assert np.array_equal(untile_f6(host(xq), M, K), pc)


@pytest.mark.parametrize("M,K,b,dt", [(130, 4096, 4096, "float32"), (37, 4096, 4096, "float16"),
                                      (9, 14336, 128, "float16"), (300, 1024, 256, "float16"),
                                      (60, 4096, 128, "float16"), (12, 2048, 256, "float32")])
def test_quantize_act_f6_fused_matches_packed(M, K, b, dt):
    # FP6 tiles against packed tiles of the same call: the same kernel (the
    # matrix-instruction rotation for fp16 rows with K a multiple of 2048, of
    # 4096 for b = 4096; the butterfly kernel otherwise) and the same
    # arithmetic, so the same codes and scales.
    w = synth.small("qf6f", M, K, 8, x_dtype=dt, n_outlier=3, bos_factor=500.0)
    Xd = dev(synth.make_inputs(w)["X"])
    print("quantize_act f6 fused", M, K, b, dt, flush=True)
    xf, sf = W.quantize_act_int4(Xd, b, layout="f6_tiled")
    xp, sp = W.quantize_act_int4(Xd, b, layout="packed_tiled")
    assert np.array_equal(host(sf), host(sp))
    assert np.array_equal(untile_f6(host(xf), M, K), O.unpack_int4(untile_weights(host(xp), M)))


@pytest.mark.parametrize("M,K", [(65, 2048), (130, 4096), (4100, 4096), (200, 14336),
                                 (77, 16384), (1000, 6144)])
def test_quantize_act_f6_b128_matrix_rotation(M, K):
    # FP6 codes of fp16 rows with b = 128: the transform
    # runs on the fp16 matrix instruction, so its float32 sums round in
    # another order than the butterflies'; against the oracle the codes meet
    # the fused-path bar (at most 0.01% differ, each by one step) and the
    # scales agree within 1e-6.  A wrong lane exchange or tile offset would
    # move whole 8-code units and fail the bar at once.
    w = synth.small("qm128", M, K, 8, n_outlier=3, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    print("quantize_act f6 b128 matrix", M, K, flush=True)
    xq, sx = W.quantize_act_int4(dev(X), 128, layout="f6_tiled")
    _, ps, pc, _ = O.quantize_activation(O.rotate(X, 128), 0)
    got = untile_f6(host(xq), M, K).astype(np.int16)
    diff = got - pc.astype(np.int16)
    assert np.all(np.abs(diff) <= 1)
    assert np.count_nonzero(diff) <= 1e-4 * diff.size
    assert np.all(np.abs(host(sx).astype(np.float64) - ps) <= 1e-6 * ps)
    # the packed codes of the butterfly kernel meet the same bar against these
    xp, sp = W.quantize_act_int4(dev(X), 128, layout="packed")
    d2 = got - O.unpack_int4(host(xp)).astype(np.int16)
    assert np.all(np.abs(d2) <= 1)
    assert np.count_nonzero(d2) <= 2e-4 * d2.size


@pytest.mark.parametrize("N,K,b,g,sdt", [(4096, 4096, 4096, 0, torch.float16),
                                         (100, 14336, 128, 128, torch.float16),
                                         (33, 1024, 256, 0, torch.float32),
                                         (70, 4096, 128, 256, torch.float32)])
def test_quantize_weight_f6_matches_tiled(N, K, b, g, sdt):
    rng = np.random.default_rng(N + K)
    Wt = dev(rng.standard_normal((N, K)).astype(np.float16 if sdt == torch.float16 else np.float32))
    print("quantize_weight f6", N, K, b, g, flush=True)
    wf, sf = W.quantize_weight_int4(Wt, b, g, sdt, layout="tiled_f6")
    wt, st = W.quantize_weight_int4(Wt, b, g, sdt, layout="tiled")
    assert tuple(wf.shape) == (W.pad16(N), 3 * K // 4)
    assert np.array_equal(host(sf), host(st))
    assert np.array_equal(untile_f6(host(wf), N, K),
                          O.unpack_int4(untile_weights(host(wt), N)))


def f6_operands(qx, qw, rng):
    return tile_f6(qx, rng), tile_f6(qw, rng)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (8, 4096, 4096), (17, 33, 256), (32, 300, 14336),
                                   (33, 70, 384), (130, 260, 384), (300, 129, 1024),
                                   (2048, 4096, 4096), (2100, 4100, 1024), (4096, 4096, 128),
                                   (129, 4096, 16384)])
def test_qgemm_f6_exact_and_dequant(M, N, K):
    rng = np.random.default_rng(M * 5 + N + K)
    qx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, (N, K)).astype(np.int8)
    qx[0, :] = -7   # the largest sums of either sign
    qw[0, :] = -7
    qx[-1, :] = 7
    qw[-1, :] = 7
    sx = rng.uniform(0.01, 2.0, M).astype(np.float32)
    sw = rng.uniform(1e-3, 0.05, N).astype(np.float16)
    xin, win = f6_operands(qx, qw, rng)
    print("qgemm f6", M, N, K, flush=True)
    y, acc = W.qgemm_w4a4(dev(xin), dev(sx), dev(win), dev(sw), 0, want_y=True, want_acc=True,
                          layout="f6_tiled", w_layout="tiled_f6", M=M, N=N)
    ref_acc = O.int_gemm(qx, qw)
    assert np.array_equal(host(acc), ref_acc)
    ref = O.epilogue(ref_acc, sx, sw.astype(np.float32), None).astype(np.float64)
    mag = np.abs(sx)[:, None] * np.abs(sw.astype(np.float64))[None, :] * 64 * K
    assert np.all(np.abs(host(y) - ref) <= 4 * 2.0 ** -23 * mag)


@pytest.mark.parametrize("M,N,K,g", [(130, 260, 1024, 128), (2048, 4096, 4096, 128),
                                     (40, 96, 14336, 128), (300, 200, 2048, 512),
                                     (4096, 512, 14336, 128)])
def test_qgemm_f6_grouped(M, N, K, g):
    rng = np.random.default_rng(M + N * 3 + K + g)
    qx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, (N, K)).astype(np.int8)
    sx = rng.uniform(0.01, 2.0, M).astype(np.float32)
    sw = rng.uniform(1e-3, 0.05, (N, K // g)).astype(np.float16)
    xin, win = f6_operands(qx, qw, rng)
    print("qgemm f6 grouped", M, N, K, g, flush=True)
    y, acc = W.qgemm_w4a4(dev(xin), dev(sx), dev(win), dev(sw), g, want_y=True, want_acc=True,
                          layout="f6_tiled", w_layout="tiled_f6", M=M, N=N)
    assert np.array_equal(host(acc), O.int_gemm(qx, qw))
    groups = O.int_gemm_groups(qx, qw, g)
    ref = O.epilogue(groups, sx, sw.astype(np.float32), None).astype(np.float64)
    # float32 group sums: one rounding per fma and per scale product
    mag = np.abs(sx)[:, None] * (np.abs(sw.astype(np.float64)).sum(axis=1) * 49 * g)[None, :]
    assert np.all(np.abs(host(y) - ref) <= (K // g + 4) * 2.0 ** -23 * mag)


def test_qgemm_f6_rejects_mixed_layouts():
    M, N, K = 64, 32, 256
    sx = torch.ones(M, device=DEV)
    sw = torch.ones(N, device=DEV, dtype=torch.float16)
    x6 = torch.zeros((W.pad16(M), 3 * K // 4), dtype=torch.uint8, device=DEV)
    wt = torch.zeros((W.pad16(N), K // 2), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), device=DEV)
    for xl, xb, wl, wb in ((W.CODES_F6_TILED, x6, W.WEIGHTS_TILED, wt),
                           (W.CODES_PACKED_TILED, wt, W.WEIGHTS_TILED_F6, x6)):
        st = W.lib().w4a4_qgemm_w4a4(W._ptr(xb), xl, W._ptr(sx), W._ptr(wb), wl, W._ptr(sw), W.F16,
                                     0, M, N, K, W._ptr(y), None, None)
        assert st == W.ERR_INVALID_ARG
    # the 8-bit activations of W4A8 have no FP6 form
    st = W.lib().w4a8_qlinear_forward(W._ptr(y), W.F32, W._ptr(x6), W.WEIGHTS_TILED_F6, W._ptr(sw),
                                      W.F16, M, N, K, 256, 0, None, None, 0, W._ptr(y),
                                      W._ptr(y), y.numel() * 4, None)
    assert st == W.ERR_UNSUPPORTED


def run_layer_f6(w, rows=None):
    d = synth.make_inputs(w, rows)
    X, Wt, A, B = d["X"], d["W"], d["A"], d["B"]
    wq, ws, qw = O.prepare_weight(Wt, w.had_block, w.w_group, w.w_scale_dtype)
    N, K = Wt.shape
    M = X.shape[0]
    Xd, wsd = dev(X), dev(ws)
    Ad = dev(A.T) if A is not None else None
    Bd = dev(B.T) if B is not None else None
    print("layer f6", w.name, M, K, N, w.had_block, w.w_group, w.rank, flush=True)
    ws_buf = W.qlinear_workspace(M, N, K, w.rank, DEV)
    y = host(W.qlinear_forward(Xd, dev(tile_f6(qw)), wsd, w.had_block, w.w_group, Ad, Bd,
                               workspace=ws_buf, w_layout="tiled_f6"))
    wsb = host(ws_buf)
    co, cl, so = W.qlinear_workspace_layout(M, N, K, w.rank, "tiled_f6", w.w_group)
    assert cl == "f6_tiled"
    _, gc = workspace_codes(wsb, co, M, K, cl)
    gc = gc.astype(np.int16)
    gsx = wsb[so:so + 4 * M].view(np.float32)
    _, ps, pc, _ = O.quantize_activation(X, w.had_block)
    diff = gc - pc
    assert np.all(np.abs(diff) <= 1) and np.count_nonzero(diff) <= 1e-4 * diff.size + 1
    assert np.all(np.abs(gsx.astype(np.float64) - ps) <= 1e-6 * ps)
    y_codes = O.qlinear_from_codes(gc, gsx, wq, ws, w.w_group, X, A, B)
    y_oracle = O.qlinear_forward(X, wq, ws, w.had_block, w.w_group, A, B)
    check_y(y, y_codes, y_oracle)
    # the same codes through the int8 instruction
    wt = tile_weights(wq)
    if w.w_group == 0:
        y_int = host(W.qlinear_forward(Xd, dev(ob_weights(wt, N, K)), wsd, w.had_block, 0, Ad, Bd,
                                       w_layout="tiled_ob"))
    else:
        y_int = host(W.qlinear_forward(Xd, dev(wt), wsd, w.had_block, w.w_group, Ad, Bd,
                                       w_layout="tiled"))
    if M > 32:   # decode-sized int8 calls take the skinny kernel's summation order for groups
        assert np.array_equal(y, y_int)
    elif w.w_group == 0:
        assert np.array_equal(y, y_int)
    else:
        check_y(y_int, y_codes, y_oracle)


@pytest.mark.parametrize("M,K,N,b,g,r,dt", [
    (1, 256, 64, 256, 0, 0, "float16"), (33, 4096, 100, 4096, 0, 64, "float16"),
    (65, 14336, 96, 128, 128, 0, "float16"), (300, 1024, 1030, 256, 0, 40, "float16"),
    (40, 384, 100, 128, 128, 0, "float32"), (20, 4096, 520, 128, 0, 24, "float16"),
    (130, 1024, 260, 128, 256, 16, "float32"), (8, 4096, 4096, 4096, 0, 64, "float16"),
    (257, 2048, 384, 128, 128, 32, "float16"), (16, 2048, 64, 128, 0, 8, "float16")])
def test_qlinear_f6_ragged(M, K, N, b, g, r, dt):
    w = synth.small("rf6", M, K, N, x_dtype=dt, had_block=b, w_group=g, rank=r,
                    w_scale_dtype="float16" if dt == "float16" else "float32")
    run_layer_f6(w)


def test_qlinear_f6_prefill_full_size():
    run_layer_f6(synth.PREFILL)
