"""Parity of the offset-binary tiled operands (a storage encoding of the same
int4 codes, include/w4a4.h "Offset-binary tiled layouts") against the CPU
oracle, through the C ABI.

Bars:
* weight conversion: bit-exact tiles (padding rows included) and row sums;
* activation codes on the oracle's rotation (had_block 0): the tiles XOR 0x08
  are the oracle's packed codes and the row sums the oracle codes' sums over
  the odd channels, bit-exact; scales bit-exact;
* GEMM: the int32 product bit-exact; y within the bound of the plain tiled
  GEMM's test;
* layer: as the plain tiled layer (codes within one step on at most 0.01%,
  max |Y - epilogue(GPU codes)| <= 1e-3 RMS(Y_oracle)), and equal bit for
  bit to the layer on the plain tiled weights (both scale an exact integer
  product by the same powers of two).
"""
import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth
from bit_gemm_block_amd import w4a4 as W
from layouts import ob_codes, ob_weights, split_ob, tile_weights, untile_weights, workspace_codes
from bars import check_y

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("N,K", [(16, 128), (33, 256), (100, 4096), (4096, 4096), (70, 14336)])
def test_weights_to_ob_exact(N, K):
    rng = np.random.default_rng(N + K)
    tiled = rng.integers(0, 256, (W.pad16(N), K // 2), dtype=np.uint8)
    print("weights_to_ob", N, K, flush=True)
    out = host(W.weights_tiled_to_ob(dev(tiled), N))
    ref = ob_weights(tiled, N, K)
    gt, gs = split_ob(out, N, K)
    rt, rs = split_ob(ref, N, K)
    assert np.array_equal(gt, rt)
    assert np.array_equal(gs, rs)


def test_weights_to_ob_in_place():
    rng = np.random.default_rng(3)
    N, K = 40, 1024
    tiled = rng.integers(0, 256, (W.pad16(N), K // 2), dtype=np.uint8)
    buf = torch.zeros((W.ob_bytes(N, K),), dtype=torch.uint8, device=DEV)
    buf[:tiled.size] = dev(tiled.reshape(-1))
    W.weights_tiled_to_ob(buf[:tiled.size].view(W.pad16(N), K // 2), N, out=buf)
    assert np.array_equal(split_ob(host(buf), N, K)[0], split_ob(ob_weights(tiled, N, K), N, K)[0])
    assert np.array_equal(split_ob(host(buf), N, K)[1], split_ob(ob_weights(tiled, N, K), N, K)[1])


@pytest.mark.parametrize("M,K,b,dt", [(37, 4096, 4096, "float16"), (20, 14336, 128, "float16"),
                                      (3, 256, 64, "float32"), (100, 1024, 1024, "float16"),
                                      (2048, 4096, 4096, "float16"), (1, 128, 128, "float16")])
def test_quantize_act_ob_exact(M, K, b, dt):
    w = synth.small("qob", M, K, 8, x_dtype=dt, n_outlier=3, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xr = O.rotate(X, b)
    print("quantize_act ob", M, K, b, dt, flush=True)
    xq, sx = W.quantize_act_int4(dev(xr), 0, layout="packed_tiled_ob")
    assert tuple(xq.shape) == (W.ob_bytes(M, K),)
    pq, ps, pc, _ = O.quantize_activation(xr, 0)
    tiles, sums = split_ob(host(xq), M, K)
    assert np.array_equal(host(sx), ps)
    assert np.array_equal(untile_weights(tiles ^ 0x08, M), pq)
    assert np.array_equal(sums, pc[:, 1::2].astype(np.int64).sum(axis=1))


def test_quantize_act_ob_fused_rotation_matches_plain_codes():
    # Same kernel and rotation as the plain packed tiled codes: the offset
    # form is those bytes XOR 0x08, and its sums those of the plain codes.
    w = synth.small("qobf", 130, 4096, 8, n_outlier=3, bos_factor=500.0)
    Xd = dev(synth.make_inputs(w)["X"])
    xq_ob, sx_ob = W.quantize_act_int4(Xd, 4096, layout="packed_tiled_ob")
    xq, sx = W.quantize_act_int4(Xd, 4096, layout="packed_tiled")
    tiles, sums = split_ob(host(xq_ob), 130, 4096)
    assert np.array_equal(host(sx_ob), host(sx))
    assert np.array_equal(untile_weights(tiles ^ 0x08, 130), untile_weights(host(xq), 130))
    codes = O.unpack_int4(untile_weights(host(xq), 130)).astype(np.int64)
    assert np.array_equal(sums, codes[:, 1::2].sum(axis=1))


def ob_operands(qx, qw, rng):
    M, K = qx.shape
    N = qw.shape[0]
    return ob_codes(tile_weights(O.pack_int4(qx), rng), M, K), \
        ob_weights(tile_weights(O.pack_int4(qw), rng), N, K)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (8, 4096, 4096), (17, 33, 256), (32, 300, 14336),
                                   (33, 70, 384), (130, 260, 384), (300, 129, 1024),
                                   (2048, 4096, 4096), (2100, 4100, 1024), (4096, 4096, 128)])
def test_qgemm_ob_exact_and_dequant(M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    qx = rng.integers(-8, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qx[0, :] = -8
    qw[0, :] = -8
    qx[-1, :] = 7
    qw[-1, :] = 7
    sx = rng.uniform(0.01, 2.0, M).astype(np.float32)
    sw = rng.uniform(1e-3, 0.05, N).astype(np.float16)
    xin, win = ob_operands(qx, qw, rng)
    print("qgemm ob", M, N, K, flush=True)
    y, acc = W.qgemm_w4a4(dev(xin), dev(sx), dev(win), dev(sw), 0, want_y=True, want_acc=True,
                          layout="packed_tiled_ob", w_layout="tiled_ob", M=M, N=N)
    ref_acc = O.int_gemm(qx, qw)
    assert np.array_equal(host(acc), ref_acc)
    ref = O.epilogue(ref_acc, sx, sw.astype(np.float32), None).astype(np.float64)
    mag = np.abs(sx)[:, None] * np.abs(sw.astype(np.float64))[None, :] * 64 * K
    assert np.all(np.abs(host(y) - ref) <= 4 * 2.0 ** -23 * mag)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (8, 4096, 4096), (17, 33, 256), (32, 300, 14336)])
def test_qgemm_ob_weights_with_plain_codes_decode(M, N, K):
    # Decode-sized products take plain packed tiled codes with offset-binary
    # weights (the skinny kernel converts the weights).
    rng = np.random.default_rng(M + N + K)
    qx = rng.integers(-8, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qw[0, :] = -8
    sx = rng.uniform(0.01, 2.0, M).astype(np.float32)
    sw = rng.uniform(1e-3, 0.05, N).astype(np.float16)
    win = ob_weights(tile_weights(O.pack_int4(qw), rng), N, K)
    print("qgemm ob weights decode", M, N, K, flush=True)
    y, acc = W.qgemm_w4a4(dev(tile_weights(O.pack_int4(qx), rng)), dev(sx), dev(win), dev(sw), 0,
                          want_y=True, want_acc=True, layout="packed_tiled", w_layout="tiled_ob",
                          M=M, N=N)
    ref_acc = O.int_gemm(qx, qw)
    assert np.array_equal(host(acc), ref_acc)
    ref = O.epilogue(ref_acc, sx, sw.astype(np.float32), None).astype(np.float64)
    mag = np.abs(sx)[:, None] * np.abs(sw.astype(np.float64))[None, :] * 64 * K
    assert np.all(np.abs(host(y) - ref) <= 4 * 2.0 ** -23 * mag)


def test_qgemm_ob_rejects_mismatched_layouts():
    M, N, K = 64, 32, 256
    xq = torch.zeros((W.ob_bytes(M, K),), dtype=torch.uint8, device=DEV)
    wt = torch.zeros((W.pad16(N), K // 2), dtype=torch.uint8, device=DEV)
    sx = torch.ones(M, device=DEV)
    sw = torch.ones(N, device=DEV, dtype=torch.float16)
    # offset-binary codes with plain tiled weights
    with pytest.raises(W.W4A4Error):
        st = W.lib().w4a4_qgemm_w4a4(W._ptr(xq), W.CODES_PACKED_TILED_OB, W._ptr(sx), W._ptr(wt),
                                     W.WEIGHTS_TILED, W._ptr(sw), W.F16, 0, M, N, K,
                                     W._ptr(torch.empty((M, N), device=DEV)), None, None)
        W._check("qgemm_w4a4", st)
    # offset-binary weights with plain codes above the decode size
    wob = torch.zeros((W.ob_bytes(N, K),), dtype=torch.uint8, device=DEV)
    xt = torch.zeros((W.pad16(M), K // 2), dtype=torch.uint8, device=DEV)
    with pytest.raises(W.W4A4Error):
        W.qgemm_w4a4(xt, sx, wob, sw, 0, layout="packed_tiled", w_layout="tiled_ob", M=M, N=N)


def run_layer_ob(w, rows=None):
    assert w.w_group == 0
    d = synth.make_inputs(w, rows)
    X, Wt, A, B = d["X"], d["W"], d["A"], d["B"]
    wq, ws, _ = O.prepare_weight(Wt, w.had_block, w.w_group, w.w_scale_dtype)
    N, K = Wt.shape
    Xd, wsd = dev(X), dev(ws)
    Ad = dev(A.T) if A is not None else None
    Bd = dev(B.T) if B is not None else None
    wt = tile_weights(wq)
    print("layer ob", w.name, w.M, w.K, w.N, w.had_block, w.rank, flush=True)
    M = X.shape[0]
    ws_buf = W.qlinear_workspace(M, N, K, w.rank, DEV)
    y = host(W.qlinear_forward(Xd, dev(ob_weights(wt, N, K)), wsd, w.had_block, 0, Ad, Bd,
                               workspace=ws_buf, w_layout="tiled_ob"))
    y_plain = host(W.qlinear_forward(Xd, dev(wt), wsd, w.had_block, 0, Ad, Bd, w_layout="tiled"))
    wsb = host(ws_buf)
    co, cl, so = W.qlinear_workspace_layout(M, N, K, w.rank, "tiled_ob", 0)
    assert cl == ("packed_tiled" if M <= 32 else "packed_tiled_ob")
    _, packed = workspace_codes(wsb, co, M, K, cl)
    gc = O.unpack_int4(packed).astype(np.int16)
    gsx = wsb[so:so + 4 * M].view(np.float32)
    if cl == "packed_tiled_ob":   # the row sums of the odd channels' codes follow the tiles
        sums = wsb[co + W.pad16(M) * (K // 2):].view(np.int32)[:M]
        assert np.array_equal(sums, gc[:, 1::2].sum(axis=1))
    _, ps, pc, _ = O.quantize_activation(X, w.had_block)
    y_codes = O.qlinear_from_codes(gc, gsx, wq, ws, 0, X, A, B)
    y_oracle = O.qlinear_forward(X, wq, ws, w.had_block, 0, A, B)
    rms = float(np.sqrt(np.mean(y_oracle.astype(np.float64) ** 2)))
    diff = gc - pc
    assert np.all(np.abs(diff) <= 1) and np.count_nonzero(diff) <= 1e-4 * diff.size
    assert np.all(np.abs(gsx.astype(np.float64) - ps) <= 1e-6 * ps)
    check_y(y, y_codes, y_oracle)
    assert np.array_equal(y, y_plain)
    return float(np.max(np.abs(y - y_oracle)) / rms)


@pytest.mark.parametrize("M,K,N,b,r,dt", [
    (1, 256, 64, 256, 0, "float16"), (33, 4096, 100, 4096, 64, "float16"),
    (65, 14336, 96, 128, 32, "float16"), (300, 1024, 1030, 256, 40, "float16"),
    (40, 384, 100, 128, 0, "float32"), (20, 4096, 520, 128, 24, "float16"),
    (130, 1024, 260, 128, 16, "float32")])
def test_qlinear_ob_ragged(M, K, N, b, r, dt):
    w = synth.small("rob", M, K, N, x_dtype=dt, had_block=b, rank=r,
                    w_scale_dtype="float16" if dt == "float16" else "float32")
    run_layer_ob(w)


def test_qlinear_ob_prefill_full_size():
    print("prefill ob max|Y-Y_oracle|/RMS =", run_layer_ob(synth.PREFILL))


def test_qlinear_ob_decode_full_size():
    print("decode ob max|Y-Y_oracle|/RMS =", run_layer_ob(synth.DECODE))
