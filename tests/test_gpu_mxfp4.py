"""Parity of the MXFP4 path (SERQ page, "Metodología" item 2, read as the
OCP microscaling format) against the CPU oracle, through the C ABI.

Bars:
* codes and E8M0 scale bytes on the oracle's rotation (had_block 0):
  bit-exact, in the row-major and tiled layouts, on block ties, zero,
  subnormal and huge blocks and saturating values;
* with the fused rotation: at most 0.01% of elements with a different
  (code, scale), each within two E2M1 steps of the block's scale;
* the GEMM on given codes: |y - y_oracle| <= 2^-23 (K/128 + 4) sum_k |x_k w_k|
  (float32 accumulation of exact products, one sum per instruction);
* the layer: max |Y - epilogue(GPU codes)| <= 1e-3 RMS(Y_oracle).
"""
import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth
from bit_gemm_block_amd import w4a4 as W
from bars import check_y
from layouts import tile_mx_scales, tile_weights, untile_mx_scales, untile_weights

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def nibbles(packed):
    """Unsigned 4-bit codes of packed bytes (element 2j in the low nibble)."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_codes(c):
    c = np.asarray(c, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def gpu_mx(x, b, layout):
    M, K = x.shape
    xq, xs = W.quantize_mxfp4(dev(x), b, layout)
    q, s = host(xq), host(xs)
    if layout == "packed_tiled":
        return nibbles(untile_weights(q, M)), untile_mx_scales(s, M, K).astype(np.int64) - 127
    return nibbles(q), s.astype(np.int64) - 127


@pytest.mark.parametrize("layout", ["packed", "packed_tiled"])
@pytest.mark.parametrize("M,K,dt", [(37, 4096, "float16"), (100, 4096, "float32"), (5, 128, "float32"),
                                    (130, 14336, "float16"), (300, 1024, "float16"), (1, 256, "float32")])
def test_quantize_mxfp4_exact_on_oracle_rotation(M, K, dt, layout):
    w = synth.small("mx", M, K, 8, x_dtype=dt, n_outlier=3, bos_factor=500.0)
    xr = O.rotate(synth.make_inputs(w)["X"], 128 if K % 128 == 0 else 64)
    print("mxfp4 quantizer", M, K, layout, flush=True)
    codes, e = gpu_mx(xr, 0, layout)
    pc, pe = O.quantize_mxfp4(xr)
    assert np.array_equal(e, pe)
    assert np.array_equal(codes, pc)


def test_quantize_mxfp4_edge_blocks():
    rng = np.random.default_rng(9)
    K = 256
    rows = [np.zeros(K), 2.0 ** -140 * rng.standard_normal(K), 2.0 ** -126 * rng.standard_normal(K),
            2.0 ** 120 * rng.standard_normal(K), rng.standard_normal(K)]
    tie = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4)   # block max 6: scale 2^0
    sgn = np.where(rng.integers(0, 2, K) > 0, 1.0, -1.0)
    rows.append(np.tile(tie, K // 32) * sgn * 2.0 ** -3)
    sat = rng.uniform(-7.9, 7.9, K)
    sat[::32] = 7.9                                                     # max in (6, 8): saturation
    rows.append(sat)
    x = np.array(rows, dtype=np.float32)
    for layout in ("packed", "packed_tiled"):
        codes, e = gpu_mx(x, 0, layout)
        pc, pe = O.quantize_mxfp4(x)
        assert np.array_equal(e, pe)
        assert np.array_equal(codes, pc)


def test_quantize_mxfp4_row_major_small_k():
    x = np.random.default_rng(3).standard_normal((9, 64)).astype(np.float32)
    codes, e = gpu_mx(x, 0, "packed")
    pc, pe = O.quantize_mxfp4(x)
    assert np.array_equal(e, pe) and np.array_equal(codes, pc)


@pytest.mark.parametrize("M,K,b", [(64, 4096, 128), (48, 14336, 128), (100, 4096, 4096), (8, 2048, 256),
                                   (130, 4096, 128), (2048, 4096, 4096), (300, 8192, 1024),
                                   (97, 6144, 2048), (77, 16384, 4096), (1000, 14336, 128)])
def test_quantize_mxfp4_fused_rotation(M, K, b):
    # fp16 rows with K a multiple of 2048: the rotation on the matrix
    # instruction (the tiled layout; the row-major one keeps the butterfly kernel)
    w = synth.small("mxf", M, K, 8, n_outlier=4, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    codes, e = gpu_mx(X, b, "packed_tiled")
    pc, pe = O.quantize_mxfp4(O.rotate(X, b))
    dg, do = O.mxfp4_values(codes, e), O.mxfp4_values(pc, pe)
    diff = dg != do
    assert np.count_nonzero(diff) <= 1e-4 * diff.size
    step = np.repeat(np.exp2(np.maximum(e, pe)), 32, axis=1)
    assert np.all(np.abs(dg - do) <= 2 * step)


@pytest.mark.parametrize("M,K,b", [(130, 4096, 4096), (300, 4096, 128), (65, 8192, 512)])
def test_quantize_mxfp4_matrix_rotation_matches_butterfly(M, K, b):
    # the tiled layout (matrix instruction) against the row-major one
    # (butterflies) on the same input: the same rule on float32 sums that
    # round in another order, so at most 0.02% of the values differ, each by
    # at most two E2M1 steps of the larger scale
    w = synth.small("mxm", M, K, 8, n_outlier=4, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    ct, et = gpu_mx(X, b, "packed_tiled")
    cr, er = gpu_mx(X, b, "packed")
    vt, vr = O.mxfp4_values(ct, et), O.mxfp4_values(cr, er)
    assert np.count_nonzero(vt != vr) <= 2e-4 * vt.size
    step = np.repeat(np.exp2(np.maximum(et, er)), 32, axis=1)
    assert np.all(np.abs(vt - vr) <= 2 * step)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (7, 33, 256), (130, 260, 1024), (2048, 4096, 4096),
                                   (300, 129, 14336), (2100, 4100, 1024), (16, 300, 16384),
                                   (25, 77, 1024), (8, 4096, 4096), (32, 48, 2048)])
def test_qgemm_mxfp4(M, N, K):
    rng = np.random.default_rng(M + N + K)
    cx = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
    ex = rng.integers(-12, 6, (M, K // 32))
    ew = rng.integers(-12, 6, (N, K // 32))
    ex[0, 0] = -127
    print("qgemm_mxfp4", M, N, K, flush=True)
    y = host(W.qgemm_mxfp4(dev(tile_weights(pack_codes(cx), rng)), dev(tile_mx_scales((ex + 127).astype(np.uint8), rng)),
                           dev(tile_weights(pack_codes(cw), rng)), dev(tile_mx_scales((ew + 127).astype(np.uint8), rng)),
                           M, N, K))
    rows = np.arange(M) if M <= 300 else np.unique(np.r_[0, 1, rng.integers(0, M, 50), M - 1])
    ref = O.mxfp4_gemm(cx[rows], ex[rows], cw, ew)
    mag = np.abs(O.mxfp4_values(cx[rows], ex[rows])) @ np.abs(O.mxfp4_values(cw, ew)).T
    assert np.all(np.abs(y[rows] - ref) <= 2.0 ** -23 * (K / 128 + 4) * mag)


def run_mx_layer(w, sample_rows=None):
    d = synth.make_inputs(w)
    X, Wt, A, B = d["X"], d["W"], d["A"], d["B"]
    b = w.had_block
    wq, ws = W.quantize_mxfp4(dev(Wt), b, "packed_tiled")
    Xd = dev(X)
    Ad = dev(A.T) if A is not None else None
    Bd = dev(B.T) if B is not None else None
    print("mxfp4 layer", w.name, w.M, w.K, w.N, b, w.rank, flush=True)
    ws_buf = W.qlinear_workspace(w.M, w.N, w.K, w.rank, DEV)
    y = host(W.qlinear_forward_mxfp4(Xd, wq, ws, w.N, b, Ad, Bd, workspace=ws_buf))
    wc = nibbles(untile_weights(host(wq), w.N))
    we = untile_mx_scales(host(ws), w.N, w.K).astype(np.int64) - 127
    pwc, pwe = O.quantize_mxfp4(O.rotate(Wt, b))
    dw = O.mxfp4_values(wc, we) != O.mxfp4_values(pwc, pwe)
    assert np.count_nonzero(dw) <= 1e-4 * dw.size
    rows = np.arange(w.M) if sample_rows is None else sample_rows
    # the codes and scale tiles the layer left in its workspace
    wsb = host(ws_buf)
    co, _, _ = W.qlinear_workspace_layout(w.M, w.N, w.K, w.rank, "tiled", 0)
    Mp = W.pad16(w.M)
    so = co + (Mp * w.K // 2 + 255) // 256 * 256
    xc = nibbles(untile_weights(wsb[co:co + Mp * w.K // 2].reshape(Mp, w.K // 2), w.M))
    xe = untile_mx_scales(wsb[so:so + Mp * w.K // 32], w.M, w.K).astype(np.int64) - 127
    pxc, pxe = O.quantize_mxfp4(O.rotate(X[rows], b)) if b > 1 else O.quantize_mxfp4(X[rows])
    dx = O.mxfp4_values(xc[rows], xe[rows]) != O.mxfp4_values(pxc, pxe)
    assert np.count_nonzero(dx) <= 1e-4 * dx.size + 1
    y_codes = O.mxfp4_gemm(xc[rows], xe[rows], wc, we)
    lr = O.lowrank(X[rows], A, B)
    if lr is not None:
        y_codes = y_codes + lr
    y_oracle = O.qlinear_forward_mxfp4(X[rows], Wt, b, A, B)
    rms = float(np.sqrt(np.mean(y_oracle.astype(np.float64) ** 2)))
    check_y(y[rows], y_codes, y_oracle)
    return float(np.max(np.abs(y[rows] - y_oracle)) / rms)


@pytest.mark.parametrize("M,K,N,b,r,dt", [
    (1, 256, 64, 256, 0, "float16"), (130, 1024, 260, 128, 16, "float16"),
    (33, 4096, 100, 4096, 64, "float16"), (65, 14336, 96, 128, 32, "float16"),
    (40, 384, 100, 128, 0, "float32"), (16, 512, 48, 128, 8, "float32"),
    (8, 6144, 96, 128, 64, "float16"), (8, 12288, 64, 128, 64, "float16"),
    (8, 4096, 96, 4096, 40, "float16"), (24, 2048, 100, 128, 72, "float16")])
def test_qlinear_mxfp4_ragged(M, K, N, b, r, dt):
    w = synth.small("mxl", M, K, N, x_dtype=dt, had_block=b, rank=r)
    run_mx_layer(w)


@pytest.mark.parametrize("name", ["prefill_2048x4096x4096", "llama3_8b_o_4096x4096x4096"])
def test_qlinear_mxfp4_full_size(name):
    w = synth.by_name(name)
    rows = np.unique(np.r_[0, 1, np.random.default_rng(4).integers(0, w.M, 40), w.M - 1])
    print(name, "mxfp4 max|Y-Y_oracle|/RMS =", run_mx_layer(w, rows))
