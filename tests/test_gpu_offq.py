"""Parity of the asymmetric group-wise activation path (OffQ page,
"Metodología" steps 2-3) against the CPU oracle, through the C ABI.

Bars:
* codes, scales and zero points when both sides start from the oracle's
  rotated float32 activations (had_block 0): bit-exact;
* weight group sums: exact;
* the GEMM on given codes: |y - y_oracle| <= |s_w| 2^-20 (G + 8)
  (A1 + A2 + max_g |o| W1) per element, with A1 = sum_g |s acc_g| (acc_g
  over q - 8), A2 = sum_g |o_g wsum_g|, o = s (z - 8), W1 = sum_g |wsum_g|:
  float32 group flushes, the float32 offset o, its fp16 pair (about 22
  bits) and float32 accumulation, each a few units of 2^-24 of these sums;
* the fused layer: effective codes q - z within one step of the oracle's on
  at most 0.01% of elements, scales within 1e-6 relative, and
  max |Y - epilogue(GPU codes)| <= 1e-3 RMS(Y_oracle).
"""
import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth
from bit_gemm_block_amd import w4a4 as W
from bars import check_y
from layouts import tile_weights, untile_weights

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_codes(xq, M, layout):
    """uint4 codes q from the stored nibbles q - 8."""
    b = host(xq)
    if layout == "packed_tiled":
        return gpu_codes_tiled_bytes(b, M)
    return (O.unpack_int4(b).astype(np.int16) + 8).astype(np.uint8)


def gpu_codes_tiled_bytes(b, M):
    """uint4 codes q from packed tiled bytes of the nibbles q - 8."""
    return (O.unpack_int4(untile_weights(b, M)).astype(np.int16) + 8).astype(np.uint8)


# --------------------------------------------------------------------------
# Quantizer: exact on the oracle's rotation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["packed", "packed_tiled"])
@pytest.mark.parametrize("M,K,g,dt", [
    (37, 4096, 128, "float16"), (20, 14336, 128, "float16"), (5, 4096, 4096, "float16"),
    (100, 1024, 256, "float32"), (3, 256, 128, "float32"), (70, 8192, 2048, "float16"),
    (1, 128, 128, "float32"), (17, 16384, 512, "float16")])
def test_quantize_act_asym_exact_on_oracle_rotation(M, K, g, dt, layout):
    w = synth.small("aq", M, K, 8, x_dtype=dt, n_outlier=3, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xr = O.rotate(X, g)
    print("asym quantizer", M, K, g, layout, flush=True)
    xq, sx, zx = W.quantize_act_asym_int4(dev(xr), 0, g, layout=layout)
    q, s, z = O.quantize_act_asym(xr, g)
    assert np.array_equal(host(sx), s)
    assert np.array_equal(host(zx).astype(np.int64), z)
    assert np.array_equal(gpu_codes(xq, M, layout), q)


def test_quantize_act_asym_edge_groups():
    # zero, constant (both signs), offsets far beyond the spread (zero points
    # far outside [0, 15]), tiny and huge ranges (the division path), and
    # exact ties on a power-of-two grid.
    rng = np.random.default_rng(11)
    K, g = 1024, 128
    rows = []
    rows.append(np.zeros(K))
    rows.append(np.full(K, 3.0))
    rows.append(np.full(K, -2.5))
    rows.append(1000.0 + 1e-3 * rng.standard_normal(K))
    rows.append(-7e4 + rng.standard_normal(K))
    rows.append(2.0 ** -120 * rng.standard_normal(K))
    rows.append(2.0 ** 110 * rng.standard_normal(K))
    s = 2.0 ** -5
    t = rng.integers(0, 15, K) + 0.5                       # ties between codes
    t[::g] = 0
    t[1::g] = 15
    rows.append(s * (t - 6))
    mixed = rng.standard_normal(K)
    mixed[:g] = 5.0
    mixed[g:2 * g] = 1.0 + 2.0 ** -20 * rng.standard_normal(g)
    rows.append(mixed)
    xr = np.array(rows, dtype=np.float32)
    for layout in ("packed", "packed_tiled"):
        xq, sx, zx = W.quantize_act_asym_int4(dev(xr), 0, g, layout=layout)
        q, sp, zp = O.quantize_act_asym(xr, g)
        assert np.array_equal(host(sx), sp)
        assert np.array_equal(host(zx).astype(np.int64), zp)
        assert np.array_equal(gpu_codes(xq, len(rows), layout), q)
    assert np.abs(zp).max() > 1000  # offsets were absorbed by zero points beyond the code range


@pytest.mark.parametrize("M,K,b,dt,layout", [
    (64, 4096, 128, "float16", "packed"), (48, 14336, 128, "float16", "packed"),
    (8, 4096, 4096, "float16", "packed"), (100, 2048, 256, "float32", "packed"),
    (130, 4096, 128, "float16", "packed_tiled"), (2048, 4096, 128, "float16", "packed_tiled"),
    (300, 14336, 128, "float16", "packed_tiled"), (65, 2048, 128, "float16", "packed_tiled")])
def test_quantize_act_asym_fused_rotation(M, K, b, dt, layout):
    # The tiled cases of fp16 rows (b = 128, K a multiple of 2048) take the rotation
    # on the matrix instruction.
    w = synth.small("af", M, K, 8, x_dtype=dt, n_outlier=4, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    xq, sx, zx = W.quantize_act_asym_int4(dev(X), b, b, layout=layout)
    q, s, z = O.quantize_act_asym(O.rotate(X, b), b)
    gq = gpu_codes(xq, M, layout).astype(np.int64)
    gz, gs = host(zx).astype(np.int64), host(sx).astype(np.float64)
    eff = (gq - np.repeat(gz, b, axis=1)) - (q.astype(np.int64) - np.repeat(z, b, axis=1))
    assert np.all(np.abs(eff) <= 1)
    assert np.count_nonzero(eff) <= 1e-4 * eff.size
    assert np.all(np.abs(gz - z) <= 1)
    assert np.all(np.abs(gs - s) <= 1e-6 * s)


# --------------------------------------------------------------------------
# Weight group sums
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,g", [(1, 128, 128), (33, 384, 128), (100, 4096, 4096),
                                   (300, 14336, 128), (64, 2048, 64), (17, 1024, 256)])
@pytest.mark.parametrize("wl", ["rowmajor", "tiled"])
def test_weight_group_sums_exact(N, K, g, wl):
    if wl == "tiled" and K % 128:
        pytest.skip("tiled weights need K % 128 == 0")
    rng = np.random.default_rng(N + K + g)
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qw[0] = -8
    packed = O.pack_int4(qw)
    wq = tile_weights(packed, rng) if wl == "tiled" else packed
    got = host(W.weight_group_sums(dev(wq), g, N, w_layout=wl))
    assert np.array_equal(got.astype(np.int64), O.weight_group_sums(qw, g))


# --------------------------------------------------------------------------
# GEMM on given codes
# --------------------------------------------------------------------------
def asym_bound(q, s, z, qw, sw, g, rows):
    """Per-element tolerance of the asymmetric GEMM (module docstring)."""
    qs = q[rows].astype(np.int64) - 8
    G = qs.shape[1] // g
    ws = O.weight_group_sums(qw, g).astype(np.float64)                      # [N, G]
    o = np.abs(s[rows].astype(np.float64) * (z[rows].astype(np.float64) - 8))  # [m, G]
    A1 = np.zeros((len(rows), qw.shape[0]))
    for j in range(G):
        acc = np.abs(O.int_gemm(qs[:, j * g:(j + 1) * g], qw[:, j * g:(j + 1) * g]))
        A1 += np.abs(s[rows, j].astype(np.float64))[:, None] * acc
    A2 = o @ np.abs(ws).T
    tail = o.max(axis=1)[:, None] * np.abs(ws).sum(axis=1)[None, :]
    return np.abs(sw.astype(np.float64))[None, :] * 2.0 ** -20 * (G + 8) * (A1 + A2 + tail)


@pytest.mark.parametrize("M,N,K,g", [
    (1, 1, 128, 128), (7, 33, 256, 128), (130, 260, 1024, 256), (64, 128, 4096, 4096),
    (300, 129, 14336, 128), (2100, 4100, 1024, 128), (2048, 4096, 4096, 128),
    (16, 300, 2048, 512), (65, 70, 16384, 128), (2048, 4096, 4096, 4096), (130, 260, 1024, 1024),
    (300, 129, 2048, 2048), (32, 100, 1024, 256), (17, 40, 4096, 128), (8, 4096, 4096, 4096)])
def test_qgemm_asym(M, N, K, g):
    rng = np.random.default_rng(M + 3 * N + K + g)
    G = K // g
    q = rng.integers(0, 16, (M, K)).astype(np.uint8)
    z = rng.integers(-300, 300, (M, G)).astype(np.int64)
    z[0] = rng.integers(-2 ** 26, 2 ** 26, G)        # offsets far beyond the spread
    s = rng.uniform(1e-3, 0.5, (M, G)).astype(np.float32)
    if M > 2:
        s[2] = 0.0
        z[2] = 0
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    qw[0] = -8
    sw = rng.uniform(1e-3, 0.05, N).astype(np.float16)
    xq = tile_weights(O.pack_int4((q.astype(np.int16) - 8).astype(np.int8)), rng)
    wq = tile_weights(O.pack_int4(qw), rng)
    gsum = W.weight_group_sums(dev(wq), g, N, w_layout="tiled")
    print("qgemm_asym", M, N, K, g, flush=True)
    y = host(W.qgemm_asym(dev(xq), dev(s), dev(z.astype(np.int32)), g, dev(wq), dev(sw), gsum))
    rows = np.arange(M) if M <= 300 else np.unique(np.r_[0, 1, 2, rng.integers(0, M, 60), M - 1])
    ref = O.asym_from_codes(q[rows], s[rows], z[rows], qw, sw.astype(np.float32), g)
    bound = asym_bound(q, s, z, qw, sw, g, rows)
    err = np.abs(y[rows].astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= bound + 2.0 ** -24 * np.abs(ref)), float(np.max(err - bound))


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def run_asym_layer(w, sample_rows=None):
    d = synth.make_inputs(w)
    X, Wt, A, B = d["X"], d["W"], d["A"], d["B"]
    b = w.had_block
    wq, ws, qw = O.prepare_weight(Wt, b, 0, w.w_scale_dtype)
    wqd = dev(tile_weights(wq))
    gsum = W.weight_group_sums(wqd, b, w.N, w_layout="tiled")
    Xd = dev(X)
    Ad = dev(A.T) if A is not None else None
    Bd = dev(B.T) if B is not None else None
    print("asym layer", w.name, w.M, w.K, w.N, b, w.rank, flush=True)
    ws_buf = W.qlinear_workspace(w.M, w.N, w.K, w.rank, DEV)
    y = host(W.qlinear_forward_asym(Xd, wqd, dev(ws), gsum, b, Ad, Bd, workspace=ws_buf))
    # the codes, group scales and zero points the layer left in its workspace
    wsb = host(ws_buf)
    co, _, _ = W.qlinear_workspace_layout(w.M, w.N, w.K, w.rank, "tiled", 0)
    Mp, G = W.pad16(w.M), w.K // b
    so = co + (Mp * w.K // 2 + 255) // 256 * 256
    zo = so + (w.M * G * 4 + 255) // 256 * 256
    gq = gpu_codes_tiled_bytes(wsb[co:co + Mp * w.K // 2].reshape(Mp, w.K // 2), w.M)
    gs = wsb[so:so + 4 * w.M * G].view(np.float32).reshape(w.M, G)
    gz = wsb[zo:zo + 4 * w.M * G].view(np.int32).reshape(w.M, G).astype(np.int64)
    rows = np.arange(w.M) if sample_rows is None else sample_rows
    Xr = X[rows]
    q, s, z = O.quantize_act_asym(O.rotate(Xr, b), b)
    lr = (A, B) if A is not None else (None, None)
    y_codes = O.asym_from_codes(gq[rows], gs[rows], gz[rows], qw, ws.astype(np.float32), b,
                                Xr, *lr)
    y_oracle = O.qlinear_forward_asym(Xr, wq, ws, b, *lr)
    rms = float(np.sqrt(np.mean(y_oracle.astype(np.float64) ** 2)))
    eff = (gq[rows].astype(np.int64) - np.repeat(gz[rows], b, axis=1)) - \
          (q.astype(np.int64) - np.repeat(z, b, axis=1))
    assert np.all(np.abs(eff) <= 1)
    assert np.count_nonzero(eff) <= 1e-4 * eff.size
    assert np.all(np.abs(gs[rows].astype(np.float64) - s) <= 1e-6 * s)
    check_y(y[rows], y_codes, y_oracle)
    return float(np.max(np.abs(y[rows] - y_oracle)) / rms)


@pytest.mark.parametrize("M,K,N,b,r,dt", [
    (1, 256, 64, 128, 0, "float16"), (130, 1024, 260, 128, 16, "float16"),
    (33, 4096, 100, 4096, 64, "float16"), (65, 14336, 96, 128, 32, "float16"),
    (20, 4096, 520, 256, 24, "float16"), (300, 1024, 1030, 512, 40, "float16"),
    (8, 4096, 96, 128, 40, "float16"), (24, 2048, 100, 128, 72, "float16"),
    (40, 384, 100, 128, 0, "float32"), (16, 512, 48, 128, 8, "float32"),
    (33, 4096, 100, 4096, 0, "float16"), (130, 1024, 260, 1024, 0, "float32"),
    (8, 6144, 96, 128, 64, "float16"), (8, 12288, 64, 128, 64, "float16")])
def test_qlinear_asym_ragged(M, K, N, b, r, dt):
    w = synth.small("asl", M, K, N, x_dtype=dt, had_block=b, rank=r,
                    w_scale_dtype="float16" if dt == "float16" else "float32")
    run_asym_layer(w)


@pytest.mark.parametrize("name", ["llama3_8b_o_4096x4096x4096", "llama3_8b_down_4096x14336x4096",
                                  "prefill_2048x4096x4096"])
def test_qlinear_asym_full_size(name):
    w = synth.by_name(name)
    rows = np.unique(np.r_[0, 1, np.random.default_rng(5).integers(0, w.M, 40), w.M - 1])
    rel = run_asym_layer(w, rows)
    print(name, "asym max|Y-Y_oracle|/RMS =", rel)
