"""The decode-sized layer (M <= 16 rows) on tiled and offset-binary tiled int4
weights with per-channel scales: the rotation launch (with the low-rank
projection and the weight read-ahead folded in) and the skinny GEMM.

Besides the layer bars of tests/test_gpu_parity.py:
* Y on tiled weights equals, bit for bit, Y on offset-binary tiled weights
  (another GEMM kernel: the same codes, the same exact integer sums and the
  same float32 epilogue arithmetic);
* a captured HIP graph of several calls, replayed with eager work and
  synchronisations in between, gives the eager result on every replay;
* two different inputs through one workspace, alternately, each give their
  own result (nothing of the previous call is read).
"""
import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth
from bit_gemm_block_amd import w4a4 as W
from bars import check_y
from layouts import ob_weights, tile_weights, workspace_codes

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def prepared(w):
    d = synth.make_inputs(w)
    wq, ws, _ = O.prepare_weight(d["W"], w.had_block, 0, w.w_scale_dtype)
    ops = {"rowmajor": dev(wq), "tiled": dev(tile_weights(wq)),
           "tiled_ob": dev(ob_weights(tile_weights(wq), w.N, w.K))}
    At = dev(d["A"].T) if d["A"] is not None else None
    Bt = dev(d["B"].T) if d["B"] is not None else None
    return d, wq, ws, ops, At, Bt


@pytest.mark.parametrize("M,K,N,b,r,dt", [
    (8, 4096, 4096, 4096, 64, "float16"), (1, 4096, 520, 4096, 0, "float16"),
    (16, 4096, 100, 128, 8, "float16"), (5, 2048, 300, 2048, 16, "float16"),
    (8, 8192, 96, 4096, 64, "float16"), (3, 4096, 64, 256, 0, "float32"),
    (12, 2048, 33, 128, 0, "float32"), (8, 12288, 40, 4096, 32, "float16"),
    # a partial last rank chunk, ranks past the preloaded 64, two 16-row blocks
    (8, 4096, 96, 4096, 40, "float16"), (20, 4096, 64, 4096, 72, "float16"),
    (32, 2048, 130, 128, 24, "float16")])
@pytest.mark.parametrize("wl", ["tiled", "tiled_ob"])
def test_decode_layer_tiled(M, K, N, b, r, dt, wl):
    w = synth.small("dec1", M, K, N, x_dtype=dt, had_block=b, rank=r,
                    w_scale_dtype="float16" if dt == "float16" else "float32")
    print("decode layer", M, K, N, b, r, dt, wl, flush=True)
    d, wq, ws, ops, At, Bt = prepared(w)
    X = dev(d["X"])
    wsd = dev(ws)
    ws_buf = W.qlinear_workspace(M, N, K, r, DEV)
    y = host(W.qlinear_forward(X, ops[wl], wsd, b, 0, At, Bt, workspace=ws_buf, w_layout=wl))
    # the other tiled weight layout: same codes, same arithmetic
    other = "tiled_ob" if wl == "tiled" else "tiled"
    y_other = host(W.qlinear_forward(X, ops[other], wsd, b, 0, At, Bt, w_layout=other))
    assert np.array_equal(y, y_other)
    wsb = host(ws_buf)
    co, cl, so = W.qlinear_workspace_layout(M, N, K, r, wl, 0)
    _, packed = workspace_codes(wsb, co, M, K, cl)
    gc = O.unpack_int4(packed).astype(np.int16)
    gsx = wsb[so:so + 4 * M].view(np.float32)
    _, ps, pc, _ = O.quantize_activation(d["X"], b)
    diff = gc - pc
    assert np.all(np.abs(diff) <= 1) and np.count_nonzero(diff) <= 1e-4 * diff.size + 1
    assert np.all(np.abs(gsx.astype(np.float64) - ps) <= 1e-6 * ps)
    y_codes = O.qlinear_from_codes(gc, gsx, wq, ws, 0, d["X"], d["A"], d["B"])
    y_or = O.qlinear_forward(d["X"], wq, ws, b, 0, d["A"], d["B"])
    check_y(y, y_codes, y_or)


def test_decode_graph_replays():
    # Several calls in one captured graph (two workspaces, alternating),
    # replayed three times with eager calls and synchronisations between
    # replays: every replay gives the eager Y.
    w = synth.DECODE
    d, wq, ws, ops, At, Bt = prepared(w)
    X = dev(d["X"])
    wsd = dev(ws)
    bufs = [W.qlinear_workspace(w.M, w.N, w.K, w.rank, DEV) for _ in range(2)]
    ys = [torch.empty((w.M, w.N), dtype=torch.float32, device=DEV) for _ in range(4)]
    eager = host(W.qlinear_forward(X, ops["tiled_ob"], wsd, w.had_block, 0, At, Bt,
                                   workspace=bufs[0], w_layout="tiled_ob"))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(4):
                W.qlinear_forward(X, ops["tiled_ob"], wsd, w.had_block, 0, At, Bt, y=ys[i],
                                  workspace=bufs[i % 2], w_layout="tiled_ob")
    torch.cuda.synchronize()
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for y in ys:
            assert np.array_equal(host(y), eager), rep
        # eager work on the same workspaces between replays
        y2 = host(W.qlinear_forward(X, ops["tiled"], wsd, w.had_block, 0, At, Bt,
                                    workspace=bufs[1], w_layout="tiled"))
        assert np.array_equal(y2, eager)


def test_decode_back_to_back_sizes():
    # One workspace serves calls of different sizes in a row.
    w_big = synth.small("dbb", 16, 8192, 777, had_block=4096, rank=64)
    ws_buf = W.qlinear_workspace(16, 777, 8192, 64, DEV)
    for M, K, N, r in [(16, 8192, 777, 64), (2, 4096, 300, 0), (9, 2048, 64, 8), (16, 8192, 777, 64)]:
        w = synth.small("dbb", M, K, N, had_block=min(K, 4096), rank=r)
        d, wq, ws, ops, At, Bt = prepared(w)
        X = dev(d["X"])
        y = host(W.qlinear_forward(X, ops["tiled_ob"], dev(ws), w.had_block, 0, At, Bt,
                                   workspace=ws_buf, w_layout="tiled_ob"))
        # the same call with a workspace of its own
        y_own = host(W.qlinear_forward(X, ops["tiled_ob"], dev(ws), w.had_block, 0, At, Bt,
                                       w_layout="tiled_ob"))
        assert np.array_equal(y, y_own)
    del w_big


@pytest.mark.parametrize("wl", ["tiled", "tiled_ob"])
def test_decode_alternating_inputs(wl):
    # Two different activations through one workspace, alternately: a GEMM
    # that read codes, scales or T left by the previous call would give the
    # other input's result.
    w = synth.small("dalt", 8, 4096, 1024, had_block=4096, rank=64)
    d, wq, ws, ops, At, Bt = prepared(w)
    X1 = dev(d["X"])
    X2 = dev(np.ascontiguousarray(d["X"][::-1] * np.float16(-0.5)))
    wsd = dev(ws)
    refs = [host(W.qlinear_forward(X, ops[wl], wsd, 4096, 0, At, Bt, w_layout=wl))
            for X in (X1, X2)]   # each with a workspace of its own
    assert not np.array_equal(refs[0], refs[1])
    ws_buf = W.qlinear_workspace(w.M, w.N, w.K, w.rank, DEV)
    for i in range(8):
        y = host(W.qlinear_forward((X1, X2)[i % 2], ops[wl], wsd, 4096, 0, At, Bt,
                                   workspace=ws_buf, w_layout=wl))
        assert np.array_equal(y, refs[i % 2]), i
