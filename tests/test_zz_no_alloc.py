"""w4a4_qlinear_forward_noalloc (the layer with its scratch in the library's
fixed per-device array) against w4a4_qlinear_forward with a caller-provided
workspace.  Both run the same kernels on the same inputs, so Y must agree bit
for bit; two calls in a row, the second on a smaller input, check that the
array's leftovers from one call do not leak into the next."""
import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth
from bit_gemm_block_amd import w4a4 as W
from layouts import ob_weights, tile_f6, tile_weights

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def operands(w, wl):
    d = synth.make_inputs(w)
    wq, ws, qw = O.prepare_weight(d["W"], w.had_block, w.w_group, w.w_scale_dtype)
    op = {"rowmajor": wq, "tiled": tile_weights(wq),
          "tiled_ob": ob_weights(tile_weights(wq), w.N, w.K) if w.w_group == 0 else None,
          "tiled_f6": tile_f6(qw)}[wl]
    At = dev(d["A"].T) if d["A"] is not None else None
    Bt = dev(d["B"].T) if d["B"] is not None else None
    return d, wq, ws, dev(op), At, Bt


def check_call(w, wl):
    print("noalloc", w.name, w.M, w.K, w.N, wl, flush=True)
    assert W.qlinear_workspace_size(w.M, w.N, w.K, w.rank) <= W.NOALLOC_SCRATCH_BYTES
    d, wq, ws, op, At, Bt = operands(w, wl)
    X, wsd = dev(d["X"]), dev(ws)
    y_na = torch.full((w.M, w.N), float("nan"), dtype=torch.float32, device=DEV)
    W.qlinear_forward_noalloc(X, op, wsd, w.had_block, w.w_group, At, Bt, y=y_na, w_layout=wl)
    y_na = host(y_na)
    y_ws = host(W.qlinear_forward(X, op, wsd, w.had_block, w.w_group, At, Bt, w_layout=wl))
    assert np.array_equal(y_na, y_ws)
    y_or = O.qlinear_forward(d["X"], wq, ws, w.had_block, w.w_group, d["A"], d["B"])
    rms = float(np.sqrt(np.mean(y_or.astype(np.float64) ** 2)))
    print("  max|Y - Y_oracle|/RMS =", float(np.max(np.abs(y_na - y_or)) / rms), flush=True)


def test_noalloc_equals_workspace_forward_two_calls():
    first = synth.PREFILL                                            # 8 MiB of scratch
    second = synth.small("na2", 8, 4096, 1000, had_block=4096, rank=64)
    check_call(first, "tiled_ob")
    check_call(second, "tiled_ob")


def test_noalloc_equals_workspace_forward_forms():
    # row-major, tiled and FP6 tiled weights, a weight group, fp32 input,
    # low-rank terms
    for w, wl in [(synth.small("na3", 300, 1024, 260, had_block=256, rank=16), "tiled"),
                  (synth.small("na6", 200, 2048, 384, had_block=128, w_group=128, rank=32),
                   "tiled_f6"),
                  (synth.small("na4", 65, 14336, 96, had_block=128, w_group=128, rank=32), "tiled"),
                  (synth.small("na5", 40, 384, 100, x_dtype="float32", w_scale_dtype="float32"),
                   "rowmajor"),
                  (synth.TINY, "rowmajor")]:
        check_call(w, wl)


def test_noalloc_rejects_inputs_beyond_its_array():
    M, N, K = 4096, 64, 16384
    assert W.qlinear_workspace_size(M, N, K, 0) > W.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    wq = torch.zeros((N, K // 2), dtype=torch.uint8, device=DEV)
    ws = torch.ones(N, dtype=torch.float16, device=DEV)
    y = torch.full((M, N), 7.0, device=DEV)
    with pytest.raises(W.W4A4Error) as e:
        W.qlinear_forward_noalloc(x, wq, ws, 128, 0, y=y)
    assert e.value.status == W.ERR_WORKSPACE
    assert bool((y == 7.0).all())        # nothing was enqueued
