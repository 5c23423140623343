"""Full-size parity of every workload the benchmark times, on sampled rows.

Each case runs qlinear_forward at its real size, in the launch configurations
bench.py times: weights rotated and quantized on the GPU into the FP6 tiled
layout (the prefill workloads' form), and into the int4 tiled layout (then
converted to the offset-binary layout when the scales are per channel: the
decode workload's form and the other int4 forms); the activations rotated and
quantized inside the call.  The
reference is the CPU oracle's epilogue evaluated on the codes and scales the
call itself left in its workspace and on the GPU's own weight codes, for rows
0 (the BOS-like token), 1, 40 random rows and the last row.

Bars (see tests/test_gpu_parity.py for their source):
* activation codes against the oracle's: each within one step, at most 0.01%
  differing; per-token scales within 1e-6 relative;
* weight codes against the oracle's weight preparation: the same bar; the
  stored float16 scales equal or one float16 ulp apart;
* Y: per row, max |Y - epilogue(GPU codes)| <= 1e-3 * RMS of that row of the
  oracle's Y, and over the sample <= 1e-3 * RMS(Y_oracle).
"""
import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth
from bit_gemm_block_amd import w4a4 as W
from layouts import untile_f6, untile_weights, workspace_codes

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def sample_rows(M, seed):
    return np.unique(np.r_[0, 1, np.random.default_rng(seed).integers(0, M, 40), M - 1])


def gpu_weights(w, Wt_dev, form="int4"):
    """The benchmark's weight preparation: fused rotation into FP6 tiles
    (form "f6"), or into tiled int4, offset-binary for per-channel scales.
    Returns (operand, layout, scales, row-major packed codes read back)."""
    sdt = torch.float16 if w.w_scale_dtype == "float16" else torch.float32
    if form == "f6":
        wf, ws = W.quantize_weight_int4(Wt_dev, w.had_block, w.w_group, sdt, layout="tiled_f6")
        return wf, "tiled_f6", ws, O.pack_int4(untile_f6(host(wf), w.N, w.K))
    wt, ws = W.quantize_weight_int4(Wt_dev, w.had_block, w.w_group, sdt, layout="tiled")
    packed = untile_weights(host(wt), w.N)
    if w.w_group == 0:
        return W.weights_tiled_to_ob(wt, w.N), "tiled_ob", ws, packed
    return wt, "tiled", ws, packed


def check_weights(gpacked, gs, opacked, os_):
    d = O.unpack_int4(gpacked).astype(np.int16) - O.unpack_int4(opacked)
    assert np.all(np.abs(d) <= 1)
    assert np.count_nonzero(d) <= 1e-4 * d.size
    o64 = np.asarray(os_, np.float64)
    rel = np.abs(np.asarray(gs, np.float64) - o64) / np.where(o64 == 0, 1, o64)
    assert np.all(rel <= 1e-3)      # float16 storage: equal or one ulp apart


def check_rows(y, y_codes, y_oracle, label):
    """Per-row and sample-wide bars on Y against the epilogue of the GPU's codes."""
    e = np.abs(y.astype(np.float64) - y_codes)
    row_rms = np.sqrt(np.mean(y_oracle.astype(np.float64) ** 2, axis=1))
    rms = float(np.sqrt(np.mean(y_oracle.astype(np.float64) ** 2)))
    worst = float(np.max(e.max(axis=1) / row_rms))
    print(f"{label}: max_row max|Y - epilogue|/row RMS = {worst:.3e}; "
          f"max|Y - Y_oracle|/RMS = {float(np.max(np.abs(y - y_oracle)) / rms):.3e}", flush=True)
    assert np.all(e.max(axis=1) <= 1e-3 * row_rms), worst
    assert float(e.max()) <= 1e-3 * rms


def run_full(w, seed, form="int4"):
    print("full-size layer", w.name, form, flush=True)
    d = synth.make_inputs(w)
    X, Wt, A, B = d["X"], d["W"], d["A"], d["B"]
    Xd = dev(X)
    op, wl, ws, gpacked = gpu_weights(w, dev(Wt), form)
    opacked, os_, _ = O.prepare_weight(Wt, w.had_block, w.w_group, w.w_scale_dtype)
    check_weights(gpacked, host(ws), opacked, os_)
    Ad = dev(A.T) if A is not None else None
    Bd = dev(B.T) if B is not None else None
    ws_buf = W.qlinear_workspace(w.M, w.N, w.K, w.rank, DEV)
    y_dev = W.qlinear_forward(Xd, op, ws, w.had_block, w.w_group, Ad, Bd, workspace=ws_buf,
                              w_layout=wl)
    rows = sample_rows(w.M, seed)
    y = host(y_dev[torch.from_numpy(rows).to(DEV)])
    wsb = host(ws_buf)
    co, cl, so = W.qlinear_workspace_layout(w.M, w.N, w.K, w.rank, wl, w.w_group)
    kind, codes = workspace_codes(wsb, co, w.M, w.K, cl)
    gc = (O.unpack_int4(codes) if kind == "packed" else codes).astype(np.int16)[rows]
    gsx = wsb[so:so + 4 * w.M].view(np.float32)[rows]
    Xr = X[rows]
    _, ps, pc, _ = O.quantize_activation(Xr, w.had_block)
    diff = gc - pc
    assert np.all(np.abs(diff) <= 1)
    assert np.count_nonzero(diff) <= 1e-4 * diff.size
    assert np.all(np.abs(gsx.astype(np.float64) - ps) <= 1e-6 * ps)
    gws = host(ws)
    y_codes = O.qlinear_from_codes(gc, gsx, gpacked, gws, w.w_group, Xr, A, B)
    y_oracle = O.qlinear_forward(Xr, opacked, os_, w.had_block, w.w_group, A, B)
    check_rows(y, y_codes, y_oracle, f"{w.name} {form}")


PREFILL_WORKLOADS = ["downproj_4096x14336x4096_g128", "llama3_8b_qkv_4096x4096x6144",
                     "llama3_8b_o_4096x4096x4096", "llama3_8b_gateup_4096x4096x28672",
                     "llama3_8b_down_4096x14336x4096", "prefill_2048x4096x4096"]


@pytest.mark.parametrize("name", PREFILL_WORKLOADS)
def test_layer_full_size_as_benchmarked_f6(name):
    # the prefill workloads as bench.py times them: FP6 tiled weights
    run_full(synth.by_name(name), seed=len(name) + 1, form="f6")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", PREFILL_WORKLOADS + ["decode_8x4096x4096_r64"])
def test_layer_full_size_as_benchmarked(name):
    # the decode workload as bench.py times it, and the int4 operand forms
    w = synth.by_name(name)
    run_full(w, seed=len(name))
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N,K,b,g", [(4096, 4096, 4096, 0), (6144, 4096, 128, 0),
                                     (4096, 14336, 128, 128), (512, 14336, 128, 0)])
@pytest.mark.parametrize("layout", ["tiled", "tiled_f6"])
def test_quantize_weight_tiled_fused_rotation(N, K, b, g, layout):
    # The benchmark's weight preparation path (rotation fused into the tiled
    # quantizer) against the oracle's dense rotation and quantizer.
    rng = np.random.default_rng(N + K + b)
    Wt = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    Wt[:, 11] *= 40
    wt, ws = W.quantize_weight_int4(dev(Wt), b, g, torch.float16, layout=layout)
    opacked, os_, _ = O.prepare_weight(Wt, b, g, "float16")
    got = (untile_weights(host(wt), N) if layout == "tiled"
           else O.pack_int4(untile_f6(host(wt), N, K)))
    check_weights(got, host(ws), opacked, os_)
