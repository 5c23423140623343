#!/usr/bin/env python3
"""Benchmark of the W4A4 quantized linear layer on one MI355X.

Headline: qlinear_forward on the prefill workload (X fp16 2048 x 4096, W
4096 x 4096 int4 per-channel fp16 scales, Hadamard block 4096, no low-rank
term) in int TOP/s (2*M*N*K per call).  Beside it: the decode workload
(X 8 x 4096, rank-64 X.A.B term) in algorithmic HBM GB/s, with the weights
rotated through enough distinct copies that the 256 MB last-level cache
cannot serve them.

One step = one qlinear_forward call (rotate + quantize, [X.A], int4 GEMM with
the dequant and low-rank epilogue).  Inputs and pre-quantized weights are
resident in device memory before the timed region.  The timed region is a
captured HIP graph of exactly --steps calls, bracketed by device
synchronisation and timed with events on the stream the kernels run on.

A third leg runs the layer with asymmetric group-wise activations (per
token and 128-channel group: scale and zero point) on the Llama-3-8B o-proj
shape (4096 x 4096 x 4096, rank-32 term), beside the symmetric layer on the
same workload.  A fourth runs the same shape with the in-GEMM 4-bit residual
of 32 salient channels in place of the rank-32 term.  A fifth runs the
prefill workload in MXFP4 (E2M1 elements, one E8M0 scale per 32) on the
scaled FP4 matrix instruction, against the dense FP4 peak.

The roofline object is the GEMM kernel alone (the dominant kernel): its
average launch duration from events around --steps back-to-back launches,
against the chip's dense int8 matrix peak.  cpu_baseline is the float64 CPU
oracle timed on a bounded row sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from bit_gemm_block_amd import synth  # noqa: E402
from bit_gemm_block_amd import w4a4 as W  # noqa: E402

PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 matrix peak, TOP/s
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense FP4 (MXFP4) matrix peak, TFLOP/s
PEAK_FP6_TOPS = 10100.0    # MI355X dense FP6 matrix peak (the int4 codes as E2M3), TOP/s
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, GB/s
LLC_BYTES = 256 << 20     # MI355X Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Layer:
    """Device-resident inputs of one workload with weights quantized on GPU."""

    def __init__(self, wl: synth.Workload, copies: int = 1, w_layout: str = "tiled_ob"):
        self.wl = wl
        self.w_layout = w_layout
        d = synth.make_inputs(wl)
        dev = "cuda:0"
        self.x = torch.from_numpy(d["X"]).to(dev)
        # Low-rank factors are stored transposed (At [r, K], Bt [N, r]).
        self.A = torch.from_numpy(d["A"].T.copy()).to(dev) if d["A"] is not None else None
        self.B = torch.from_numpy(d["B"].T.copy()).to(dev) if d["B"] is not None else None
        Wd = torch.from_numpy(d["W"]).to(dev)
        sdt = torch.float16 if wl.w_scale_dtype == "float16" else torch.float32
        ob = w_layout == "tiled_ob"
        f6 = w_layout == "tiled_f6"
        wq, ws = W.quantize_weight_int4(Wd, wl.had_block, wl.w_group, sdt,
                                        layout="tiled" if ob else w_layout)
        # Offset-binary weights are converted from the tiled ones; the W4A8
        # layer keeps the tiled form (the offset-binary and FP6 forms serve
        # 4-bit codes).
        wq8 = wq
        if ob:
            wq = W.weights_tiled_to_ob(wq, wl.N)
        if f6:
            wq8, _ = W.quantize_weight_int4(Wd, wl.had_block, wl.w_group, sdt, layout="tiled")
        del Wd
        # Distinct copies of the weights (and low-rank factors) so a decode
        # loop streams them from HBM rather than from the last-level cache.
        self.sets = [(wq, ws, self.A, self.B)]
        self.sets8 = [(wq8, ws, self.A, self.B)]
        for _ in range(copies - 1):
            c = (wq.clone(), ws.clone(), self.A.clone() if self.A is not None else None,
                 self.B.clone() if self.B is not None else None)
            self.sets.append(c)
            self.sets8.append((wq8.clone() if (ob or f6) else c[0],) + c[1:])
        self.y = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)
        self.ws = W.qlinear_workspace(wl.M, wl.N, wl.K, wl.rank, dev)
        torch.cuda.synchronize()

    def forward(self, i: int = 0, act_bits: int = 4):
        if act_bits == 8:
            wq, ws, A, B = self.sets8[i % len(self.sets8)]
            wl = "tiled" if self.w_layout in ("tiled_ob", "tiled_f6") else self.w_layout
        else:
            wq, ws, A, B = self.sets[i % len(self.sets)]
            wl = self.w_layout
        W.qlinear_forward(self.x, wq, ws, self.wl.had_block, self.wl.w_group, A, B,
                          y=self.y, workspace=self.ws, w_layout=wl, act_bits=act_bits)

    def forward_asym(self, i: int = 0):
        """The layer with asymmetric group-wise activations (tiled weights,
        per-channel scales, group = the Hadamard block)."""
        wq, ws, A, B = self.sets[i % len(self.sets)]
        W.qlinear_forward_asym(self.x, wq, ws, self.gsum, self.wl.had_block, A, B, y=self.y,
                               workspace=self.ws)

    def prepare_asym(self):
        self.gsum = W.weight_group_sums(self.sets8[0][0], self.wl.had_block, self.wl.N,
                                        w_layout="tiled")
        torch.cuda.synchronize()

    def algorithmic_bytes(self) -> int:
        wl = self.wl
        xb = 2 if wl.x_dtype == "float16" else 4
        sb = 2 if wl.w_scale_dtype == "float16" else 4
        nsc = wl.N if wl.w_group == 0 else wl.N * (wl.K // wl.w_group)
        lr = (wl.K * wl.rank + wl.rank * wl.N) * xb
        return wl.M * wl.K * xb + wl.N * wl.K // 2 + nsc * sb + lr + wl.M * wl.N * 4

    def ops(self) -> int:
        return 2 * self.wl.M * self.wl.N * self.wl.K


def gemm_bytes(wl: synth.Workload, w_layout: str = "tiled") -> int:
    """Bytes the GEMM must move once: the codes and scales of X, the weight
    codes and their scales, float32 Y.  Codes take 4 bits (6 bits in the FP6
    layouts); offset-binary operands add one int32 sum per row of X and of
    the weights."""
    sb = 2 if wl.w_scale_dtype == "float16" else 4
    nsc = wl.N if wl.w_group == 0 else wl.N * (wl.K // wl.w_group)
    sums = 4 * (wl.M + wl.N) if w_layout == "tiled_ob" else 0
    cb = 3 / 4 if w_layout == "tiled_f6" else 1 / 2   # bytes per code
    return int(cb * wl.M * wl.K) + 4 * wl.M + int(cb * wl.N * wl.K) + nsc * sb + \
        4 * wl.M * wl.N + sums


def gemm_peak(w_layout: str) -> float:
    """Dense peak of the matrix instruction the GEMM runs on, TOP/s."""
    return PEAK_FP6_TOPS if w_layout == "tiled_f6" else PEAK_INT8_TOPS


def gemm_kernel_name(layer: "Layer") -> str:
    if layer.w_layout == "tiled_f6":
        return "qgemm_f6_kernel (FP6 E2M3 operands)"
    if layer.wl.M <= 32:
        return "qgemm_skinny_kernel"
    return "qgemm_pipe_kernel" + (" (offset-binary)" if layer.w_layout == "tiled_ob" else "")


WARM_SECONDS = 0.25   # untimed replays before a timed one: clocks ramp up under load


def capture(fn, steps: int, warmup: int) -> "torch.cuda.CUDAGraph":
    """`steps` calls of fn(i) captured in one HIP graph after `warmup` eager calls."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                fn(i)
    torch.cuda.synchronize()
    return g


def warm(g, seconds: float = WARM_SECONDS) -> None:
    """Replays g (untimed) for about `seconds` of wall time, at least three
    times: first-launch costs, and the clocks rise from idle under load."""
    t0 = time.perf_counter()
    n = 0
    while n < 3 or time.perf_counter() - t0 < seconds:
        g.replay()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_graph(fn, steps: int, warmup: int) -> float:
    """Seconds per step: `steps` calls of fn(i) captured in one HIP graph,
    timed as one replay after the warm replays."""
    g = capture(fn, steps, warmup)
    warm(g)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    start.record(cur)
    g.replay()
    end.record(cur)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def replay_stats(fn, steps: int, warmup: int, reps: int = 15) -> dict:
    """Spread of the per-step time over `reps` replays of one graph of
    `steps` calls (each replay timed alone with events, after the warm
    replays): median, p10, p90."""
    g = capture(fn, steps, warmup)
    warm(g)
    cur = torch.cuda.current_stream()
    t = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(cur)
        g.replay()
        b.record(cur)
        torch.cuda.synchronize()
        t.append(a.elapsed_time(b) / steps)
    q = np.percentile(np.array(t), [10, 50, 90])
    return {"median_ms_per_step": float(q[1]), "p10_ms_per_step": float(q[0]),
            "p90_ms_per_step": float(q[2]), "replays": reps, "steps_per_replay": steps}


def read_clocks() -> list:
    """The current clock lines rocm-smi reports (informational)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=15)
        return [l.strip() for l in r.stdout.splitlines() if "clk" in l.lower()][:8]
    except Exception as e:  # pragma: no cover - informational only
        return [f"unavailable: {type(e).__name__}"]


def clocks_under_load(fn, steps: int, warmup: int, seconds: float = 1.5) -> list:
    """Clock readings taken while the GPU replays the graph of fn back to back
    (the clocks of the timed work, not of the idle device): a second thread
    samples rocm-smi while this one keeps the device busy."""
    import threading
    g = capture(fn, steps, warmup)
    warm(g)
    samples = []
    th = threading.Thread(target=lambda: samples.append(read_clocks()))
    th.start()
    t0 = time.perf_counter()
    n = 0
    while th.is_alive() or time.perf_counter() - t0 < seconds:
        g.replay()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
        if time.perf_counter() - t0 > 30:
            break
    torch.cuda.synchronize()
    th.join()
    return samples[0] if samples else []


def environment() -> dict:
    """ROCm and device identification, and the clocks rocm-smi reports at idle."""
    prop = torch.cuda.get_device_properties(0)
    return {"rocm": torch.version.hip, "torch": torch.__version__, "device": prop.name,
            "compute_units": prop.multi_processor_count,
            "arch": getattr(prop, "gcnArchName", None), "clocks_idle": read_clocks()}


def prefill_shapes(steps: int, warmup: int, w_layout: str) -> dict:
    """qlinear_forward TOP/s on the other prefill shapes: the grouped
    down-projection and the Llama-3-8B decoder linears (4096 tokens)."""
    out = {}
    for wl in [synth.DOWN_PROJ] + synth.LLAMA3_8B:
        # FP6 weights serve every shape; else offset-binary weights serve
        # per-channel scales and grouped ones stay tiled
        lay = w_layout if w_layout == "tiled_f6" else "tiled_ob" if wl.w_group == 0 else "tiled"
        layer = Layer(wl, w_layout=lay)
        t = time_graph(layer.forward, steps, warmup)
        tops = layer.ops() / t / 1e12
        out[wl.name] = {"TOP/s": tops, "frac_of_matrix_peak": tops / gemm_peak(lay),
                        "ms_per_step": t * 1e3, "had_block": wl.had_block,
                        "w_group": wl.w_group, "rank": wl.rank, "w_layout": layer.w_layout}
        log(f"shape {wl.name}: {t * 1e6:.1f} us/step, {tops:.0f} TOP/s")
        del layer
        torch.cuda.empty_cache()
    return out


def kernel_launches(layer: Layer) -> dict:
    """The kernels of the path as separate launches with the same arguments
    and code layout as inside qlinear_forward (rotation + quantization into
    the GEMM's code layout, then the GEMM)."""
    wl = layer.wl
    tiled = layer.w_layout in ("tiled", "tiled_ob")
    # the code layout qlinear_forward hands the GEMM: FP6 tiles with FP6
    # weights, packed tiles with tiled weights (offset-binary ones above 32
    # rows with offset-binary weights), int8 rows otherwise
    ob = layer.w_layout == "tiled_ob" and wl.M > 32
    f6 = layer.w_layout == "tiled_f6"
    lay = "f6_tiled" if f6 else "packed_tiled_ob" if ob else "packed_tiled" if tiled else "i8"
    if f6:
        xq = torch.empty((W.pad16(wl.M), 3 * wl.K // 4), dtype=torch.uint8, device="cuda:0")
    elif ob:
        xq = torch.empty((W.ob_bytes(wl.M, wl.K),), dtype=torch.uint8, device="cuda:0")
    else:
        xq = torch.empty((W.pad16(wl.M) if tiled else wl.M, wl.K // 2 if tiled else wl.K),
                         dtype=torch.uint8, device="cuda:0")
    sx = torch.empty((wl.M,), dtype=torch.float32, device="cuda:0")
    W.quantize_act_int4(layer.x, wl.had_block, xq, sx, layout=lay)
    torch.cuda.synchronize()
    return {
        "rotq": lambda i: W.quantize_act_int4(layer.x, wl.had_block, xq, sx, layout=lay),
        "qgemm": lambda i: W.qgemm_w4a4(xq, sx, layer.sets[i % len(layer.sets)][0],
                                        layer.sets[i % len(layer.sets)][1], wl.w_group,
                                        y=layer.y, layout=lay, w_layout=layer.w_layout,
                                        M=wl.M, N=wl.N),
    }


def kernel_times(layer: Layer, steps: int, warmup: int) -> dict:
    """Average duration of each kernel of the path, launched alone:
    `steps` launches replayed from one HIP graph, timed with events on the
    stream they run on."""
    return {k: time_graph(f, steps, warmup) for k, f in kernel_launches(layer).items()}


def asym_kernel_times(layer: Layer, steps: int, warmup: int) -> dict:
    """Kernel durations of the asymmetric path, launched alone with the
    arguments of qlinear_forward_asym (packed tiled codes)."""
    wl = layer.wl
    G = wl.K // wl.had_block
    xq = torch.empty((W.pad16(wl.M), wl.K // 2), dtype=torch.uint8, device="cuda:0")
    sx = torch.empty((wl.M, G), dtype=torch.float32, device="cuda:0")
    zx = torch.empty((wl.M, G), dtype=torch.int32, device="cuda:0")
    q = lambda i: W.quantize_act_asym_int4(layer.x, wl.had_block, wl.had_block, "packed_tiled",
                                           xq, sx, zx)
    q(0)
    torch.cuda.synchronize()
    out = {"rotq_asym": time_graph(q, steps, warmup)}
    out["qgemm_asym"] = time_graph(
        lambda i: W.qgemm_asym(xq, sx, zx, wl.had_block, layer.sets[0][0], layer.sets[0][1],
                               layer.gsum, y=layer.y), steps, warmup)
    return out


def decode_forms(wl: synth.Workload, copies: int, steps: int, warmup: int) -> dict:
    """The decode workload in the other 4-bit forms, each with `copies`
    distinct weight sets so that the weights stream from HBM: MXFP4 and the
    asymmetric layer with the workload's low-rank term, the in-GEMM residual
    (its rank as residual channels) in its place.  Algorithmic bytes: X, the
    form's weight codes and per-weight side data, A and B when used, Y."""
    dev = "cuda:0"
    d = synth.make_inputs(wl)
    x = torch.from_numpy(d["X"]).to(dev)
    Wd = torch.from_numpy(d["W"]).to(dev)
    At = torch.from_numpy(d["A"].T.copy()).to(dev)
    Bt = torch.from_numpy(d["B"].T.copy()).to(dev)
    M, N, K, r, b = wl.M, wl.N, wl.K, wl.rank, wl.had_block
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    wsb = W.qlinear_workspace(M, N, K, r, dev)
    base = 2 * M * K + 4 * M * N
    lr = 2 * (K * r + r * N)
    out = {}

    def run(name, prep, fwd, side_bytes, uses_lr):
        sets = [prep()]
        for _ in range(copies - 1):
            sets.append(tuple(t.clone() for t in sets[0]))
        t = time_graph(lambda i: fwd(*sets[i % copies]), steps, warmup)
        nbytes = base + N * K // 2 + side_bytes + (lr if uses_lr else 0)
        out[name] = {"us_per_step": t * 1e6, "GB/s": nbytes / t / 1e9, "bytes_per_step": nbytes}
        log(f"decode {name}: {t * 1e6:.2f} us/step, {nbytes / t / 1e9:.0f} GB/s")
        del sets

    run("mxfp4", lambda: W.quantize_mxfp4(Wd, b, "packed_tiled"),
        lambda wq, ws: W.qlinear_forward_mxfp4(x, wq, ws, N, b, At, Bt, y=y, workspace=wsb),
        N * K // 32, True)

    def prep_asym():
        wq, ws = W.quantize_weight_int4(Wd, b, 0, torch.float16, layout="tiled")
        return wq, ws, W.weight_group_sums(wq, b, N, w_layout="tiled")
    run("asymmetric", prep_asym,
        lambda wq, ws, gs: W.qlinear_forward_asym(x, wq, ws, gs, b, At, Bt, y=y, workspace=wsb),
        2 * N + 4 * N * (K // b), True)
    run("residual", lambda: W.quantize_weight_residual_int4(Wd, b, r, torch.float16),
        lambda wq, ws: W.qlinear_forward_residual(x, wq, ws, r, b, y=y, workspace=wsb),
        2 * N + N * W.res_pad(r) // 2, False)
    del x, Wd, At, Bt, y, wsb
    return out


CALIB_BYTES = 256 << 20   # the calibration copy reads and writes this much
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qgemm_prefill_traffic.txt")
GEMM_SOURCES = [os.path.join(ROOT, "bit_gemm_block_amd", "csrc", f)
                for f in ("qgemm.hip", "qgemm_f6.hip", "gemm_common.h", "w4a4_internal.h")]


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profile_kernels(steps: int, w_layout: str, decode_w_layout: str) -> None:
    """Launch the kernels alone, eagerly, for hardware counters: the prefill
    rotation + quantization and GEMM `steps` times each; the decode layer
    (rotation launch with the low-rank and read-ahead roles, then the skinny
    GEMM) `steps` times over weight copies that exceed the last-level cache;
    then a plain elementwise copy of CALIB_BYTES, whose counter readings
    calibrate the byte counters."""
    pre = Layer(synth.PREFILL, w_layout=w_layout)
    for name, f in kernel_launches(pre).items():
        for i in range(steps):
            f(i)
        torch.cuda.synchronize()
    del pre
    probe = synth.DECODE
    per_set = probe.N * probe.K // 2 + probe.N * 2 + 2 * (probe.K + probe.N) * probe.rank * 2
    dec = Layer(probe, copies=int(np.ceil(3 * LLC_BYTES / per_set)), w_layout=decode_w_layout)
    for i in range(steps):
        dec.forward(i)
    torch.cuda.synchronize()
    del dec
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"profiled {steps} launches of each prefill kernel, {steps} decode layers and 5 "
        f"copies of {CALIB_BYTES} bytes")


def read_traffic(algorithmic: float, w_layout: str) -> dict | None:
    """HBM bytes per GEMM launch from the committed counter summary, or None
    when the summary is missing, was taken on another weight layout, or the
    GEMM source changed since it was made."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256_16") != gemm_source_hash() or kv.get("w_layout") != w_layout:
        return None
    try:
        fetch = float(kv["gemm_fetch_bytes_per_launch"])
        write = float(kv["gemm_write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None
    return {"fetch_bytes": fetch, "write_bytes": write, "bytes": fetch + write,
            "vs_algorithmic": (fetch + write) / algorithmic}


def cpu_baseline(wl: synth.Workload, seconds: float) -> dict:
    """The float64 oracle on the whole workload, repeated until `seconds` of
    CPU time have passed (at least once)."""
    from oracle import w4a4_oracle as O
    blas = None
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((p.get("num_threads", 1) for p in info), default=1)
        blas = ", ".join(sorted({str(p.get("internal_api")) for p in info if p.get("user_api") == "blas"}))
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    d = synth.make_inputs(wl)
    X = d["X"]
    wq, ws, _ = O.prepare_weight(d["W"], wl.had_block, wl.w_group, wl.w_scale_dtype)
    A, B = d["A"], d["B"]
    O.qlinear_forward(X[:8], wq, ws, wl.had_block, wl.w_group, A, B)  # warm caches
    calls = 0
    t0 = time.perf_counter()
    while True:
        O.qlinear_forward(X, wq, ws, wl.had_block, wl.w_group, A, B)
        calls += 1
        t = time.perf_counter() - t0
        if t >= seconds:
            break
    return {"value": calls * 2 * wl.M * wl.N * wl.K / t / 1e12, "unit": "TOP/s",
            "cores": int(threads), "kind": "oracle", "seconds": t, "blas": blas,
            "ms_per_call": t / calls * 1e3,
            "sample": f"{calls} oracle calls on the whole {wl.M}-row {wl.name} workload "
                      f"(weights prepared untimed)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--w-layout", choices=["tiled_f6", "tiled_ob", "tiled", "rowmajor"],
                    default="tiled_f6", help="weight layout of the prefill workloads")
    ap.add_argument("--decode-w-layout", choices=["tiled_ob", "tiled", "rowmajor", "tiled_f6"],
                    default="tiled_ob", help="weight layout of the decode workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-offq", action="store_true")
    ap.add_argument("--no-serq", action="store_true")
    ap.add_argument("--no-mxfp4", action="store_true")
    ap.add_argument("--no-shapes", action="store_true")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="only launch the prefill kernels and a calibration copy (for counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the W4A4 linear path of this library runs on a "
              "single device and has no multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    W.lib()
    if args.profile_kernels:
        profile_kernels(args.steps, args.w_layout, args.decode_w_layout)
        return 0

    # ---- prefill: the headline ------------------------------------------------
    pre = Layer(synth.PREFILL, w_layout=args.w_layout)
    log(f"prefill: {pre.wl.name} ({args.w_layout} weights) timing {args.steps} steps")
    t_step = time_graph(pre.forward, args.steps, args.warmup)
    kt = kernel_times(pre, args.steps, args.warmup)
    # W4A8 layers (8-bit activations beside the 4-bit weights), same workload.
    t_step8 = time_graph(lambda i: pre.forward(i, act_bits=8), args.steps, args.warmup)
    pre_stats = replay_stats(pre.forward, args.steps, args.warmup)
    clocks_load = clocks_under_load(pre.forward, args.steps, args.warmup)
    tops = pre.ops() / t_step / 1e12
    gemm_tops = pre.ops() / kt["qgemm"] / 1e12
    peak = gemm_peak(args.w_layout)
    code_bytes = pre.wl.M * pre.wl.K * 3 // 4 if args.w_layout == "tiled_f6" else pre.wl.M * pre.wl.K // 2
    rot_bytes = pre.wl.M * pre.wl.K * 2 + code_bytes + 4 * pre.wl.M  # X in, codes + scales out
    log(f"prefill: {t_step * 1e6:.2f} us/step, {tops:.1f} TOP/s; qgemm {kt['qgemm'] * 1e6:.2f} us "
        f"({gemm_tops:.1f} TOP/s), rotq {kt['rotq'] * 1e6:.2f} us "
        f"({rot_bytes / kt['rotq'] / 1e9:.0f} GB/s)")

    # ---- decode ----------------------------------------------------------------
    decode = None
    if not args.no_decode:
        probe = synth.DECODE
        per_set = probe.N * probe.K // 2 + probe.N * 2 + 2 * (probe.K + probe.N) * probe.rank * 2
        copies = int(np.ceil(3 * LLC_BYTES / per_set))
        dec = Layer(probe, copies=copies, w_layout=args.decode_w_layout)
        log(f"decode: {dec.wl.name} with {copies} weight copies, timing {args.steps} steps")
        t_dec = time_graph(dec.forward, args.steps, args.warmup)
        dec_stats = replay_stats(dec.forward, args.steps, args.warmup)
        kd = kernel_times(dec, args.steps, args.warmup)
        gbs = dec.algorithmic_bytes() / t_dec / 1e9
        log(f"decode: {t_dec * 1e6:.2f} us/step, {gbs:.0f} GB/s")
        t_dec8 = time_graph(lambda i: dec.forward(i, act_bits=8), args.steps, args.warmup)
        forms = decode_forms(probe, copies, args.steps, args.warmup)
        decode = {
            "metric": "W4A4 qlinear HBM GB/s (M=8)", "value": gbs, "unit": "GB/s",
            "ms_per_step": t_dec * 1e3, "frac_of_hbm": gbs / PEAK_HBM_GBS,
            "spread": dec_stats,
            "roofline": {"bound": "hbm", "scope": "whole call (every kernel of one step)",
                         "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "bytes_per_step": dec.algorithmic_bytes(),
                         "us_per_step": t_dec * 1e6},
            "bytes_per_step": dec.algorithmic_bytes(), "weight_copies": copies,
            "kernels_us": {k: v * 1e6 for k, v in kd.items()},
            "w4a8": {"value": dec.algorithmic_bytes() / t_dec8 / 1e9, "unit": "GB/s",
                     "ms_per_step": t_dec8 * 1e3},
            "other_forms": forms,
            "config": {"workload": dec.wl.name, "M": dec.wl.M, "N": dec.wl.N, "K": dec.wl.K,
                       "had_block": dec.wl.had_block, "w_group": dec.wl.w_group,
                       "rank": dec.wl.rank},
        }
        del dec

    # ---- asymmetric group-wise activations (OffQ), Llama-3-8B o-proj shape ------
    offq = None
    if not args.no_offq:
        ow = synth.by_name("llama3_8b_o_4096x4096x4096")
        lay = Layer(ow, w_layout="tiled")
        lay.prepare_asym()
        log(f"offq: {ow.name} timing {args.steps} steps (asymmetric and symmetric)")
        t_asym = time_graph(lay.forward_asym, args.steps, args.warmup)
        t_sym = time_graph(lay.forward, args.steps, args.warmup)
        ka = asym_kernel_times(lay, args.steps, args.warmup)
        ks = kernel_times(lay, args.steps, args.warmup)
        gemm_tops_a = lay.ops() / ka["qgemm_asym"] / 1e12
        log(f"offq: asym {t_asym * 1e6:.2f} us/step ({lay.ops() / t_asym / 1e12:.1f} TOP/s), "
            f"sym {t_sym * 1e6:.2f} us/step; qgemm_asym {ka['qgemm_asym'] * 1e6:.2f} us, "
            f"rotq_asym {ka['rotq_asym'] * 1e6:.2f} us")
        offq = {
            "metric": "W4A4 qlinear TOPS, asymmetric group-wise activations",
            "value": lay.ops() / t_asym / 1e12, "unit": "TOP/s", "ms_per_step": t_asym * 1e3,
            "symmetric_same_workload": {"value": lay.ops() / t_sym / 1e12, "unit": "TOP/s",
                                        "ms_per_step": t_sym * 1e3},
            "gemm": {"kernel": "qgemm_pipe_kernel (asymmetric groups)", "achieved": gemm_tops_a,
                     "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": gemm_tops_a / PEAK_INT8_TOPS},
            "kernels_us": {**{k: v * 1e6 for k, v in ka.items()},
                           **{k + "_sym": v * 1e6 for k, v in ks.items()}},
            "config": {"workload": ow.name, "M": ow.M, "N": ow.N, "K": ow.K,
                       "had_block": ow.had_block, "group": ow.had_block, "rank": ow.rank},
        }
        del lay

    # ---- in-GEMM 4-bit residual of salient channels, same o-proj shape -------
    serq = None
    if not args.no_serq:
        rw = synth.by_name("llama3_8b_o_4096x4096x4096")
        r, b = rw.rank, rw.had_block       # the residual takes the rank-32 term's place
        d = synth.make_inputs(rw)
        dev = "cuda:0"
        x = torch.from_numpy(d["X"]).to(dev)
        Wd = torch.from_numpy(d["W"]).to(dev)
        wq, ws = W.quantize_weight_residual_int4(Wd, b, r, torch.float16)
        del Wd, d
        y = torch.empty((rw.M, rw.N), dtype=torch.float32, device=dev)
        wsb = W.qlinear_workspace(rw.M, rw.N, rw.K, 0, dev)
        log(f"serq: {rw.name} with an in-GEMM residual of {r} channels, timing {args.steps} steps")
        t_res = time_graph(lambda i: W.qlinear_forward_residual(x, wq, ws, r, b, y=y, workspace=wsb),
                           args.steps, args.warmup)
        xq, sx = W.quantize_act_int4(x, b, layout="packed_tiled")
        torch.cuda.synchronize()
        t_g = time_graph(lambda i: W.qgemm_residual(xq, sx, wq, ws, r, rw.M, rw.N, rw.K, y=y),
                         args.steps, args.warmup)
        ops = 2 * rw.M * rw.N * rw.K
        log(f"serq: {t_res * 1e6:.2f} us/step ({ops / t_res / 1e12:.1f} TOP/s); qgemm_residual "
            f"{t_g * 1e6:.2f} us ({ops / t_g / 1e12:.1f} TOP/s)")
        serq = {
            "metric": "W4A4 qlinear TOPS with the in-GEMM 4-bit residual",
            "value": ops / t_res / 1e12, "unit": "TOP/s", "ms_per_step": t_res * 1e3,
            "gemm": {"kernel": "qgemm_pipe_kernel (residual)", "achieved": ops / t_g / 1e12,
                     "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": ops / t_g / 1e12 / PEAK_INT8_TOPS, "us_per_launch": t_g * 1e6,
                     "ops_per_launch": ops},
            "dense_lowrank_same_workload": (offq or {}).get("symmetric_same_workload"),
            "config": {"workload": rw.name, "M": rw.M, "N": rw.N, "K": rw.K, "had_block": b,
                       "residual_channels": r},
        }
        del x, wq, ws, y, wsb, xq, sx

    # ---- MXFP4 form of the layer, prefill workload ---------------------------
    mxfp4 = None
    if not args.no_mxfp4:
        mw = synth.PREFILL
        d = synth.make_inputs(mw)
        dev = "cuda:0"
        x = torch.from_numpy(d["X"]).to(dev)
        Wd = torch.from_numpy(d["W"]).to(dev)
        wq, ws = W.quantize_mxfp4(Wd, mw.had_block, "packed_tiled")
        del Wd, d
        y = torch.empty((mw.M, mw.N), dtype=torch.float32, device=dev)
        wsb = W.qlinear_workspace(mw.M, mw.N, mw.K, 0, dev)
        log(f"mxfp4: {mw.name} timing {args.steps} steps")
        t_mx = time_graph(lambda i: W.qlinear_forward_mxfp4(x, wq, ws, mw.N, mw.had_block, y=y,
                                                            workspace=wsb),
                          args.steps, args.warmup)
        xq, xs = W.quantize_mxfp4(x, mw.had_block, "packed_tiled")
        torch.cuda.synchronize()
        t_q = time_graph(lambda i: W.quantize_mxfp4(x, mw.had_block, "packed_tiled", xq, xs),
                         args.steps, args.warmup)
        t_g = time_graph(lambda i: W.qgemm_mxfp4(xq, xs, wq, ws, mw.M, mw.N, mw.K, y=y),
                         args.steps, args.warmup)
        ops = 2 * mw.M * mw.N * mw.K
        log(f"mxfp4: {t_mx * 1e6:.2f} us/step ({ops / t_mx / 1e12:.1f} TFLOP/s); qgemm_mxfp4 "
            f"{t_g * 1e6:.2f} us ({ops / t_g / 1e12:.1f} TFLOP/s), quantize {t_q * 1e6:.2f} us")
        mxfp4 = {
            "metric": "MXFP4 qlinear TFLOP/s (M=2048), K=N=4096",
            "value": ops / t_mx / 1e12, "unit": "TFLOP/s", "ms_per_step": t_mx * 1e3,
            "gemm": {"kernel": "qgemm_mx_kernel", "achieved": ops / t_g / 1e12,
                     "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": ops / t_g / 1e12 / PEAK_FP4_TFLOPS, "us_per_launch": t_g * 1e6,
                     "ops_per_launch": ops},
            "kernels_us": {"quantize_mxfp4": t_q * 1e6, "qgemm_mxfp4": t_g * 1e6},
            "config": {"workload": mw.name, "M": mw.M, "N": mw.N, "K": mw.K,
                       "had_block": mw.had_block, "block": 32},
        }
        del x, wq, ws, y, wsb, xq, xs

    shapes = None if args.no_shapes else prefill_shapes(min(args.steps, 50), args.warmup,
                                                        args.w_layout)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle for {args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(synth.PREFILL, args.cpu_seconds)

    out = {
        "metric": "W4A4 qlinear TOPS (M=2048), K=N=4096",
        "value": tops,
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": pre.wl.name, "M": pre.wl.M, "N": pre.wl.N, "K": pre.wl.K,
                   "had_block": pre.wl.had_block, "w_group": pre.wl.w_group,
                   "rank": pre.wl.rank, "x_dtype": pre.wl.x_dtype,
                   "w_layout": args.w_layout,
                   "matrix_operands": ("int4 codes as FP6 E2M3, float32 sums (exact integers)"
                                       if args.w_layout == "tiled_f6"
                                       else "int4 codes widened to int8, int32 sums")},
        "frac_of_matrix_peak": tops / peak,
        "roofline": {"bound": "mfma", "kernel": gemm_kernel_name(pre), "achieved": gemm_tops,
                     "peak": peak, "unit": "TOP/s", "frac": gemm_tops / peak,
                     "ops_per_launch": pre.ops(), "us_per_launch": kt["qgemm"] * 1e6,
                     "algorithmic_bytes_per_launch": gemm_bytes(pre.wl, args.w_layout),
                     "traffic": read_traffic(gemm_bytes(pre.wl, args.w_layout), args.w_layout)},
        "spread": pre_stats,
        "kernels_us": {k: v * 1e6 for k, v in kt.items()},
        "rotq_gbs": rot_bytes / kt["rotq"] / 1e9,
        "w4a8": {"metric": "W4A8 qlinear TOPS (M=2048), K=N=4096", "value": pre.ops() / t_step8 / 1e12,
                 "unit": "TOP/s", "ms_per_step": t_step8 * 1e3},
        "decode": decode,
        "offq": offq,
        "serq": serq,
        "mxfp4": mxfp4,
        "prefill_shapes": shapes,
        "cpu_baseline": cpu,
        "environment": {**environment(), "clocks_under_prefill_load": clocks_load},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
