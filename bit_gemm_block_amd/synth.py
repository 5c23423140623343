"""Seeded synthetic inputs for the W4A4 quantized linear layer.

This module only draws random numbers and arranges them into the shapes and
outlier structure of the workloads; it holds none of the method's arithmetic
(no rotation, no quantization, no packing).  Both the CPU oracle tests and the
GPU path take their inputs from here.

Outlier structure (DynamicPTQ, "Planteamiento del problema": massive
activations sit in a few fixed channels and are often tied to the BOS token;
OffQ, "Declaración del problema": sparse, very large values in specific
channels dominate the dynamic range):

* activations are standard normal;
* ``n_outlier`` fixed channels ``{7 + i*K/n_outlier}`` are multiplied by
  ``outlier_factor`` on every row except row 0;
* when ``bos_factor`` is set, row 0 (the BOS-like token) is multiplied by it
  on every channel.  The two factors do not compound: a factor of 500 times
  100 would overflow fp16, so the BOS row takes only its own factor.

Weights are ``0.02 * N(0, 1)``; the low-rank factors are ``0.01 * N(0, 1)``;
the second argument of N(mu, sigma) is the standard deviation.  Draws are
taken in the order X, W, A, B from ``numpy.random.default_rng(seed)`` in
float32 and then cast to the activation dtype with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one W4A4 linear call."""
    name: str
    M: int
    K: int
    N: int
    x_dtype: str            # "float32" or "float16"
    n_outlier: int          # number of massive channels
    outlier_factor: float
    bos_factor: Optional[float]
    had_block: int          # Hadamard block size b (power of two dividing K)
    w_group: int            # weight scale group along K, 0 = one scale per output channel
    rank: int               # rank r of the X.A.B correction, 0 = none
    w_scale_dtype: str      # "float32" or "float16"
    seed: int = 0
    extra: dict = field(default_factory=dict)


def outlier_channels(K: int, n_outlier: int) -> np.ndarray:
    """Fixed massive-channel indices {7 + i*K/n : i < n}."""
    if n_outlier <= 0:
        return np.zeros(0, dtype=np.int64)
    step = K // n_outlier
    return np.array([7 + i * step for i in range(n_outlier)], dtype=np.int64)


def make_activation(rng: np.random.Generator, M: int, K: int, x_dtype: str,
                    n_outlier: int, outlier_factor: float,
                    bos_factor: Optional[float]) -> np.ndarray:
    x = rng.standard_normal((M, K), dtype=np.float32)
    ch = outlier_channels(K, n_outlier)
    if ch.size and M > 0:
        first = 1 if bos_factor is not None else 0
        x[first:, ch] *= np.float32(outlier_factor)
    if bos_factor is not None and M > 0:
        x[0, :] *= np.float32(bos_factor)
    return x.astype(np.dtype(x_dtype))


def make_inputs(w: Workload, rows: Optional[int] = None) -> dict:
    """Draw X [M,K], W [N,K] (float32), and A [K,r], B [r,N] (X's dtype).

    ``rows`` lets a caller draw a smaller M with the same recipe (the first
    ``rows`` rows are not the same numbers as the full draw; use it only for
    self-contained cases).
    """
    M = w.M if rows is None else rows
    rng = np.random.default_rng(w.seed)
    X = make_activation(rng, M, w.K, w.x_dtype, w.n_outlier,
                        w.outlier_factor, w.bos_factor)
    W = (np.float32(0.02) * rng.standard_normal((w.N, w.K), dtype=np.float32))
    out = {"X": X, "W": W, "A": None, "B": None}
    if w.rank > 0:
        A = np.float32(0.01) * rng.standard_normal((w.K, w.rank), dtype=np.float32)
        B = np.float32(0.01) * rng.standard_normal((w.rank, w.N), dtype=np.float32)
        out["A"] = A.astype(np.dtype(w.x_dtype))
        out["B"] = B.astype(np.dtype(w.x_dtype))
    return out


# The workloads the path is measured and checked on.
TINY = Workload("tiny_16x256x256_r8", 16, 256, 256, "float32", 1, 50.0, None,
                256, 0, 8, "float32")
PREFILL = Workload("prefill_2048x4096x4096", 2048, 4096, 4096, "float16", 4,
                   100.0, 500.0, 4096, 0, 0, "float16")
DECODE = Workload("decode_8x4096x4096_r64", 8, 4096, 4096, "float16", 4,
                  100.0, 500.0, 4096, 0, 64, "float16")
DOWN_PROJ = Workload("downproj_4096x14336x4096_g128", 4096, 14336, 4096,
                     "float16", 8, 80.0, None, 128, 128, 0, "float16")
LLAMA3_8B = [
    Workload("llama3_8b_qkv_4096x4096x6144", 4096, 4096, 6144, "float16", 4,
             100.0, 500.0, 128, 0, 32, "float16"),
    Workload("llama3_8b_o_4096x4096x4096", 4096, 4096, 4096, "float16", 4,
             100.0, 500.0, 128, 0, 32, "float16"),
    Workload("llama3_8b_gateup_4096x4096x28672", 4096, 4096, 28672, "float16",
             4, 100.0, 500.0, 128, 0, 32, "float16"),
    Workload("llama3_8b_down_4096x14336x4096", 4096, 14336, 4096, "float16",
             4, 100.0, 500.0, 128, 0, 32, "float16"),
]

ALL = [TINY, PREFILL, DECODE, DOWN_PROJ] + LLAMA3_8B


def by_name(name: str) -> Workload:
    for w in ALL:
        if w.name == name:
            return w
    raise KeyError(name)


def small(name: str, M: int, K: int, N: int, *, x_dtype="float16", n_outlier=2,
          outlier_factor=100.0, bos_factor: Optional[float] = 500.0,
          had_block=128, w_group=0, rank=0, w_scale_dtype="float16",
          seed=0) -> Workload:
    """A reduced workload with the same recipe, for parity tests."""
    return Workload(name, M, K, N, x_dtype, n_outlier, outlier_factor,
                    bos_factor, had_block, w_group, rank, w_scale_dtype, seed)
