"""The seeded synthetic inputs are deterministic and have the stated structure."""
import hashlib

import numpy as np

from bit_gemm_block_amd import synth


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_deterministic():
    w = synth.small("t", 16, 256, 64, rank=8)
    a, b = synth.make_inputs(w), synth.make_inputs(w)
    for k in ("X", "W", "A", "B"):
        assert _h(a[k]) == _h(b[k])
    w2 = synth.small("t", 16, 256, 64, rank=8, seed=1)
    assert _h(synth.make_inputs(w2)["X"]) != _h(a["X"])


def test_dtypes_and_shapes():
    d = synth.make_inputs(synth.TINY)
    assert d["X"].dtype == np.float32 and d["X"].shape == (16, 256)
    assert d["W"].dtype == np.float32 and d["W"].shape == (256, 256)
    assert d["A"].shape == (256, 8) and d["B"].shape == (8, 256)
    w = synth.small("t", 8, 512, 32, rank=4)
    d = synth.make_inputs(w)
    assert d["X"].dtype == np.float16 and d["A"].dtype == np.float16


def test_outlier_structure():
    w = synth.small("t", 256, 4096, 8, n_outlier=4, outlier_factor=100.0, bos_factor=500.0)
    X = synth.make_inputs(w)["X"].astype(np.float32)
    ch = synth.outlier_channels(4096, 4)
    assert ch.tolist() == [7, 1031, 2055, 3079]
    body = X[1:]
    others = np.delete(body, ch, axis=1)
    assert np.std(body[:, ch]) > 50 * np.std(others)
    assert abs(np.std(X[0]) - 500) < 50          # BOS row
    assert np.all(np.isfinite(X))


def test_no_bos_outliers_on_every_row():
    w = synth.small("t", 64, 1024, 8, n_outlier=8, outlier_factor=80.0, bos_factor=None)
    X = synth.make_inputs(w)["X"].astype(np.float32)
    ch = synth.outlier_channels(1024, 8)
    assert np.std(X[:, ch]) > 40 * np.std(np.delete(X, ch, axis=1))


def test_named_workloads():
    assert synth.PREFILL.M == 2048 and synth.PREFILL.had_block == 4096
    assert synth.DECODE.rank == 64 and synth.DECODE.M == 8
    assert synth.DOWN_PROJ.w_group == 128 and synth.DOWN_PROJ.K == 14336
    assert [w.N for w in synth.LLAMA3_8B] == [6144, 4096, 28672, 4096]
    assert synth.by_name(synth.TINY.name) is synth.TINY
