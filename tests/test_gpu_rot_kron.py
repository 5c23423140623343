"""Parity of the rotation on the fp16 matrix instruction for b = 256..4096
(rotq_mfma.hip: the 128-point transform of each sub-block on the matrix
instruction, then H_n across the n = b / 128 sub-blocks with lane and register
stages; Sylvester's construction gives H_b = H_n (x) H_128) against the CPU
oracle, through the C ABI.  It runs for the tiled 4-bit codes of fp16 rows with
one scale per row, and K a multiple of 4096 here (2048 for b up to 2048).

Bars (the fused-path bar, as for the butterfly kernel: the float32 sums of the
transform round in another order than the oracle's float64 ones):
* codes within one step of the oracle's on at most 0.01% of the elements;
* scales within 1e-6 relative;
* offset-binary tiles: the row sums equal the sums of the same call's codes
  at odd channels, bit-exact, and the tiles are the plain packed tiles of the
  same call XOR 0x08;
* against the butterfly kernel (the non-tiled packed layout of the same
  input), codes within one step on at most 0.02%.
A wrong lane permutation, stage sign or tile offset moves or mixes whole
sub-blocks, which fails the first bar at once.
"""
import numpy as np
import pytest
import torch

from oracle import w4a4_oracle as O
from bit_gemm_block_amd import synth
from bit_gemm_block_amd import w4a4 as W
from layouts import split_ob, untile_f6, untile_weights

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def codes_of(xq, M, K, layout):
    if layout == "f6_tiled":
        return untile_f6(host(xq), M, K).astype(np.int16), None
    if layout == "packed_tiled":
        return O.unpack_int4(untile_weights(host(xq), M)).astype(np.int16), None
    tiles, sums = split_ob(host(xq), M, K)
    return O.unpack_int4(untile_weights(tiles ^ 0x08, M)).astype(np.int16), sums


@pytest.mark.parametrize("M,K,b,layout", [
    (65, 4096, 4096, "f6_tiled"), (2048, 4096, 4096, "f6_tiled"),
    (4100, 4096, 4096, "packed_tiled"), (2048, 4096, 4096, "packed_tiled_ob"),
    (130, 8192, 4096, "f6_tiled"), (77, 16384, 4096, "packed_tiled_ob"),
    (300, 12288, 256, "f6_tiled"), (200, 4096, 512, "packed_tiled"),
    (97, 8192, 1024, "f6_tiled"), (150, 4096, 2048, "packed_tiled_ob"),
    (1000, 16384, 2048, "f6_tiled"), (90, 4096, 1024, "packed_tiled")])
def test_quantize_act_kron_matrix_rotation(M, K, b, layout):
    w = synth.small("qkron", M, K, 8, n_outlier=4, bos_factor=500.0)
    X = synth.make_inputs(w)["X"]
    print("quantize_act kron", M, K, b, layout, flush=True)
    xq, sx = W.quantize_act_int4(dev(X), b, layout=layout)
    _, ps, pc, _ = O.quantize_activation(X, b)
    got, sums = codes_of(xq, M, K, layout)
    diff = got - pc.astype(np.int16)
    assert np.all(np.abs(diff) <= 1)
    assert np.count_nonzero(diff) <= 1e-4 * diff.size
    assert np.all(np.abs(host(sx).astype(np.float64) - ps) <= 1e-6 * ps)
    if sums is not None:
        assert np.array_equal(sums, got[:, 1::2].astype(np.int64).sum(axis=1))
        xp, sp = W.quantize_act_int4(dev(X), b, layout="packed_tiled")
        tiles, _ = split_ob(host(xq), M, K)
        assert np.array_equal(untile_weights(tiles ^ 0x08, M), untile_weights(host(xp), M))
        assert np.array_equal(host(sp), host(sx))
    # the butterfly kernel's codes meet the same bar against these
    xb, _ = W.quantize_act_int4(dev(X), b, layout="packed")
    d2 = got - O.unpack_int4(host(xb)).astype(np.int16)
    assert np.all(np.abs(d2) <= 1)
    assert np.count_nonzero(d2) <= 2e-4 * d2.size


def test_quantize_act_kron_zero_and_constant_rows():
    # An all-zero row takes scale 0 and codes 0; a row with one non-zero
    # element rotates to +-v / 64 everywhere (codes +-7: the product with the
    # reciprocal of the scale is within 2^-21 of 7, far from a tie), so any
    # sign slip in the stages shows as a flipped code.
    M, K, b = 96, 4096, 4096
    X = np.zeros((M, K), np.float16)
    rng = np.random.default_rng(5)
    for r in range(1, M):
        X[r, rng.integers(0, K)] = np.float16(rng.uniform(0.5, 4.0) * (1 if r % 2 else -1))
    xq, sx = W.quantize_act_int4(dev(X), b, layout="f6_tiled")
    _, ps, pc, _ = O.quantize_activation(X, b)
    got = untile_f6(host(xq), M, K).astype(np.int16)
    assert np.array_equal(got, pc.astype(np.int16))
    assert np.array_equal(host(sx).astype(np.float64), ps)
    assert host(sx)[0] == 0 and not got[0].any()
