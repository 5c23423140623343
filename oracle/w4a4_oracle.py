"""Plain CPU oracle of the W4A4 quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The GPU library never calls it,
and it shares no code with the GPU library: no kernels, no helpers, no tables.

What is computed, and where the pages fix it
---------------------------------------------
* Rotation: each row of X is cut into contiguous blocks of ``b`` channels and
  every block is multiplied by a Hadamard matrix whose first row is all ones,
  so that a single-channel outlier becomes a constant offset over its block
  (OffQ page, "Metodología", step 2 "Absorción mediante Desplazamiento", and
  step 3 "Implementación por Grupos").  We take the Sylvester matrix
  H[i, j] = (-1)^popcount(i & j), normalised by 1/sqrt(b) so that the rotation
  keeps the L2 norm.  It is applied as a dense float64 matmul, not as a fast
  transform, and rounded once to float32.
* Activation quantization: per token ("on the fly") symmetric int4 with an
  absmax scale (SERQ page, "Resumen técnico" §1 and §2 item 2: the main path
  stays at 4 bits, INT4).  In float32: a = max|x|, s = a / 7, q = clamp(rint(x / s),
  -7, 7) with round-half-to-even; when s is 0 every code is 0.
* Weight preparation (offline): the same rotation, then symmetric
  round-to-nearest int4 per output channel, or per group of ``g`` channels
  along K (DynamicPTQ page, "Resultados": RTN weight quantizer).  The scale is
  stored in its storage dtype, and the codes are taken against the stored
  scale.
* Packing: two's-complement nibbles, element 2j in the low nibble of byte j.
* Integer GEMM: acc[m, n] = sum_k qx[m, k] * qw[n, k], computed as a float64
  matmul of the integer codes, which is exact because every partial sum is an
  integer of magnitude at most 127*8*K < 2^53 (8-bit activation codes included).
* Low-rank term: the single low-rank compensation added to the 4-bit product
  (SERQ page, "Resumen técnico" §2 item 2).  Written as (X @ A) @ B in float64
  on the unrotated input as given.
* Epilogue: Y = s_x[m] * s_w[n] * acc[m, n] (or the sum over weight groups)
  + low-rank term, in float64, rounded once to float32.
* Asymmetric group-wise activations (OffQ page, "Metodología" steps 2-3):
  the all-ones Hadamard row turns a group's outlier into a constant offset,
  which the zero point of an asymmetric per-group quantizer absorbs.  With
  the group equal to the Hadamard block, per token and group in float32:
  s = (max - min) / 15, z = rint(-min / s), q = clamp(rint(x / s) + z, 0, 15),
  so that x ~ s (q - z).  The zero point is an integer that is not clamped
  to the code range: an offset larger than the group's spread moves z past
  0 or 15, and only then is it absorbed whole.  A group with no spread
  (max = min = c) takes the range spanned by c and 0, so that it is coded
  as c rather than as 0; s = 0 (c = 0) gives q = z = 0.  The product is
  Y = sum_g s_x[m,g] s_w[n] (sum_{k in g} q_x q_w - z[m,g] sum_{k in g} q_w[n,k])
  + the low-rank term; the weight sums are an offline input.
* In-GEMM 4-bit residual of salient channels (SERQ page, "Metodología"
  items 2-3): the weight rows that collect the most error (input channels,
  permuted offline to the front, so that they are the first r channels) are
  reconstructed by one 4-bit matrix R, the quantization error of those
  channels, and the layer adds X_s . R^T, X_s being the same 4-bit
  activation codes of those channels.  With per-channel weight scale s:
  e = x~ - s q (float32), q_r = clamp(rint(e / (s/8)), -8, 7) for k < r, and
  Y = s_x s_w (sum_k q_x q_w + (1/8) sum_{k<r} q_x q_r).  The step s/8 lets
  R cover the whole rounding error (|e| <= s/2 gives |q_r| <= 4) and keeps
  both sums in one integer: 8 sum_k q_x q_w + sum_{k<r} q_x q_r.
* MXFP4 (SERQ page, "Metodología" item 2 and "Contribuciones Clave": the
  4-bit path may be INT4 or MXFP4, the microscaling format): read as the
  OCP microscaling definition.  Every 32 consecutive elements along K share
  a power-of-two scale 2^e (an E8M0 byte e + 127) with
  e = max(floor(log2(max|v|)) - 2, -127) (e = -127 for an all-zero block);
  each element is v / 2^e rounded to the nearest FP4 E2M1 value
  {0, 0.5, 1, 1.5, 2, 3, 4, 6} (ties to the even encoding, saturating at 6),
  with the sign of the quotient in bit 3 (as an IEEE conversion keeps it,
  so a negative zero, and a negative quotient that rounds to zero, encode
  as -0).  Rotation as
  above; Y = sum_blocks 2^(e_x + e_w) sum_k fp4_x fp4_w, exact in float64,
  rounded once to float32, + the low-rank term.
* W4A8 layers: the layers a phase-aware policy keeps at 8-bit activations
  while the weights stay 4-bit (DynamicPTQ page, "Metodología" §2).  The
  same rotation and the same per-token symmetric absmax rule with qmax 127:
  s = a / 127, q = clamp(rint(x / s), -127, 127).

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

from functools import lru_cache
from typing import Optional

import numpy as np

QMAX = 7


# ----------------------------------------------------------------------------
# Rotation (OffQ page, "Metodología", steps 2-3)
# ----------------------------------------------------------------------------
@lru_cache(maxsize=16)
def _hadamard_cached(b: int) -> np.ndarray:
    return _hadamard_build(b)


def hadamard_matrix(b: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order b: H[i, j] = (-1)^popcount(i & j).

    Row 0 and column 0 are all ones (the property OffQ's offsetting uses).
    """
    return _hadamard_cached(int(b)).copy()


def _hadamard_build(b: int) -> np.ndarray:
    if b < 1 or (b & (b - 1)) != 0:
        raise ValueError("Hadamard order must be a power of two")
    i = np.arange(b, dtype=np.int64)
    and_ = i[:, None] & i[None, :]
    parity = np.zeros_like(and_)
    v = and_.copy()
    while np.any(v):
        parity ^= v & 1
        v >>= 1
    return np.where(parity == 0, 1.0, -1.0)


def rotate64(x: np.ndarray, b: int) -> np.ndarray:
    """Block rotation in float64: every contiguous block of b channels of
    every row becomes block @ H_b / sqrt(b).  No rounding to float32."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if K % b != 0:
        raise ValueError("block size must divide K")
    H = _hadamard_cached(int(b))
    blocks = x.reshape(M * (K // b), b)
    return (blocks @ H / np.sqrt(b)).reshape(M, K)


def rotate(x: np.ndarray, b: int) -> np.ndarray:
    """The oracle's rotated activations: rotate64 rounded once to float32."""
    return rotate64(x, b).astype(np.float32)


# ----------------------------------------------------------------------------
# Quantization (SERQ page, "Resumen técnico" §1-2)
# ----------------------------------------------------------------------------
def quantize_act(xrot32: np.ndarray, qmax: int = QMAX):
    """Per-token symmetric quantization of already-rotated float32
    activations: int4 (qmax 7) or, for W4A8 layers, int8 (qmax 127).

    Returns (codes int8 [M,K] in [-qmax,qmax], scales float32 [M])."""
    xrot32 = np.asarray(xrot32, dtype=np.float32)
    s = _row_scales(xrot32, qmax)
    return _codes_rows(xrot32, s, qmax), s


def _row_scales(v32: np.ndarray, qmax: int = QMAX) -> np.ndarray:
    """absmax / qmax in float32 for every row of a 2-D float32 array."""
    if v32.shape[1] == 0:
        return np.zeros(v32.shape[0], np.float32)
    a = np.max(np.abs(v32), axis=1).astype(np.float32)
    return (a / np.float32(qmax)).astype(np.float32)


def _codes_rows(v32: np.ndarray, s32: np.ndarray, qmax: int = QMAX) -> np.ndarray:
    """q = clamp(rint(v / s), -qmax, qmax) for every row with its own float32
    scale: the quotient rounded to float32 (IEEE division), rint rounding half
    to even.  A zero scale gives all-zero codes."""
    s32 = np.asarray(s32, np.float32)
    safe = np.where(s32 == 0, np.float32(1), s32).astype(np.float32)
    quot = (v32 / safe[:, None]).astype(np.float32)
    q = np.clip(np.rint(quot), -qmax, qmax).astype(np.int8)
    q[s32 == 0, :] = 0
    return q


def quantize_weight(wrot32: np.ndarray, group: int, scale_dtype: str):
    """Symmetric round-to-nearest int4 of rotated weights, one scale per
    output channel (group == 0) or per group of ``group`` channels along K.

    The scale is rounded to ``scale_dtype`` first and the codes are taken
    against that stored value.  Returns (codes int8 [N,K], scales [N] or
    [N, K/group] in scale_dtype)."""
    wrot32 = np.asarray(wrot32, dtype=np.float32)
    N, K = wrot32.shape
    g = K if group == 0 else group
    if K % g != 0:
        raise ValueError("group must divide K")
    G = K // g
    segs = wrot32.reshape(N * G, g)
    stored = _row_scales(segs).astype(np.dtype(scale_dtype))
    q = _codes_rows(segs, stored.astype(np.float32)).reshape(N, K)
    s = stored.reshape(N, G)
    if group == 0:
        s = s[:, 0]
    return q, s


# ----------------------------------------------------------------------------
# Packing
# ----------------------------------------------------------------------------
def pack_int4(q: np.ndarray) -> np.ndarray:
    """byte[.., j] = (q[.., 2j] & 0xF) | (q[.., 2j+1] & 0xF) << 4."""
    q = np.asarray(q).astype(np.int16)
    if q.shape[-1] % 2 != 0:
        raise ValueError("even number of codes required")
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: nibbles read as two's-complement 4-bit values."""
    p = np.asarray(p, dtype=np.uint8).astype(np.int16)
    lo = p & 0xF
    hi = p >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ----------------------------------------------------------------------------
# Integer GEMM, low-rank term, epilogue (SERQ page, "Resumen técnico" §2-3)
# ----------------------------------------------------------------------------
def int_gemm(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qx[m, k] * qw[n, k], exact, as int64."""
    a = np.asarray(qx, dtype=np.float64)
    w = np.asarray(qw, dtype=np.float64)
    return (a @ w.T).astype(np.int64)


def int_gemm_groups(qx: np.ndarray, qw: np.ndarray, group: int) -> np.ndarray:
    """One exact int64 partial per K-group: [G, M, N]."""
    K = qx.shape[1]
    G = K // group
    return np.stack([int_gemm(qx[:, j * group:(j + 1) * group],
                              qw[:, j * group:(j + 1) * group]) for j in range(G)])


def lowrank(x: np.ndarray, A: Optional[np.ndarray], B: Optional[np.ndarray]) -> np.ndarray:
    """(X @ A) @ B in float64 on the values exactly as given; 0 without A."""
    if A is None or B is None:
        return None
    t = np.asarray(x, np.float64) @ np.asarray(A, np.float64)
    return t @ np.asarray(B, np.float64)


def epilogue(acc_or_groups: np.ndarray, s_x: np.ndarray, s_w: np.ndarray,
             lr: Optional[np.ndarray]) -> np.ndarray:
    """Y = s_x[m] * s_w[n] * acc[m, n] (+ lr), float64, rounded once to float32.

    With per-group weight scales, acc_or_groups is [G, M, N] and
    Y = sum_j s_x[m] * s_w[n, j] * acc_j[m, n]."""
    sx = np.asarray(s_x, np.float64)
    sw = np.asarray(s_w, np.float64)
    if sw.ndim == 1:
        y = sx[:, None] * sw[None, :] * np.asarray(acc_or_groups, np.float64)
    else:
        acc = np.asarray(acc_or_groups, np.float64)
        y = np.zeros(acc.shape[1:])
        for j in range(acc.shape[0]):
            y += sx[:, None] * sw[None, :, j] * acc[j]
    if lr is not None:
        y = y + lr
    return y.astype(np.float32)


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------
def prepare_weight(W: np.ndarray, had_block: int, group: int, scale_dtype: str):
    """Offline weight preparation: rotate, quantize, pack.

    Returns (packed uint8 [N, K/2], scales, codes int8 [N, K])."""
    wrot = rotate(W, had_block) if had_block > 1 else np.asarray(W, np.float32)
    q, s = quantize_weight(wrot, group, scale_dtype)
    return pack_int4(q), s, q


def quantize_activation(X: np.ndarray, had_block: int, qmax: int = QMAX):
    """Rotate (had_block > 1) and quantize per token.

    Returns (packed uint8 [M, K/2] (None for 8-bit codes), scales float32
    [M], codes, rotated fp32)."""
    xrot = rotate(X, had_block) if had_block > 1 else np.asarray(X, np.float32)
    q, s = quantize_act(xrot, qmax)
    return (pack_int4(q) if qmax <= 7 else None), s, q, xrot


def qlinear_forward(X: np.ndarray, wq_packed: np.ndarray, w_scale: np.ndarray,
                    had_block: int, group: int, A=None, B=None, act_bits: int = 4) -> np.ndarray:
    """The quantized forward Y [M, N] float32; act_bits 8 is the W4A8 layer."""
    qmax = QMAX if act_bits == 4 else 127
    _, s_x, qx, _ = quantize_activation(X, had_block, qmax)
    qw = unpack_int4(wq_packed)
    if group == 0:
        acc = int_gemm(qx, qw)
    else:
        acc = int_gemm_groups(qx, qw, group)
    return epilogue(acc, s_x, np.asarray(w_scale).astype(np.float32),
                    lowrank(X, A, B))


def qlinear_from_codes(qx: np.ndarray, s_x: np.ndarray, wq_packed: np.ndarray,
                       w_scale: np.ndarray, group: int, X=None, A=None, B=None) -> np.ndarray:
    """Epilogue of the layer evaluated on given activation codes and scales
    (used to judge a GPU result on the GPU's own codes)."""
    qw = unpack_int4(wq_packed)
    acc = int_gemm(qx, qw) if group == 0 else int_gemm_groups(qx, qw, group)
    lr = lowrank(X, A, B) if X is not None else None
    return epilogue(acc, s_x, np.asarray(w_scale).astype(np.float32), lr)


# ----------------------------------------------------------------------------
# Asymmetric group-wise activations (OffQ page, "Metodología" steps 2-3)
# ----------------------------------------------------------------------------
AQMAX = 15


def quantize_act_asym(xrot32: np.ndarray, group: int):
    """Asymmetric uint4 quantization of rotated float32 activations, one
    (scale, zero point) per token and group of `group` channels.

    Returns (codes uint8 [M, K] in [0, 15], scales float32 [M, K/group],
    zero points int64 [M, K/group], not clamped)."""
    x = np.asarray(xrot32, dtype=np.float32)
    M, K = x.shape
    G = K // group
    xg = x.reshape(M, G, group)
    lo = xg.min(axis=2).astype(np.float32)
    hi = xg.max(axis=2).astype(np.float32)
    flat = hi == lo
    lo = np.where(flat, np.minimum(lo, np.float32(0)), lo).astype(np.float32)
    hi = np.where(flat, np.maximum(hi, np.float32(0)), hi).astype(np.float32)
    s = ((hi - lo).astype(np.float32) / np.float32(AQMAX)).astype(np.float32)
    live = s > 0
    safe = np.where(live, s, np.float32(1)).astype(np.float32)
    z = np.rint((-lo / safe).astype(np.float32)).astype(np.int64)
    quot = (xg / safe[:, :, None]).astype(np.float32)
    q = np.clip(np.rint(quot).astype(np.int64) + z[:, :, None], 0, AQMAX)
    q[~live, :] = 0
    z[~live] = 0
    return q.reshape(M, K).astype(np.uint8), s, z


def weight_group_sums(qw: np.ndarray, group: int) -> np.ndarray:
    """sum_{k in g} qw[n, k] for every output channel and K-group: [N, K/group]."""
    N, K = qw.shape
    return qw.astype(np.int64).reshape(N, K // group, group).sum(axis=2)


def asym_from_codes(qx: np.ndarray, s_x: np.ndarray, z_x: np.ndarray, qw: np.ndarray,
                    s_w: np.ndarray, group: int, X=None, A=None, B=None) -> np.ndarray:
    """Y = sum_g s_x s_w (acc_g - z_x[m,g] wsum[n,g]) + low-rank, float64 then
    rounded once to float32; qw are the signed weight codes [N, K]."""
    acc = int_gemm_groups(qx.astype(np.int64), qw, group)          # [G, M, N]
    ws = weight_group_sums(qw, group)                              # [N, G]
    corr = acc - np.asarray(z_x, np.int64).T[:, :, None] * ws.T[:, None, :]
    y = np.einsum("gmn,mg->mn", corr.astype(np.float64), np.asarray(s_x, np.float64))
    y = y * np.asarray(s_w, np.float64).reshape(1, -1)
    lr = lowrank(X, A, B) if X is not None else None
    if lr is not None:
        y = y + lr
    return y.astype(np.float32)


def qlinear_forward_asym(X: np.ndarray, wq_packed: np.ndarray, w_scale: np.ndarray,
                         had_block: int, A=None, B=None) -> np.ndarray:
    """The forward with asymmetric group-wise activations, the group being the
    Hadamard block; per-channel weight scales."""
    xrot = rotate(X, had_block)
    q, s, z = quantize_act_asym(xrot, had_block)
    qw = unpack_int4(wq_packed)
    return asym_from_codes(q, s, z, qw, np.asarray(w_scale).astype(np.float32), had_block, X, A, B)



# ----------------------------------------------------------------------------
# In-GEMM residual of salient channels (SERQ page, "Metodología" items 2-3)
# ----------------------------------------------------------------------------
RES_STEPS = 8   # residual step = weight scale / RES_STEPS


def quantize_weight_residual(wrot32: np.ndarray, r: int, scale_dtype: str):
    """Per-channel RTN int4 weights (quantize_weight with group 0) plus the
    4-bit residual of the first r channels, taken against the stored scale:
    e = RN(x~ - RN(s q)), q_r = clamp(rint(RN(e / RN(s / 8))), -8, 7).

    Returns (codes int8 [N, K], scales [N] in scale_dtype, residual codes
    int8 [N, r])."""
    wrot32 = np.asarray(wrot32, dtype=np.float32)
    q, s = quantize_weight(wrot32, 0, scale_dtype)
    s32 = np.asarray(s).astype(np.float32)
    recon = (s32[:, None] * q[:, :r].astype(np.float32)).astype(np.float32)
    e = (wrot32[:, :r] - recon).astype(np.float32)
    t = (s32 / np.float32(RES_STEPS)).astype(np.float32)
    live = t > 0
    safe = np.where(live, t, np.float32(1)).astype(np.float32)
    qr = np.clip(np.rint((e / safe[:, None]).astype(np.float32)), -8, 7)
    qr[~live, :] = 0
    return q, s, qr.astype(np.int8)


def prepare_weight_residual(W: np.ndarray, had_block: int, r: int, scale_dtype: str):
    """Offline preparation with the residual: rotate, quantize, pack.

    Returns (packed uint8 [N, K/2], scales [N], codes int8 [N, K], residual
    codes int8 [N, r])."""
    wrot = rotate(W, had_block) if had_block > 1 else np.asarray(W, np.float32)
    q, s, qr = quantize_weight_residual(wrot, r, scale_dtype)
    return pack_int4(q), s, q, qr


def residual_int_gemm(qx: np.ndarray, qw: np.ndarray, qr: np.ndarray) -> np.ndarray:
    """The one integer of the residual product, exact int64:
    8 sum_k qx qw + sum_{k<r} qx qr."""
    r = qr.shape[1]
    return RES_STEPS * int_gemm(qx, qw) + int_gemm(qx[:, :r], qr)


def residual_from_codes(qx: np.ndarray, s_x: np.ndarray, qw: np.ndarray, s_w: np.ndarray,
                        qr: np.ndarray) -> np.ndarray:
    """Y = s_x s_w (sum_k qx qw + (1/8) sum_{k<r} qx qr), float64 then rounded
    once to float32."""
    acc = residual_int_gemm(qx, qw, qr).astype(np.float64)
    y = np.asarray(s_x, np.float64)[:, None] * np.asarray(s_w, np.float64)[None, :] * acc
    return (y / RES_STEPS).astype(np.float32)


def qlinear_forward_residual(X: np.ndarray, wq_packed: np.ndarray, w_scale: np.ndarray,
                             qr: np.ndarray, had_block: int) -> np.ndarray:
    """The forward with the in-GEMM residual of the first r channels."""
    _, s_x, qx, _ = quantize_activation(X, had_block)
    qw = unpack_int4(wq_packed)
    return residual_from_codes(qx, s_x, qw, np.asarray(w_scale).astype(np.float32), qr)


# ----------------------------------------------------------------------------
# MXFP4 (SERQ page, "Metodología" item 2; the OCP microscaling format)
# ----------------------------------------------------------------------------
MX_BLOCK = 32
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_code(p: np.ndarray) -> np.ndarray:
    """FP4 E2M1 encoding of float values p: magnitude bits from the nearest
    of E2M1 (ties to the even encoding, |p| > 6 saturates to 6), sign bit 8
    from the sign of p (negative zero included)."""
    p = np.asarray(p, dtype=np.float64)
    a = np.abs(p)
    # upper bounds of each magnitude code; '<=' where the tie goes down
    # (to the even code), '<' where it goes up
    mag = np.full(p.shape, 7, dtype=np.int16)
    for code, bound, inclusive in ((6, 5.0, True), (5, 3.5, False), (4, 2.5, True),
                                   (3, 1.75, False), (2, 1.25, True), (1, 0.75, False),
                                   (0, 0.25, True)):
        hit = (a <= bound) if inclusive else (a < bound)
        mag = np.where(hit, code, mag)
    return (mag | np.where(np.signbit(p), 8, 0)).astype(np.uint8)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    """Value of FP4 E2M1 codes (0..15)."""
    c = np.asarray(code).astype(np.int64)
    v = E2M1[c & 7]
    return np.where(c & 8, -v, v)


def mx_block_exponent(amax: np.ndarray) -> np.ndarray:
    """e = max(floor(log2(amax)) - 2, -127), with -127 for amax = 0."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.full(amax.shape, -127, dtype=np.int64)
    pos = amax > 0
    e[pos] = np.maximum(np.floor(np.log2(amax[pos])).astype(np.int64) - 2, -127)
    return e


def quantize_mxfp4(v32: np.ndarray):
    """MXFP4 of float32 rows [R, K] (K a multiple of 32).

    Returns (codes uint8 [R, K] in 0..15, block exponents int [R, K/32]);
    the E8M0 byte of a block is exponent + 127."""
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    R, K = v.shape
    blocks = v.reshape(R, K // MX_BLOCK, MX_BLOCK)
    e = mx_block_exponent(np.abs(blocks).max(axis=2))
    p = blocks / np.exp2(e)[:, :, None]           # exact: a power-of-two scaling
    return e2m1_code(p).reshape(R, K), e


def mxfp4_values(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    """Dequantized values fp4(code) 2^e, float64 [R, K]."""
    R, K = codes.shape
    v = e2m1_value(codes).reshape(R, K // MX_BLOCK, MX_BLOCK) * np.exp2(e)[:, :, None]
    return v.reshape(R, K)


def mxfp4_gemm(cx: np.ndarray, ex: np.ndarray, cw: np.ndarray, ew: np.ndarray) -> np.ndarray:
    """sum_blocks 2^(ex + ew) sum_k fp4_x fp4_w as float64 [M, N] (exact:
    every product of two E2M1 values is a multiple of 1/4 and the partial
    sums stay far below 2^53 times the smallest scale)."""
    return mxfp4_values(cx, ex) @ mxfp4_values(cw, ew).T


def qlinear_forward_mxfp4(X: np.ndarray, W: np.ndarray, had_block: int, A=None, B=None) -> np.ndarray:
    """The MXFP4 layer: rotate X and W, quantize both to MXFP4, multiply,
    add the low-rank term; float64 then rounded once to float32."""
    xr = rotate(X, had_block) if had_block > 1 else np.asarray(X, np.float32)
    wr = rotate(W, had_block) if had_block > 1 else np.asarray(W, np.float32)
    cx, ex = quantize_mxfp4(xr)
    cw, ew = quantize_mxfp4(wr)
    y = mxfp4_gemm(cx, ex, cw, ew)
    lr = lowrank(X, A, B)
    if lr is not None:
        y = y + lr
    return y.astype(np.float32)
