"""Pins of the oracle's int4 quantizers and nibble packing.

Per-token symmetric int4 activations and per-channel / per-group symmetric
RTN int4 weights (SERQ page, "Resumen técnico" §1-2; DynamicPTQ page,
"Resultados", RTN).  The rounding rule, the range [-7, 7] and the nibble order
are readings of the pages, which state none of them.
"""
import numpy as np
import pytest

from oracle import w4a4_oracle as O


def test_ties_round_to_even():
    # absmax 7 gives s = 1 exactly, so x / s = x and the ties are exact.
    x = np.array([[7, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 4.5, -6.5]], np.float32)
    q, s = O.quantize_act(x)
    assert s[0] == np.float32(1.0)
    assert q[0].tolist() == [7, 0, 2, 2, 0, -2, -2, 4, 4, -6]


def test_absmax_maps_to_seven_with_sign():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 64)).astype(np.float32)
    q, s = O.quantize_act(x)
    for m in range(50):
        i = np.argmax(np.abs(x[m]))
        assert q[m, i] == (7 if x[m, i] > 0 else -7)
        assert np.all(np.abs(q[m]) <= 7)


def test_error_at_most_half_step():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((40, 256)) * rng.uniform(0.01, 100, (40, 1))).astype(np.float32)
    q, s = O.quantize_act(x)
    err = np.abs(x.astype(np.float64) - s[:, None].astype(np.float64) * q)
    assert np.all(err <= s[:, None] * (0.5 + 1e-6))


def test_codes_match_brute_force_nearest():
    # Brute force: the code is the integer in [-7, 7] nearest to the float32
    # quotient, ties to the even one.
    rng = np.random.default_rng(2)
    x = rng.uniform(-3, 3, (1, 2000)).astype(np.float32)
    x[0, 0] = 3.0
    q, s = O.quantize_act(x)
    quot = (x[0] / s[0]).astype(np.float32).astype(np.float64)
    cand = np.arange(-7, 8)
    for i in range(x.shape[1]):
        d = np.abs(quot[i] - cand)
        best = cand[d == d.min()]
        want = best[0] if best.size == 1 else best[best % 2 == 0][0]
        assert q[0, i] == want


def test_power_of_two_scaling_invariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    q, s = O.quantize_act(x)
    for e in (-20, -3, 5, 30):
        q2, s2 = O.quantize_act((x * np.float32(2.0 ** e)).astype(np.float32))
        assert np.array_equal(q, q2)
        assert np.array_equal(s2, (s * np.float32(2.0 ** e)).astype(np.float32))


def test_zero_row_and_underflowing_scale():
    x = np.zeros((3, 16), np.float32)
    x[1, 3] = np.float32(1e-45)          # smallest denormal: a / 7 rounds to 0
    x[2, 5] = np.float32(-2.0)
    q, s = O.quantize_act(x)
    assert s[0] == 0 and s[1] == 0
    assert np.all(q[0] == 0) and np.all(q[1] == 0)
    assert q[2, 5] == -7 and s[2] == np.float32(np.float32(2.0) / np.float32(7))


def test_scale_is_float32_division():
    x = np.array([[3.0, -1.0]], np.float32)
    _, s = O.quantize_act(x)
    assert s.dtype == np.float32
    assert s[0] == np.float32(np.float32(3.0) / np.float32(7.0))


@pytest.mark.parametrize("scale_dtype", ["float16", "float32"])
def test_weight_codes_taken_against_stored_scale(scale_dtype):
    rng = np.random.default_rng(4)
    w = (0.02 * rng.standard_normal((16, 256))).astype(np.float32)
    q, s = O.quantize_weight(w, 0, scale_dtype)
    assert s.dtype == np.dtype(scale_dtype) and s.shape == (16,)
    for n in range(16):
        a = np.float32(np.max(np.abs(w[n])))
        stored = np.float32(a / np.float32(7)).astype(np.dtype(scale_dtype))
        assert s[n] == stored
        quot = (w[n] / np.float32(stored)).astype(np.float32)
        assert np.array_equal(q[n], np.clip(np.rint(quot), -7, 7).astype(np.int8))


@pytest.mark.parametrize("scale_dtype", ["float16", "float32"])
def test_clamp_only_acts_on_subnormal_float16_scales(scale_dtype):
    # With s = RN(max|x| / 7) stored in float32 or as a normal float16, every
    # quotient x / s rounds into [-7, 7] without the clamp; only a float16
    # scale below 2^-14 can leave a quotient at or past 7.5.
    rng = np.random.default_rng(21)
    n = 400
    w = rng.standard_normal((n, 64)) * rng.uniform(0.5, 2.0, (n, 1))
    w = (w * 2.0 ** rng.integers(-40, 12, (n, 1))).astype(np.float32)
    q, s = O.quantize_weight(w, 0, scale_dtype)
    s32 = s.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        raw = np.rint((w / s32[:, None]).astype(np.float32))
    normal = s32 >= np.float32(2.0 ** -14) if scale_dtype == "float16" else s32 > 0
    assert np.count_nonzero(normal) > 100
    assert np.all(np.abs(raw[normal]) <= 7)
    assert np.array_equal(q[normal], raw[normal].astype(np.int8))
    if scale_dtype == "float16":
        sub = (s32 > 0) & ~normal
        assert np.any(np.abs(raw[sub]) > 7)  # the clamp does decide codes there


def test_weight_groups_equal_per_segment_quantization():
    rng = np.random.default_rng(5)
    w = (0.02 * rng.standard_normal((6, 512))).astype(np.float32)
    w[:, 130] *= 50
    q, s = O.quantize_weight(w, 128, "float16")
    assert s.shape == (6, 4)
    for j in range(4):
        qj, sj = O.quantize_weight(w[:, j * 128:(j + 1) * 128], 0, "float16")
        assert np.array_equal(q[:, j * 128:(j + 1) * 128], qj)
        assert np.array_equal(s[:, j], sj)
    # the outlier only coarsens its own group
    q_all, _ = O.quantize_weight(w, 0, "float16")
    assert np.count_nonzero(q[:, 256:]) > np.count_nonzero(q_all[:, 256:])


def test_pack_unpack_exhaustive_bytes():
    every = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(O.pack_int4(O.unpack_int4(every)), every)


def test_pack_unpack_exhaustive_code_pairs():
    a, b = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8), indexing="ij")
    codes = np.stack([a.ravel(), b.ravel()], axis=1).astype(np.int8)  # [256, 2]
    p = O.pack_int4(codes)
    assert p.shape == (256, 1)
    assert np.array_equal(O.unpack_int4(p), codes)


def test_nibble_order_examples():
    assert O.pack_int4(np.array([[1, -1]], np.int8)).tolist() == [[0xF1]]
    assert O.pack_int4(np.array([[-8, 7]], np.int8)).tolist() == [[0x78]]
    assert O.pack_int4(np.array([[7, -7, 0, -3]], np.int8)).tolist() == [[0x97, 0xD0]]


def test_division_not_reciprocal_multiply():
    # Near the half-integer boundaries, x / s and x * (1 / s) can round to
    # different float32 quotients and so to different codes.  The reading is
    # IEEE division; find such inputs and check the oracle follows division.
    f = np.float32
    cases = []
    for a in (3.0, 1.0, 0.3):
        s = f(f(a) / f(7))
        r = f(f(1) / s)
        for n in range(7):
            xv = f((n + 0.5) * float(s))
            for _ in range(8):
                xv = np.nextafter(xv, f(np.inf), dtype=np.float32)
                if np.rint(f(xv / s)) != np.rint(f(xv * r)):
                    cases.append((a, xv, int(np.rint(f(xv / s)))))
    assert len(cases) >= 3
    for a, xv, want in cases:
        q, s = O.quantize_act(np.array([[a, xv]], np.float32))
        assert q[0, 1] == want
