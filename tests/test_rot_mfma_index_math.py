"""CPU check of the index math of the rotation on the matrix instruction
(rotq_mfma.hip), against definitions that do not come from the kernel: the
Sylvester Hadamard matrices of scipy, the lane layouts of
v_mfma_f32_16x16x32_f16 (A: lane 16 g + r holds A[r][8 g + t]; B: lane
16 g + c holds B[8 g + t][c]; D: lane 16 g + c holds D[4 g + i][c]), the
lane exchanges of v_permlane32_swap (lanes 32-63 of the first operand
trade places with lanes 0-31 of the second) and v_permlane16_swap (the odd
16-lane rows of the first operand with the even rows of the second), and the
data-parallel lane moves within a 16-lane row (quad permutation, half-row
mirror, rotation by 8).

The GPU tests check the kernels' codes against the oracle; these tests pin
the fragment signs, the load addresses, the output positions, the 4 x 4 unit
transpose into the tile order, and for b = 128 n the load permutation and the
signs of the stages across sub-blocks, on the host, so a slip in any of them
shows up without a GPU.
"""
import numpy as np
import scipy.linalg

H = scipy.linalg.hadamard(128).astype(np.float64)  # Sylvester order, H[i][k] = +-1
LANES = np.arange(64)
G, R = LANES >> 4, LANES & 15


def a_fragment(mb, kc):
    """The +-1 operand A of output block mb, K step kc, as the kernel builds
    it: a per-lane part (r & t, r3 & g0), a lane-group sign for odd mb (g1),
    and a sign fixed per (mb, kc)."""
    t = np.arange(8)
    par = (np.array([[bin(r & tt & 7).count("1") for tt in t] for r in R]) + ((R >> 3) & G & 1)[:, None]) & 1
    f0 = np.where(par == 1, -1.0, 1.0)
    f1 = np.where(((G >> 1) & 1)[:, None] == 1, -f0, f0)
    neg = ((mb >> 1) & kc & 1) ^ ((mb >> 2) & (kc >> 1) & 1)
    f = f1 if mb & 1 else f0
    return -f if neg else f          # [lane, t]


def test_a_fragments_are_the_hadamard_blocks():
    for mb in range(8):
        for kc in range(4):
            frag = a_fragment(mb, kc)
            A = np.zeros((16, 32))
            for lane in range(64):
                A[R[lane], 8 * G[lane]:8 * G[lane] + 8] = frag[lane]
            assert np.array_equal(A, H[16 * mb:16 * mb + 16, 32 * kc:32 * kc + 32]), (mb, kc)


def test_product_gives_each_block_transform_in_the_output_fragment():
    rng = np.random.default_rng(0)
    seg = rng.standard_normal(2048)          # one wave: 16 blocks of 128
    acc = np.zeros((8, 64, 4))
    for kc in range(4):
        # operand B of step kc: lane 16 g + c loads seg[128 c + 32 kc + 8 g, +8)
        Bf = np.stack([seg[128 * (l & 15) + 32 * kc + 8 * (l >> 4) + np.arange(8)] for l in LANES])
        B = np.zeros((32, 16))
        for lane in range(64):
            B[8 * G[lane]:8 * G[lane] + 8, R[lane]] = Bf[lane]
        for mb in range(8):
            frag = a_fragment(mb, kc)
            A = np.zeros((16, 32))
            for lane in range(64):
                A[R[lane], 8 * G[lane]:8 * G[lane] + 8] = frag[lane]
            D = A @ B
            for lane in range(64):
                acc[mb, lane] += D[4 * G[lane]:4 * G[lane] + 4, R[lane]]
    y = (H @ seg.reshape(16, 128).T).T        # y[c] = H x_c
    for lane in range(64):
        g, c = lane >> 4, lane & 15
        for mb in range(8):
            assert np.allclose(acc[mb, lane], y[c, 16 * mb + 4 * g:16 * mb + 4 * g + 4])


def swap32(a, b):
    a, b = a.copy(), b.copy()
    a[32:], b[:32] = b[:32].copy(), a[32:].copy()
    return a, b


def swap16(a, b):
    a, b = a.copy(), b.copy()
    for row in (1, 3):                        # odd rows of a <-> even rows of b
        sa, sb = slice(16 * row, 16 * row + 16), slice(16 * (row - 1), 16 * row)
        a[sa], b[sb] = b[sb].copy(), a[sa].copy()
    return a, b


def test_unit_transpose_puts_32_consecutive_codes_in_tile_order():
    # Lane 16 g + c holds element 16 mb + 4 g + i of block c (value id below);
    # after the exchanges lane 16 g' + c must hold elements [32 g', 32 g' + 32)
    # of block c with chunk offset 16 (v / 4) + 4 s + v % 4 in B[s][v].
    val = np.zeros((8, 4, 64), np.int64)      # [mb][i][lane] -> element id 128 c + e
    for lane in range(64):
        g, c = lane >> 4, lane & 15
        for mb in range(8):
            for i in range(4):
                val[mb, i, lane] = 128 * c + 16 * mb + 4 * g + i
    u = np.array([[val[2 * j + (v >> 2), v & 3] for v in range(8)] for j in range(4)])  # [j][v][lane]
    b = np.zeros_like(u)
    for v in range(8):
        s02 = swap32(u[0, v], u[2, v])
        s13 = swap32(u[1, v], u[3, v])
        t01 = swap16(s02[0], s13[0])
        t23 = swap16(s02[1], s13[1])
        b[0, v], b[1, v], b[2, v], b[3, v] = t01[0], t01[1], t23[0], t23[1]
    for lane in range(64):
        g, c = lane >> 4, lane & 15
        chunk = np.zeros(32, np.int64)
        for s in range(4):
            for v in range(8):
                chunk[16 * (v >> 2) + 4 * s + (v & 3)] = b[s, v, lane]
        assert np.array_equal(chunk, 128 * c + 32 * g + np.arange(32)), lane
        # packed nibbles: nibble 8 d + e of the lane's 16 bytes is chunk offset 8 d + e
        nib = [b[2 * (d & 1) + (e >> 2), 4 * (d >> 1) + (e & 3), lane] for d in range(4) for e in range(8)]
        assert np.array_equal(nib, 128 * c + 32 * g + np.arange(32)), lane


# --------------------------------------------------------------------------
# b = 128 n (n = 2^P sub-blocks of 128): the stages across sub-blocks
# --------------------------------------------------------------------------
MASKS = [1, 2, 7, 8]          # xor partners of the lane stages within a 16-lane row


def _par(v):
    return bin(v).count("1") & 1


def kron_tables(stages):
    """Load permutation pi, per-stage signs (coordinates) and final signs of
    the lane stages, derived from the masks as the kernel's host code does:
    coordinates over the basis {masks}, and pi(k) the j with
    (-1)^(a(i).a(k)) = (-1)^(i.j) for every i."""
    n = 1 << stages
    coord = {}
    for a in range(n):
        i = 0
        for s in range(stages):
            if a >> s & 1:
                i ^= MASKS[s]
        coord[i] = a
    assert sorted(coord) == list(range(n))
    pi, sel, sig = [], [], []
    for c in range(16):
        lo, hi = c & (n - 1), c & ~(n - 1)
        js = [j for j in range(n) if all(_par(coord[i] & coord[lo]) == _par(i & j) for i in range(n))]
        assert len(js) == 1
        pi.append(hi | js[0])
        sel.append(coord[lo])
        sig.append(_par(coord[lo]))
    return pi, sel, sig


def dpp_partner(ctrl, lane):
    """Source lane of a data-parallel move within a 16-lane row."""
    row, c = lane & ~15, lane & 15
    if ctrl == "quad_perm:[1,0,3,2]":
        return row + (c & ~3) + [1, 0, 3, 2][c & 3]
    if ctrl == "quad_perm:[2,3,0,1]":
        return row + (c & ~3) + [2, 3, 0, 1][c & 3]
    if ctrl == "row_half_mirror":
        return row + (c & 8) + 7 - (c & 7)
    if ctrl == "row_ror:8":
        return row + ((c + 8) & 15)
    raise ValueError(ctrl)


STAGE_CTRL = ["quad_perm:[1,0,3,2]", "quad_perm:[2,3,0,1]", "row_half_mirror", "row_ror:8"]


def test_dpp_controls_are_the_masks():
    for s, ctrl in enumerate(STAGE_CTRL):
        for lane in range(64):
            assert dpp_partner(ctrl, lane) == lane ^ MASKS[s]


def test_kron_stages_give_the_sylvester_transform():
    # One wave: 4096 elements as two chains of 16 sub-blocks of 128, lane
    # column c of chain h holding sub-block 16 h + pi(c) after the 128-point
    # transform.  Lane stages v += sgn * v[partner] (sgn = -1 where the
    # column's coordinate s is 1), the register stage across chains for
    # n = 32, then the final sign; the result must be H_b on every block of b.
    rng = np.random.default_rng(11)
    x = rng.standard_normal(4096)
    for P in range(1, 6):
        b = 128 << P
        stages = min(P, 4)
        pi, sel, sig = kron_tables(stages)
        lanes = np.arange(64)
        c_of = lanes & 15
        # v[h][lane][e]: lane 16 g + c holds the column's 128 outputs (all e
        # here; the kernel spreads e over g, mb, i, which the stages ignore)
        v = np.zeros((2, 64, 128))
        for h in range(2):
            for lane in lanes:
                v[h, lane] = H @ x[128 * (16 * h + pi[c_of[lane]]):][:128]
        if P == 5:
            v = np.stack([v[0] + v[1], v[0] - v[1]])
        for s in range(stages):
            sg = np.array([-1.0 if sel[c] >> s & 1 else 1.0 for c in c_of])
            src = np.array([dpp_partner(STAGE_CTRL[s], lane) for lane in lanes])
            v = v + v[:, src, :] * sg[None, :, None]
        fin = np.array([-1.0 if sig[c] else 1.0 for c in c_of])
        z = v * fin[None, :, None]
        Hb = scipy.linalg.hadamard(b).astype(np.float64)
        ref = np.concatenate([Hb @ x[k:k + b] for k in range(0, 4096, b)]).reshape(2, 16, 128)
        for h in range(2):
            for lane in lanes:
                assert np.allclose(z[h, lane], ref[h, c_of[lane]]), (P, h, lane)


def test_kron_signed_quotient_equals_unsigned():
    # A lane holds its values times sgn; with the divisor and its reciprocal
    # times sgn, each step (product, two fma refinements) sees the negated
    # operands of the unsigned computation in the places where rounding, which
    # is odd (RN(-x) = -RN(x)), gives the same float.  Here the fma is the
    # float64 sum of the exact float64 product rounded to float32, an odd
    # rounding too; a sign in the wrong place (say on rc only) fails.
    rng = np.random.default_rng(3)
    f = np.float32

    def fma(a, b, c):
        return f(np.float64(a) * np.float64(b) + np.float64(c))

    def quot(xt, sd, rc):
        q = f(xt * rc)
        q = fma(fma(-q, sd, xt), rc, q)
        return fma(fma(-q, sd, xt), rc, q)

    for _ in range(2000):
        s = f(rng.uniform(1e-3, 10.0))
        z = f(rng.uniform(-7.5, 7.5) * s)
        rc = f(f(1.0) / s)
        assert quot(z, s, rc) == quot(f(-z), f(-s), f(-rc))
        assert quot(z, s, rc) != quot(f(-z), s, f(-rc)) or quot(z, s, rc) == 0


def test_wave_reduction_pattern_reaches_every_lane():
    # The kernel's 64-lane reductions: lane ^ 1, lane ^ 2 (quad permutations),
    # the half-row mirror and the row mirror within each 16-lane row, then the
    # 32- and 16-lane swaps of the value with itself.  Every lane must end
    # with the maximum (and the sum) of all 64.
    def half_mirror(lane):
        return (lane & ~7) + 7 - (lane & 7)

    def mirror(lane):
        return (lane & ~15) + 15 - (lane & 15)

    rng = np.random.default_rng(9)
    for op, ident in ((np.maximum, None), (np.add, None)):
        v = rng.integers(-1000, 1000, 64).astype(np.int64)
        want = op.reduce(v)
        for part in (lambda l: l ^ 1, lambda l: l ^ 2, half_mirror, mirror):
            v = op(v, v[[part(l) for l in LANES]])
        a, b = swap32(v, v)
        v = op(a, b)
        a, b = swap16(v, v)
        v = op(a, b)
        assert np.all(v == want)


def test_int8_tile_bytes_follow_the_documented_order():
    # After the unit transpose, chunk offset o of a lane is b[s][v] with
    # o = 16 (v / 4) + 4 s + v % 4.  The kernel's int8 store: half h, dword
    # 2 q + odd takes bytes b[2q][4h + odd], b[2q][4h + 2 + odd],
    # b[2q + 1][4h + odd], b[2q + 1][4h + 2 + odd].  The 32 bytes must be the
    # documented W4A4_CODES_I8 order of codes 0..31 (each group of 8 as
    # 0,2,4,6,1,3,5,7), which tests/layouts.py writes independently.
    from layouts import i8_from_codes
    b = np.zeros((4, 8), np.int64)
    for s in range(4):
        for v in range(8):
            b[s, v] = 16 * (v >> 2) + 4 * s + (v & 3)
    out = []
    for h in range(2):
        for q in range(2):
            for odd in range(2):
                out += [b[2 * q][4 * h + odd], b[2 * q][4 * h + 2 + odd],
                        b[2 * q + 1][4 * h + odd], b[2 * q + 1][4 * h + 2 + odd]]
    assert out == list(i8_from_codes(np.arange(32).reshape(1, 32))[0])
