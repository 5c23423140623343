"""CPU check of the index math of the b = 128 rotation on the matrix
instruction (rotq_mfma.hip), against definitions that do not come from the
kernel: the Sylvester Hadamard matrix of scipy, the lane layouts of
v_mfma_f32_16x16x32_f16 (A: lane 16 g + r holds A[r][8 g + t]; B: lane
16 g + c holds B[8 g + t][c]; D: lane 16 g + c holds D[4 g + i][c]), and
the lane exchanges of v_permlane32_swap (lanes 32-63 of the first operand
trade places with lanes 0-31 of the second) and v_permlane16_swap (the odd
16-lane rows of the first operand with the even rows of the second).

The GPU tests check the kernel's codes against the oracle; this test pins the
fragment signs, the load addresses, the output positions and the 4 x 4 unit
transpose into the tile order on the host, so a slip in any of them shows up
without a GPU.
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
