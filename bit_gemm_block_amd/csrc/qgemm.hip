// qgemm.hip — int4 x int4 GEMM on gfx950 int8 matrix cores, with the
// dequantizing epilogue and the low-rank term (SERQ page, "Resumen técnico"
// §2-3: a 4-bit product in the linear layer plus a single low-rank
// compensation matrix added to it).
//
//   acc[m, n] = sum_k qx[m, k] * qw[n, k]          (exact int32)
//   y[m, n]   = sx[m] * sum_j sw[n, j] * acc_j[m, n] + (T . Bt^T)[m, n]
//
// Both operands are packed int4, K-contiguous ([rows, K/2] bytes).  There is
// no int4 matrix instruction on CDNA4, so codes are widened to int8 in
// registers right before v_mfma_i32_16x16x64_i8.  A nibble moved to the top
// of its byte is a valid signed int8 equal to 16*q, so the widening is one
// AND (high nibbles) or one shift+AND (low nibbles) per 8 codes, and the
// accumulator holds 256 * acc.  With codes down to -8, |acc| <= 64 K, so the
// int32 holds it exactly for K < 2^17; the library accepts K <= 16384 (the
// rotation kernel keeps a row of K values in one workgroup, 256 lanes x 64),
// and the in-GEMM residual form 8 K + r_pad < 2^17.  Low and high nibbles
// of a dword feed different int8 lanes of the instruction, i.e. the K order
// inside one instruction is permuted; A and B use the same permutation, so
// the dot products are exact.
//
// Large M: a 256-thread workgroup owns a (32 TM) x (32 TN) output tile; its
// four waves form a 2 x 2 grid of (16 TM) x (16 TN) wave tiles.  K advances
// 128 codes (64 bytes per row, two MFMA K steps) per iteration through a
// ring of LDS tiles (four stages for the tiled operands: the copies in
// flight per CU set the L2-to-LDS rate).  Tiles are handed to workgroups so that the
// workgroups resident on one XCD (each XCD has its own L2) cover a compact
// block of output tiles and share their A and B panels in that L2.
//
// Small M (decode, M <= 32): a workgroup owns 16 output columns and its waves
// split K; every lane streams its weight bytes straight from memory into
// registers (no LDS staging), the waves' partial tiles are reduced in LDS.
//
// Asymmetric activation groups (OffQ page, "Metodología" steps 2-3).  The
// codes hold q - 8 for uint4 q, with scale s[m, g] and integer zero point
// z[m, g] per token and group of channels, so that
//   y[m, n] = sw[n] * (sum_g s[m,g] acc_g[m,n] - sum_g o[m,g] wsum[n,g]),
//   acc_g = sum_{k in g} (q - 8) qw,  o = s (z - 8),
// wsum[n, g] being the weight codes summed over group g.  The first sum is
// the group flush of the main loop with per-row scales; the second, a
// rank-(K/group) product, runs on fp16 matrix instructions after the loop
// with both operands split exactly: o scaled by a power of two per row into
// an fp16 pair (hi + lo, about 22 bits), wsum as 64 a + c.
//
// Low-rank term.  fp16 path: T is given as an fp16 pair (t_hi, t_lo) [M, r]
// and Bt [N, r] is fp16; each 16x16 output block adds t_hi.Bt^T and
// t_lo.Bt^T with v_mfma_f32_16x16x32_f16, using the dequantized tile as the
// accumulator input.  fp32 path: float32 FMA loop.
#include "w4a4_internal.h"
#include "gemm_common.h"

#include <hip/hip_fp16.h>

#include <type_traits>

namespace w4a4 {
namespace {


constexpr int BK_BYTES = 64;  // 128 int4 codes per row per K iteration
constexpr float kInv256 = 0.00390625f;  // both operands carry 16*q
constexpr float kInv16 = 0.0625f;       // only the weights carry 16*q

// Widen 16 packed nibbles (two dwords) into one MFMA operand of 16 int8
// values 16*q: low nibbles of p0, high nibbles of p0, then the same for p1.
__device__ __forceinline__ i32x4 widen(uint32_t p0, uint32_t p1) {
  return i32x4{static_cast<int32_t>((p0 << 4) & 0xF0F0F0F0u), static_cast<int32_t>(p0 & 0xF0F0F0F0u),
               static_cast<int32_t>((p1 << 4) & 0xF0F0F0F0u), static_cast<int32_t>(p1 & 0xF0F0F0F0u)};
}

// The same 16 values 16*q from offset-binary weight bytes (high nibble: the
// even channel's signed code; low nibble: the odd channel's code + 8).
__device__ __forceinline__ i32x4 widen_ob(uint32_t p0, uint32_t p1) {
  return i32x4{static_cast<int32_t>(p0 & 0xF0F0F0F0u),
               static_cast<int32_t>(((p0 ^ 0x08080808u) << 4) & 0xF0F0F0F0u),
               static_cast<int32_t>(p1 & 0xF0F0F0F0u),
               static_cast<int32_t>(((p1 ^ 0x08080808u) << 4) & 0xF0F0F0F0u)};
}

// LDS tile layout ("fragment-major").  A K iteration covers 128 codes
// (64 bytes) of each tile row.  The 16-byte piece lane group g
// (lanes 16g..16g+15) of an MFMA reads holds codes [16g, 16g+16) of K step 0
// (codes 0..63 of the iteration) in its first 8 bytes and the same slice of
// K step 1 (codes 64..127) in its last 8 bytes, so that each K step is a
// contiguous range of 64 codes.  Pieces are stored as
// [row block (16 rows)][g (4)][row in block (16)][16 bytes], so the 64 lanes
// of one fragment read touch 1 KB of consecutive LDS and never collide in a
// bank; each ds_write_b64 of the staging writes two 256-byte runs.
//
// Byte offset of the piece read by lane group g for tile row r.
__device__ __forceinline__ int frag_off(int r, int g) {
  return (((r >> 4) * 4 + g) << 8) + ((r & 15) << 4);
}
// Byte offset of the logical 8 bytes [8p, 8p + 8) of tile row r.
__device__ __forceinline__ int piece_off(int r, int p) {
  return frag_off(r, p & 3) + ((p >> 2) << 3);
}

// int8 activation tiles (a_i8): a K iteration covers 128 bytes of each row;
// K step h, lane group g reads codes [64h + 16g, 64h + 16g + 16), stored as
// [row block][h (2)][g (4)][row in block (16)][16 bytes].
__device__ __forceinline__ int a8_off(int r, int h, int g) {
  return ((((r >> 4) * 2 + h) * 4 + g) << 8) + ((r & 15) << 4);
}

// The first LR_PRE 32-wide rank chunks of the fp16 low-rank operands of one
// 16x16 output block, loaded ahead of the main loop by the waves that run
// the epilogue (so that these loads overlap the weight stream).  The loads
// are unconditional, from clamped indices (rows past M or N give outputs that
// are not stored), so that no select of a loaded value makes the wave wait
// here; rank chunks past the rank are zeroed when the term is applied.
constexpr int LR_PRE = 2;
struct LowRankPre {
  half8 hi[LR_PRE], lo[LR_PRE], bb[LR_PRE];
};

__device__ __forceinline__ void load_lowrank_pre(const GemmArgs& a, int64_t mblk, int64_t nblk,
                                                 int lane, LowRankPre& p) {
  const int64_t mr0 = mblk + (lane & 15);
  const int64_t nr0 = nblk + (lane & 15);
  const int64_t mr = mr0 < a.M ? mr0 : a.M - 1;
  const int64_t nr = nr0 < a.N ? nr0 : a.N - 1;
  const int koff = (lane >> 4) * 8;
  const _Float16* th = static_cast<const _Float16*>(a.t);
  const _Float16* tl = th + a.M * a.rank;
  const _Float16* bt = static_cast<const _Float16*>(a.B);
#pragma unroll
  for (int q = 0; q < LR_PRE; ++q) {
    const int j0 = q * 32 + koff;
    const int j = j0 < a.rank ? j0 : a.rank - 8;  // the rank is a multiple of 8
    p.hi[q] = *reinterpret_cast<const half8*>(th + mr * a.rank + j);
    p.lo[q] = *reinterpret_cast<const half8*>(tl + mr * a.rank + j);
    p.bb[q] = *reinterpret_cast<const half8*>(bt + nr * a.rank + j);
  }
}

__device__ __forceinline__ f32x4 apply_lowrank_pre(const GemmArgs& a, const LowRankPre& p, int lane,
                                                   f32x4 v) {
  const half8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int q = 0; q < LR_PRE; ++q) {
    const half8 bb = q * 32 + (lane >> 4) * 8 < a.rank ? p.bb[q] : z;
    v = __builtin_amdgcn_mfma_f32_16x16x32_f16(p.lo[q], bb, v, 0, 0, 0);
    v = __builtin_amdgcn_mfma_f32_16x16x32_f16(p.hi[q], bb, v, 0, 0, 0);
  }
  return v;
}

// Writes one 16x16 block (int32 total >> shift and/or float32 y).
__device__ __forceinline__ void store_block(const GemmArgs& a, int64_t mblk, int64_t nblk, int lane,
                                            i32x4 total, f32x4 yv, int shift) {
  const int64_t n = nblk + (lane & 15);
  if (n >= a.N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = mblk + (lane >> 4) * 4 + i;
    if (m < a.M) {
      if (a.acc) a.acc[m * a.N + n] = total[i] >> shift;
      if (a.y) a.y[m * a.N + n] = yv[i];
    }
  }
}

template <int TM, int TN, bool GROUPED, int LRMODE, bool AI8>
__global__ void __launch_bounds__(256) qgemm_kernel(GemmArgs a) {
  constexpr int WM = TM * 16, WN = TN * 16;
  constexpr int BM = 2 * WM, BN = 2 * WN;
  constexpr int A_ROW = AI8 ? 2 * BK_BYTES : BK_BYTES;  // A bytes per row per iteration
  constexpr int A_UNITS = BM * A_ROW / 16 / 256;       // 16-byte loads per thread
  constexpr int B_UNITS = BN * BK_BYTES / 16 / 256;
  static_assert(A_UNITS >= 1 && B_UNITS >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * A_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * BK_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave >> 1) * WM;
  const int wn0 = (wave & 1) * WN;

  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (a.N + BN - 1) / BN;
  int64_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = tmi * BM;
  const int64_t n0 = tni * BN;
  const int64_t K = a.K;
  const int64_t row_bytes = K / 2;                 // packed rows
  const int64_t a_row_bytes = AI8 ? K : K / 2;     // activation rows
  const int nkt = static_cast<int>((K + 127) / 128);
  const bool k_tail = (K & 127) != 0;  // last iteration holds 64 codes

  // Staging pointers.  Rows past M (or N) are clamped to the last row: they
  // only feed output rows (columns) that are never stored.
  const uint8_t* pa[A_UNITS];
  const uint8_t* pb[B_UNITS];
  int sa[A_UNITS][2], sb[B_UNITS][2];  // LDS byte offsets (of the two halves)
#pragma unroll
  for (int i = 0; i < A_UNITS; ++i) {
    const int u = tid + 256 * i;
    if constexpr (AI8) {
      const int r = u >> 3, c = u & 7;
      const int64_t m = (m0 + r) < a.M ? (m0 + r) : (a.M - 1);
      pa[i] = a.xq + m * a_row_bytes + c * 16;
      sa[i][0] = a8_off(r, c >> 2, c & 3);
      sa[i][1] = 0;
    } else {
      const int r = u >> 2, c = u & 3;
      const int64_t m = (m0 + r) < a.M ? (m0 + r) : (a.M - 1);
      pa[i] = a.xq + m * a_row_bytes + c * 16;
      sa[i][0] = piece_off(r, 2 * c);
      sa[i][1] = piece_off(r, 2 * c + 1);
    }
  }
#pragma unroll
  for (int i = 0; i < B_UNITS; ++i) {
    const int u = tid + 256 * i;
    const int r = u >> 2, c = u & 3;
    const int64_t n = (n0 + r) < a.N ? (n0 + r) : (a.N - 1);
    pb[i] = a.wq + n * row_bytes + c * 16;
    sb[i][0] = piece_off(r, 2 * c);
    sb[i][1] = piece_off(r, 2 * c + 1);
  }
  // Units of this thread that lie in codes 64..127 of an iteration.
  const bool a_hi = AI8 ? (tid & 7) >= 4 : (tid & 3) >= 2;
  const bool b_hi = (tid & 3) >= 2;

  uint4 ra[A_UNITS], rb[B_UNITS];
  auto gload = [&](int kt) {
    const bool last = k_tail && kt == nkt - 1;
    const int64_t aoff = static_cast<int64_t>(kt) * A_ROW;
    const int64_t boff = static_cast<int64_t>(kt) * BK_BYTES;
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i)
      ra[i] = (last && a_hi) ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4*>(pa[i] + aoff);
#pragma unroll
    for (int i = 0; i < B_UNITS; ++i)
      rb[i] = (last && b_hi) ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4*>(pb[i] + boff);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i) {
      if constexpr (AI8) {
        *reinterpret_cast<uint4*>(&As[buf][sa[i][0]]) = ra[i];
      } else {
        *reinterpret_cast<uint2*>(&As[buf][sa[i][0]]) = make_uint2(ra[i].x, ra[i].y);
        *reinterpret_cast<uint2*>(&As[buf][sa[i][1]]) = make_uint2(ra[i].z, ra[i].w);
      }
    }
#pragma unroll
    for (int i = 0; i < B_UNITS; ++i) {
      *reinterpret_cast<uint2*>(&Bs[buf][sb[i][0]]) = make_uint2(rb[i].x, rb[i].y);
      *reinterpret_cast<uint2*>(&Bs[buf][sb[i][1]]) = make_uint2(rb[i].z, rb[i].w);
    }
  };

  i32x4 acc[TM][TN];
  f32x4 facc[GROUPED ? TM : 1][GROUPED ? TN : 1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
  if constexpr (GROUPED) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) facc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int gsteps = GROUPED ? a.group / 64 : 1;
  const int64_t ngroups = GROUPED ? K / a.group : 1;
  const int ksteps = static_cast<int>(K / 64);

  gload(0);
  lstore(0);
  __syncthreads();

  const int frow = lane & 15;  // fragment row within a 16-row block
  const int fg = lane >> 4;    // lane group

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);

    uint4 fa[AI8 ? 1 : TM], fb[TN];
    if constexpr (!AI8) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const uint4*>(&As[buf][frag_off(wm0 + i * 16 + frow, fg)]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[j] = *reinterpret_cast<const uint4*>(&Bs[buf][frag_off(wn0 + j * 16 + frow, fg)]);

#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x4 opb[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) opb[j] = h ? widen(fb[j].z, fb[j].w) : widen(fb[j].x, fb[j].y);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        i32x4 opa;
        if constexpr (AI8)
          opa = *reinterpret_cast<const i32x4*>(&As[buf][a8_off(wm0 + i * 16 + frow, h, fg)]);
        else
          opa = h ? widen(fa[i].z, fa[i].w) : widen(fa[i].x, fa[i].y);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(opa, opb[j], acc[i][j], 0, 0, 0);
      }
      if constexpr (GROUPED) {
        const int kstep = kt * 2 + h;
        if (kstep < ksteps && (kstep + 1) % gsteps == 0) {
          const int64_t grp = (kstep + 1) / gsteps - 1;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            int64_t n = n0 + wn0 + j * 16 + frow;
            n = n < a.N ? n : a.N - 1;
            const float sw = load_scale(a.sw, n * ngroups + grp, a.sw_f16);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                facc[i][j][r] = fmaf(static_cast<float>(acc[i][j][r]), sw, facc[i][j][r]);
              acc[i][j] = i32x4{0, 0, 0, 0};
            }
          }
        }
      }
    }

    if (kt + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  Output fragment (i, j) of this lane: rows
  // m0 + wm0 + 16 i + 4 (lane >> 4) + r (r < 4), column n0 + wn0 + 16 j + (lane & 15).
  const bool want_y = a.y != nullptr;
  const int64_t mlane = m0 + wm0 + (lane >> 4) * 4;
  const int64_t nlane = n0 + wn0 + (lane & 15);
  const bool interior = (m0 + BM <= a.M) && (n0 + BN <= a.N);
  float sxr[TM][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = mlane + i * 16 + r;
      sxr[i][r] = (want_y && m < a.M) ? a.sx[m] * (AI8 ? kInv16 : kInv256) : 0.f;
    }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t n = nlane + j * 16;
    const bool n_ok = n < a.N;
    const float swn = (GROUPED || !want_y || !n_ok) ? 1.f : load_scale(a.sw, n, a.sw_f16);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      f32x4 yv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (GROUPED)
          yv[r] = facc[i][j][r] * sxr[i][r];
        else
          yv[r] = static_cast<float>(acc[i][j][r]) * (sxr[i][r] * swn);
      }
      if constexpr (LRMODE != LR_NONE) {
        if (want_y) yv = add_lowrank<LRMODE>(a, yv, mlane - (lane >> 4) * 4 + i * 16, nlane - (lane & 15) + j * 16, lane);
      }
      const int64_t mb = mlane + i * 16;
      if (interior) {
        float* yp = a.y + mb * a.N + n;
        int32_t* ap = a.acc + mb * a.N + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (want_y) yp[r * a.N] = yv[r];
          if (!GROUPED && a.acc) ap[r * a.N] = acc[i][j][r] >> (AI8 ? 4 : 8);
        }
      } else if (n_ok) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (mb + r < a.M) {
            if (want_y) a.y[(mb + r) * a.N + n] = yv[r];
            if (!GROUPED && a.acc) a.acc[(mb + r) * a.N + n] = acc[i][j][r] >> (AI8 ? 4 : 8);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined kernel for int8 activation codes, K % 128 == 0 and weight groups
// that are multiples of 128.  Global memory is copied straight into LDS with
// global_load_lds_dwordx4 (each lane's 16 bytes land at lane * 16 of a 1 KB
// run), through a ring of STAGES LDS buffers, so loads run STAGES - 1
// iterations ahead of the matrix instructions without staging registers.
//
// K mapping of one 128-code iteration: K step h, lane group g covers codes
// [32g + 16h, 32g + 16h + 16): the int8 activation operand is the 16 bytes at
// that offset, the weight operand the h-th half of the 16 packed bytes
// [16g, 16g + 16) (codes [32g, 32g + 32)) after widening.
//
// LDS stage: A as [row block][h][g][16 rows][16 B], B as [row block][g][16
// rows][16 B]; every 1 KB run is filled by one wave instruction and read by
// one conflict-free ds_read_b128.
template <int TM, int TN, int STAGES, bool GROUPED, int LRMODE, bool TILED, bool APK,
          bool ASYM = false, bool G128 = false, bool AG1 = false, bool RES = false,
          bool OB = false>
__global__ void __launch_bounds__(256) qgemm_pipe_kernel(GemmArgs a) {
  // APK: activation codes packed (4 bits) in the weights' tile layout, widened
  // in registers like the weights; otherwise int8 codes.
  // ASYM: asymmetric activation groups (per-row group scales, zero points).
  static_assert(!APK || TILED, "packed activation codes come tiled");
  static_assert(!ASYM || (APK && !GROUPED), "asymmetric groups: packed codes, per-channel weights");
  // G128: groups of exactly one 128-code iteration.  The integer
  // accumulators are then double-buffered: iteration kt issues its matrix
  // instructions into one set and flushes the other (group kt - 1), so the
  // flush does not wait for the instructions just issued.
  // RES: in-GEMM residual (SERQ page, "Metodología" items 2-3).  After the
  // K / 128 main iterations, res_iters more iterations multiply code columns
  // [0, 128 res_iters) again, by the weights' residual tiles.  The main
  // accumulator is multiplied by 8 once at the switch, so that one int32
  // holds 256 (8 sum_k qx qw + sum_{k<r} qx qr); the epilogue scales by 1/8.
  // AG1: asymmetric codes with a single group per row (group = K): the
  // integer product runs over all of K like the symmetric one, and the row
  // scale and zero-point term enter in the epilogue only.
  // OB: offset-binary codes and weights (each byte: one signed nibble on top,
  // one offset nibble q + 8 below, paired crosswise between the operands).
  // Per 16 packed bytes the first K step takes the activations' high nibbles
  // with the weights' low ones and the second step the reverse, one AND per
  // dword; the accumulator holds 16 sum qx qw + 128 (row sum + column sum).
  static_assert(!OB || (APK && TILED && !GROUPED && !ASYM && !RES), "offset-binary: plain packed");
  constexpr int WM = TM * 16, WN = TN * 16;
  constexpr int BM = 2 * WM, BN = 2 * WN;
  constexpr int A_BYTES = BM * (APK ? 64 : 128), B_BYTES = BN * 64;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_RUNS = APK ? BM / 16 : BM / 16 * 2, B_RUNS = BN / 16;
  // both operands widened: 256 * acc (offset-binary: 16 * acc after the correction)
  constexpr float kInvA = (APK && !OB) ? kInv256 : kInv16;
  constexpr int kShiftA = (APK && !OB) ? 8 : 4;
  constexpr int RUNS = A_RUNS + B_RUNS;
  static_assert(RUNS % 4 == 0, "runs split evenly over 4 waves");
  static_assert(STAGES >= 2 && STAGES <= 8, "stages");
  constexpr int RUNS_PER_WAVE = RUNS / 4;
  static_assert((STAGES - 1) * RUNS_PER_WAVE < 64, "in-flight copies exceed vmcnt");
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[STAGES > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st3[STAGES > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st4[STAGES > 4 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st5[STAGES > 5 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st6[STAGES > 6 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st7[STAGES > 7 ? STAGE : 16];
  auto stage = [&](int sidx) -> uint8_t* {
    switch (sidx) {
      case 0: return st0;
      case 1: return st1;
      case 2: return st2;
      case 3: return st3;
      case 4: return st4;
      case 5: return st5;
      case 6: return st6;
      default: return st7;
    }
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar run addresses
  const int wm0 = (wave >> 1) * WM;
  const int wn0 = (wave & 1) * WN;
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (a.N + BN - 1) / BN;
  int64_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = tmi * BM;
  const int64_t n0 = tni * BN;
  const int64_t K = a.K;
  static_assert(!RES || (APK && !GROUPED && !ASYM && LRMODE == LR_NONE),
                "residual: packed codes, per-channel weights");
  const int nkt_a = static_cast<int>(K / 128);               // code tiles per row block
  const int nkt = nkt_a + (RES ? a.res_iters : 0);           // iterations (weight tiles)

  // Source pointer (at iteration 0) and LDS offset of each run this wave
  // copies.  Row-major operands: a run is 16 rows x 64 bytes, and the pointer
  // is the lane's own.  Tiled operands: a run is one contiguous 1 KB block
  // already in fragment order, and the pointer is the block's (wave-uniform)
  // start.
  const uint8_t* src[RUNS_PER_WAVE];
  int dst[RUNS_PER_WAVE];
  int step[RUNS_PER_WAVE];
  const int64_t mblocks = (a.M + 15) / 16, nblocks = (a.N + 15) / 16;
#pragma unroll
  for (int q = 0; q < RUNS_PER_WAVE; ++q) {
    const int run = wave + 4 * q;
    const int g = lane >> 4, rr = lane & 15;
    if (run < A_RUNS && APK) {
      int64_t mb = m0 / 16 + run;
      mb = mb < mblocks ? mb : mblocks - 1;
      src[q] = a.xq + mb * nkt_a * 1024;
      step[q] = 1024;
      dst[q] = (run * 4) << 8;
    } else if (run < A_RUNS) {
      const int blk = run >> 1, h = run & 1;
      if constexpr (TILED) {
        int64_t mb = m0 / 16 + blk;
        mb = mb < mblocks ? mb : mblocks - 1;
        src[q] = a.xq + (mb * nkt_a * 2 + h) * 1024;
        step[q] = 2048;
      } else {
        int64_t m = m0 + blk * 16 + rr;
        m = m < a.M ? m : a.M - 1;
        src[q] = a.xq + m * K + 32 * g + 16 * h;
        step[q] = 128;
      }
      dst[q] = ((blk * 2 + h) * 4) << 8;
    } else {
      const int blk = run - A_RUNS;
      if constexpr (TILED) {
        int64_t nb = n0 / 16 + blk;
        nb = nb < nblocks ? nb : nblocks - 1;
        src[q] = a.wq + nb * nkt * 1024;
        step[q] = 1024;
      } else {
        int64_t n = n0 + blk * 16 + rr;
        n = n < a.N ? n : a.N - 1;
        src[q] = a.wq + n * (K / 2) + 16 * g;
        step[q] = 64;
      }
      dst[q] = A_BYTES + ((blk * 4) << 8);
    }
  }
  auto issue = [&](int kt, uint8_t* base) {
    const uint32_t b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(base));
#pragma unroll
    for (int q = 0; q < RUNS_PER_WAVE; ++q) {
      int64_t t = kt;
      // residual iterations read the code columns from the start again
      if (RES && kt >= nkt_a && wave + 4 * q < A_RUNS) t -= nkt_a;
      if constexpr (TILED)  // src[q] is the run's uniform base; lane l copies bytes [16 l, 16 l + 16)
        dma16s(src[q] + t * step[q], 16 * lane, b + dst[q]);
      else
        dma16(src[q] + t * step[q], __builtin_amdgcn_readfirstlane(b + dst[q]));
    }
  };

  static_assert(!AG1 || ASYM, "single-group mode is asymmetric");
  constexpr bool FLUSH = GROUPED || (ASYM && !AG1);  // float accumulation per K-group
  static_assert(!G128 || FLUSH, "double-buffered flush needs groups");
  i32x4 acc[TM][TN];
  i32x4 acc2[G128 ? TM : 1][G128 ? TN : 1];
  f32x4 facc[FLUSH ? TM : 1][FLUSH ? TN : 1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
  if constexpr (G128) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc2[i][j] = i32x4{0, 0, 0, 0};
  }
  if constexpr (FLUSH) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) facc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int gsize = GROUPED ? a.group : ASYM ? a.agroup : 128;
  const int iters_per_group = gsize / 128;
  const int64_t ngroups = FLUSH ? K / gsize : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t gsc[];  // grouped scales

  const int frow = lane & 15;
  const int fg = lane >> 4;
  auto read_frags = [&](const uint8_t* As, i32x4 (&fa)[2][TM], uint4 (&fb)[TN]) {
    const uint8_t* Bs = As + A_BYTES;
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[j] = *reinterpret_cast<const uint4*>(Bs + ((((wn0 >> 4) + j) * 4 + fg) << 8) + (frow << 4));
    if constexpr (APK) {
      // packed: fa[0][i] holds both K halves' nibbles of row block i
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[0][i] = *reinterpret_cast<const i32x4*>(As + ((((wm0 >> 4) + i) * 4 + fg) << 8) +
                                                   (frow << 4));
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          fa[h][i] = *reinterpret_cast<const i32x4*>(
              As + (((((wm0 >> 4) + i) * 2 + h) * 4 + fg) << 8) + (frow << 4));
    }
  };
  // ZC: with G128 and no low-rank epilogue, each group's first matrix
  // instruction starts from a zero accumulator input, so a flush need not
  // clear its set (with the low-rank epilogue this would cost the kernel its
  // second wave per SIMD).
  constexpr bool ZC = G128 && LRMODE == LR_NONE;
  // Adds the float value of one set of group accumulators, scaled, to facc
  // and clears the set (unless ZC).
  auto flush = [&](i32x4 (&ac)[TM][TN], int64_t grp) {
    if constexpr (GROUPED) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = wn0 + j * 16 + frow;
        const float sw = a.sw_f16 ? __half2float(reinterpret_cast<const __half*>(gsc)[grp * BN + col])
                                  : reinterpret_cast<const float*>(gsc)[grp * BN + col];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            facc[i][j][r] = fmaf(static_cast<float>(ac[i][j][r]), sw, facc[i][j][r]);
          if constexpr (!ZC) ac[i][j] = i32x4{0, 0, 0, 0};
        }
      }
    }
    if constexpr (ASYM && !AG1) {
      const float* srow = reinterpret_cast<const float*>(gsc) + grp * BM + wm0 + 4 * fg;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const f32x4 sv = *reinterpret_cast<const f32x4*>(srow + i * 16);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            facc[i][j][r] = fmaf(static_cast<float>(ac[i][j][r]), sv[r], facc[i][j][r]);
          if constexpr (!ZC) ac[i][j] = i32x4{0, 0, 0, 0};
        }
      }
    }
  };
  // cur: the accumulators of this iteration; prev: the other set (G128).
  auto compute = [&](int kt, const i32x4 (&fa)[2][TM], const uint4 (&fb)[TN],
                     i32x4 (&cur)[TM][TN], i32x4 (&prev)[TM][TN]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x4 opb[TN];
      i32x4 opa[TM];
      if constexpr (OB) {
        // step 0: activation high x weight low nibbles; step 1: the reverse
        const uint32_t ma = h ? 0x0F0F0F0Fu : 0xF0F0F0F0u, mb = ~ma;
#pragma unroll
        for (int j = 0; j < TN; ++j)
          opb[j] = i32x4{static_cast<int32_t>(fb[j].x & mb), static_cast<int32_t>(fb[j].y & mb),
                         static_cast<int32_t>(fb[j].z & mb), static_cast<int32_t>(fb[j].w & mb)};
#pragma unroll
        for (int i = 0; i < TM; ++i) opa[i] = fa[0][i] & static_cast<int32_t>(ma);
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) opb[j] = h ? widen(fb[j].z, fb[j].w) : widen(fb[j].x, fb[j].y);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if constexpr (APK)
            opa[i] = h ? widen(fa[0][i][2], fa[0][i][3]) : widen(fa[0][i][0], fa[0][i][1]);
          else
            opa[i] = fa[h][i];
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          cur[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              opa[i], opb[j], (ZC && h == 0) ? i32x4{0, 0, 0, 0} : cur[i][j], 0, 0, 0);
    }
    if constexpr (RES) {
      if (kt == nkt_a - 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) cur[i][j] = cur[i][j] << 3;
      }
    }
    if constexpr (G128) {
      // group kt - 1 (at kt = 0 the set is all zero and any scale adds 0)
      flush(prev, kt > 0 ? kt - 1 : 0);
    } else if constexpr (FLUSH) {
      if ((kt + 1) % iters_per_group == 0) flush(cur, (kt + 1) / iters_per_group - 1);
    }
  };

  // Grouped scales: this tile's columns for every group, staged in LDS as
  // [group][column] before any copy is in flight.  Read from global memory
  // inside the loop they would make the compiler wait for every outstanding
  // vector memory operation, the stage copies included.
  if constexpr (GROUPED) {
    const int esz = a.sw_f16 ? 2 : 4;
    for (int e = tid; e < BN * ngroups; e += 256) {
      const int col = e % BN;
      const int64_t grp = e / BN;
      int64_t n = n0 + col;
      n = n < a.N ? n : a.N - 1;
      if (esz == 2)
        reinterpret_cast<__half*>(gsc)[e] = reinterpret_cast<const __half*>(a.sw)[n * ngroups + grp];
      else
        reinterpret_cast<float*>(gsc)[e] = reinterpret_cast<const float*>(a.sw)[n * ngroups + grp];
    }
    __syncthreads();
  }
  // Asymmetric groups: this tile's row scales for every group as
  // [group][row] (times the 1/256 of the widened operands), followed by one
  // word per row for the epilogue's row maxima.
  if constexpr (ASYM) {
    const int64_t nstaged = AG1 ? 0 : ngroups;  // single group: scale applied in the epilogue
    float* sl = reinterpret_cast<float*>(gsc);
    for (int e = tid; e < BM * nstaged; e += 256) {
      const int row = e % BM;
      const int64_t grp = e / BM;
      int64_t m = m0 + row;
      m = m < a.M ? m : a.M - 1;
      sl[e] = a.sx[m * ngroups + grp] * kInvA;
    }
    if (tid < BM) reinterpret_cast<uint32_t*>(gsc)[BM * nstaged + tid] = 0u;
    __syncthreads();
  }

  // EPL (offset-binary kernels): the epilogue's row scales, row sums and
  // column sums are copied into LDS before the first stage, so that the
  // epilogue reads them from LDS instead of waiting for global loads after
  // the loop: [0, BM) the row scales, [BM, 2 BM) the row sums and
  // [2 BM, 2 BM + BN) the column sums.  Rows and columns past the ends copy
  // the last valid element (never used).  The copies precede the stage
  // copies, so the prologue's wait covers them.  (Measured on the plain
  // kernel, the same staging made the 4096 x 28672 x 4096 product slower.)
  constexpr bool EPL = OB;
  __shared__ __attribute__((aligned(16))) uint32_t epl[EPL ? 2 * BM + BN : 1];
  if constexpr (EPL) {
    const uint32_t eb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(epl));
    if (a.y && a.sx) {
      for (int c = wave; c < BM / 64; c += 4) {
        int64_t m = m0 + c * 64 + lane;
        m = m < a.M ? m : a.M - 1;
        dma4(a.sx + m, eb + c * 256);
      }
    }
    if constexpr (OB) {
      for (int c = wave; c < BM / 64; c += 4) {
        int64_t m = m0 + c * 64 + lane;
        m = m < a.M ? m : a.M - 1;
        dma4(a.ob_sa + m, eb + 4 * BM + c * 256);
      }
      for (int c = wave; c < BN / 64; c += 4) {
        int64_t n = n0 + c * 64 + lane;
        n = n < a.N ? n : a.N - 1;
        dma4(a.ob_sb + n, eb + 8 * BM + c * 256);
      }
    }
  }

  // Prologue: the first STAGES stages in flight, stage 0 visible, its
  // fragments read.
#pragma unroll
  for (int sidx = 0; sidx < STAGES; ++sidx)
    if (sidx < nkt) issue(sidx, stage(sidx));
  if (nkt >= STAGES)
    wait_vmcnt<(STAGES - 1) * RUNS_PER_WAVE>();
  else
    wait_vmcnt<0>();
  stage_barrier();
  i32x4 fa0[2][TM], fa1[2][TM];
  uint4 fb0[TN], fb1[TN];
  read_frags(stage(0), fa0, fb0);

  // Iteration kt (stage buffer s = kt % STAGES): once stage kt + 1 has landed
  // and the barrier has retired every wave's reads of stage kt, the buffer
  // of stage kt is refilled with stage kt + STAGES and stage kt + 1's
  // fragments are read into the other register set; stage kt's matrix
  // instructions then run while those reads are in flight.
  // steady: kt + STAGES < nkt is known to hold (no branch on it).
  auto iterate = [&](int kt, int sbuf, i32x4 (&fac)[2][TM], uint4 (&fbc)[TN], i32x4 (&fan)[2][TM],
                     uint4 (&fbn)[TN], int odd, bool steady) {
    // The reads are unconditional (on the last iteration they read a stale,
    // in-bounds buffer) so that no branch joins between them and the matrix
    // instructions, where the compiler would wait for them.
    if (steady || kt + STAGES <= nkt)
      wait_vmcnt<(STAGES - 2) * RUNS_PER_WAVE>();
    else
      wait_vmcnt<0>();
    stage_barrier();
    if (steady || kt + STAGES < nkt) issue(kt + STAGES, stage(sbuf));
    read_frags(stage((sbuf + 1) % STAGES), fan, fbn);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
    if constexpr (G128) {
      if (odd)
        compute(kt, fac, fbc, acc2, acc);
      else
        compute(kt, fac, fbc, acc, acc2);
    } else {
      compute(kt, fac, fbc, acc, acc);
    }
  };
  // kt0 is a multiple of 2 * STAGES, so the parity of kt is that of u, a
  // compile-time constant in every unrolled iteration.  The loop runs the
  // blocks of 2 * STAGES iterations that all refill a stage, with no
  // per-iteration branch; it leaves fewer than 3 * STAGES iterations, which
  // run unrolled after it.
  // (Kernels with group flushes, and the row-major ones, keep the single
  // loop: with two copies of the iteration their registers no longer fit two
  // waves per SIMD.)
  constexpr bool SPLIT = !FLUSH && TILED;
  int kt0 = 0;
  for (; SPLIT && kt0 + 3 * STAGES <= nkt; kt0 += 2 * STAGES) {
#pragma unroll
    for (int u = 0; u < 2 * STAGES; ++u) {
      if (u & 1)
        iterate(kt0 + u, u % STAGES, fa1, fb1, fa0, fb0, 1, true);
      else
        iterate(kt0 + u, u % STAGES, fa0, fb0, fa1, fb1, 0, true);
    }
  }
  if constexpr (!SPLIT) {
    for (; kt0 < nkt; kt0 += 2 * STAGES) {
#pragma unroll
      for (int u = 0; u < 2 * STAGES; ++u) {
        const int kt = kt0 + u;
        if (kt < nkt) {
          if (u & 1)
            iterate(kt, u % STAGES, fa1, fb1, fa0, fb0, 1, false);
          else
            iterate(kt, u % STAGES, fa0, fb0, fa1, fb1, 0, false);
        }
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < 3 * STAGES; ++u) {
      const int kt = kt0 + u;
      if (kt < nkt) {
        if (u & 1)
          iterate(kt, u % STAGES, fa1, fb1, fa0, fb0, 1, false);
        else
          iterate(kt, u % STAGES, fa0, fb0, fa1, fb1, 0, false);
      }
    }
  }
  if constexpr (G128) {
    // the last group sits in the set of parity (nkt - 1) & 1; the other set
    // was flushed already (and, unless ZC, cleared)
    const int last = nkt - 1;
    if (last & 1)
      flush(acc2, last);
    else
      flush(acc, last);
  }

  // Asymmetric groups: corr[i][j] = 2^-e(m) sum_g o[m,g] wsum[n,g] for the
  // wave's blocks, e(m) the per-row exponent that brings max_g |o[m,g]| into
  // [2^13, 2^14).  The operands go through the stage buffers (free once every
  // wave is past its last fragment read) CG groups at a time; MFMA lane
  // group fg takes hi (fg < 2) or lo (fg >= 2) of o and 64 a (fg even) or c
  // (fg odd) of wsum, so that one instruction sums (hi + lo)(64 a + c) over
  // 8 groups.
  f32x4 corr[ASYM ? TM : 1][ASYM ? TN : 1];
  int eout[ASYM ? TM : 1][4];
  if constexpr (ASYM) {
    constexpr int CG = 16;
    static_assert(BM * CG * 4 <= STAGE && BN * CG * 4 <= STAGE, "operands fit a stage buffer");
    const int G = AG1 ? 1 : static_cast<int>(ngroups);
    uint32_t* rmax = reinterpret_cast<uint32_t*>(gsc) + (AG1 ? 0 : BM * G);
    stage_barrier();
    // Row maxima of |s (z - 8)|: 256 / BM consecutive threads per row, each
    // over every (256 / BM)-th group, joined by lane swaps (LDS atomics on
    // the row words serialised the 32-plus updates of each row: 10 us of the
    // 4096^3 layer).  Non-negative floats order as their bit patterns, so
    // the words are the ones an unsigned maximum of the bits gives.
    static_assert(256 % BM == 0, "whole rows per workgroup");
    {
      constexpr int TPR = 256 / BM;
      const int row = tid / TPR, part = tid % TPR;
      const int64_t m = m0 + row;
      float mx = 0.f;
      if (m < a.M) {
#pragma unroll 4
        for (int g = part; g < G; g += TPR)
          mx = fmaxf(mx, fabsf(a.sx[m * G + g] * static_cast<float>(a.zx[m * G + g] - 8)));
      }
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      if (part == 0) rmax[row] = __float_as_uint(mx);
    }
    __syncthreads();
    auto row_exp = [&](int row) -> int {
      const uint32_t u = rmax[row];
      return u ? static_cast<int>((u >> 23) & 0xFF) - 140 : 0;
    };
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) corr[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    _Float16* ao = reinterpret_cast<_Float16*>(st0);
    _Float16* bo = reinterpret_cast<_Float16*>(st1);
    for (int g0 = 0; g0 < G; g0 += CG) {
      for (int e = tid; e < BM * CG; e += 256) {
        const int row = e / CG, t = e % CG, g = g0 + t;
        const int64_t m = m0 + row;
        float o = 0.f;
        if (m < a.M && g < G) o = a.sx[m * G + g] * static_cast<float>(a.zx[m * G + g] - 8);
        const float oh = ldexpf(o, -row_exp(row));
        const _Float16 h = static_cast<_Float16>(oh);
        ao[row * 2 * CG + t] = h;
        ao[row * 2 * CG + CG + t] = static_cast<_Float16>(oh - static_cast<float>(h));
      }
      for (int e = tid; e < BN * CG; e += 256) {
        const int col = e / CG, t = e % CG, g = g0 + t;
        const int64_t n = n0 + col;
        const int w = (n < a.N && g < G) ? a.wsum[n * G + g] : 0;
        const int w64 = ((w + 32) >> 6) * 64;
        bo[col * 2 * CG + t] = static_cast<_Float16>(static_cast<float>(w64));
        bo[col * 2 * CG + CG + t] = static_cast<_Float16>(static_cast<float>(w - w64));
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < CG / 8; ++h) {
        half8 bv[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bv[j] = *reinterpret_cast<const half8*>(bo + (wn0 + 16 * j + frow) * 2 * CG +
                                                  ((fg & 1) ? CG : 0) + 8 * h);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const half8 av = *reinterpret_cast<const half8*>(ao + (wm0 + 16 * i + frow) * 2 * CG +
                                                           (fg >= 2 ? CG : 0) + 8 * h);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            corr[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv[j], corr[i][j], 0, 0, 0);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) eout[i][r] = row_exp(wm0 + 16 * i + 4 * fg + r);
  }

  // Epilogue (accumulators hold 16 * acc: only the weights carry the factor).
  const bool interior = (m0 + BM <= a.M) && (n0 + BN <= a.N);
  const bool want_y = a.y != nullptr;
  const int64_t mlane = m0 + wm0 + (lane >> 4) * 4;
  const int64_t nlane = n0 + wn0 + (lane & 15);
  float sxr[TM][4], swr[TN];
  int32_t sar[OB ? TM : 1][4];  // offset-binary: 128 * (row sum) of each lane row
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int lr0 = wm0 + (lane >> 4) * 4 + i * 16;  // the lane's first row of block i, in the tile
    // The staged rows are read unconditionally (one 16-byte LDS read per block,
    // every row of the tile is staged) and masked after.  Unstaged: one
    // 16-byte global read when the block's four rows exist, else per row.
    f32x4 sv = f32x4{0.f, 0.f, 0.f, 0.f};
    i32x4 av = i32x4{0, 0, 0, 0};
    const int64_t mf = mlane + i * 16;  // a multiple of 4: x_scale + mf is 16-byte aligned
    if constexpr (EPL) {
      sv = *reinterpret_cast<const f32x4*>(&epl[lr0]);
      av = *reinterpret_cast<const i32x4*>(&epl[BM + lr0]);
    } else if ((!ASYM || AG1) && want_y) {
      if (mf + 3 < a.M) {
        sv = *reinterpret_cast<const f32x4*>(a.sx + mf);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mf + r < a.M) sv[r] = a.sx[mf + r];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool live = (!ASYM || AG1) && want_y && mf + r < a.M;
      sxr[i][r] = live ? sv[r] * (RES ? kInvA * 0.125f : kInvA) : 0.f;
      if constexpr (OB) sar[i][r] = 128 * av[r];
    }
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t n = nlane + j * 16;
    swr[j] = (GROUPED || !want_y || n >= a.N) ? 1.f : load_scale(a.sw, n, a.sw_f16);
  }

  // fp16 low-rank term: the first 32 ranks of the wave's Bt rows are loaded
  // before the stores, and the loop below runs row blocks outermost, loading
  // each row block's T pair (hi, lo) once: TM dependent loads per wave in
  // place of one chain per output block.  Further ranks go through
  // add_lowrank; the instructions and their order are add_lowrank's, so the
  // result is the same.
  constexpr bool LRP = LRMODE == LR_F16;
  const half8 lr_z = {0, 0, 0, 0, 0, 0, 0, 0};
  const int lr_koff = (lane >> 4) * 8;
  const bool lr_kok = want_y && lr_koff < a.rank;
  half8 lr_b[LRP ? TN : 1];
  if constexpr (LRP) {
    const _Float16* bt = static_cast<const _Float16*>(a.B);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t nr = n0 + wn0 + j * 16 + (lane & 15);
      lr_b[j] = (lr_kok && nr < a.N) ? *reinterpret_cast<const half8*>(bt + nr * a.rank + lr_koff)
                                     : lr_z;
    }
  }

  // The common case (interior tile, Y only) runs a copy of the store loop
  // with no per-store checks.
  auto emit = [&](auto fast) {
    constexpr bool FAST = decltype(fast)::value;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    half8 lr_hi = lr_z, lr_lo = lr_z;
    if constexpr (LRP) {
      const int64_t mr = m0 + wm0 + i * 16 + (lane & 15);
      if (lr_kok && mr < a.M) {
        const _Float16* th = static_cast<const _Float16*>(a.t);
        lr_hi = *reinterpret_cast<const half8*>(th + mr * a.rank + lr_koff);
        lr_lo = *reinterpret_cast<const half8*>(th + (a.M + mr) * a.rank + lr_koff);
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = nlane + j * 16;
      const bool n_ok = n < a.N;
      const float swn = swr[j];
      const int32_t sbn = OB ? 128 * static_cast<int32_t>(epl[2 * BM + wn0 + (lane & 15) + j * 16]) : 0;
      if constexpr (OB) {
        // exact: the accumulator less 128 (row sum + column sum) is 16 sum qx qw
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] -= sar[i][r] + sbn;
      }
      f32x4 yv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (AG1)
          yv[r] = (static_cast<float>(acc[i][j][r]) * sxr[i][r] -
                   ldexpf(corr[i][j][r], eout[i][r])) * swn;
        else if constexpr (ASYM)
          yv[r] = (facc[i][j][r] - ldexpf(corr[i][j][r], eout[i][r])) * swn;
        else if constexpr (GROUPED)
          yv[r] = facc[i][j][r] * sxr[i][r];
        else
          yv[r] = static_cast<float>(acc[i][j][r]) * (sxr[i][r] * swn);
      }
      if constexpr (LRP) {
        if (want_y) {
          yv = __builtin_amdgcn_mfma_f32_16x16x32_f16(lr_lo, lr_b[j], yv, 0, 0, 0);
          yv = __builtin_amdgcn_mfma_f32_16x16x32_f16(lr_hi, lr_b[j], yv, 0, 0, 0);
          if (a.rank > 32)
            yv = add_lowrank<LRMODE>(a, yv, m0 + wm0 + i * 16, n0 + wn0 + j * 16, lane, 32);
        }
      } else if constexpr (LRMODE != LR_NONE) {
        if (want_y)
          yv = add_lowrank<LRMODE>(a, yv, m0 + wm0 + i * 16, n0 + wn0 + j * 16, lane);
      }
      const int64_t mb = mlane + i * 16;
      if constexpr (FAST) {
        float* yp = a.y + mb * a.N + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) yp[r * a.N] = yv[r];
      } else if (interior) {
        float* yp = a.y + mb * a.N + n;
        int32_t* ap = a.acc + mb * a.N + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (want_y) yp[r * a.N] = yv[r];
          if (!FLUSH && !ASYM && a.acc) ap[r * a.N] = acc[i][j][r] >> kShiftA;
        }
      } else if (n_ok) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (mb + r < a.M) {
            if (want_y) a.y[(mb + r) * a.N + n] = yv[r];
            if (!FLUSH && !ASYM && a.acc) a.acc[(mb + r) * a.N + n] = acc[i][j][r] >> kShiftA;
          }
        }
      }
    }
  }
  };
  if (interior && want_y && (FLUSH || ASYM || !a.acc))
    emit(std::true_type{});
  else
    emit(std::false_type{});
}

// MXFP4 GEMM (SERQ page, "Metodología" item 2: the 4-bit path in MXFP4).
// Codes are FP4 E2M1 in the packed tiled layout, with one E8M0 scale byte
// per 32 elements in 64-byte tiles.  The tile layout is already the operand
// layout of v_mfma_scale_f32_16x16x128_f8f6f4 (lane 16 g + r: row r,
// elements 32 g .. 32 g + 31 of the 128-element step, low nibble first; the
// lane's scale byte covers exactly those 32), so one instruction per 16x16
// block and 128-element step takes the fragments as they are, with no
// widening.  Per stage each wave also copies one 256-byte run of scales:
// waves 0-1 the A row blocks, waves 2-3 the B column blocks.

template <int TM, int TN, int STAGES, int LRMODE, int WGM = 2>
__global__ void __launch_bounds__(128 * WGM) qgemm_mx_kernel(GemmArgs a) {
  // WGM x 2 waves, each a (16 TM) x (16 TN) wave tile.
  constexpr int NW = 2 * WGM;
  constexpr int WM = TM * 16, WN = TN * 16;
  constexpr int BM = WGM * WM, BN = 2 * WN;
  constexpr int A_BYTES = BM * 64, B_BYTES = BN * 64;
  constexpr int SA_BYTES = BM / 16 * 64, SB_BYTES = BN / 16 * 64;
  // Scale runs: 256 bytes (4 blocks) per wave; waves past the A and B scale
  // runs repeat a B run into a spare slot, so every wave issues the same
  // number of copies.
  constexpr int SA_WAVES = SA_BYTES / 256, SB_WAVES = SB_BYTES / 256;
  static_assert(SA_WAVES + SB_WAVES <= NW, "scale runs fit the waves");
  constexpr int SPARE = 256;
  constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES + SPARE;
  constexpr int A_RUNS = BM / 16, B_RUNS = BN / 16;
  constexpr int RUNS = A_RUNS + B_RUNS;
  static_assert(RUNS % NW == 0, "runs split evenly over the waves");
  constexpr int RUNS_PER_WAVE = RUNS / NW + 1;  // + the scale run
  static_assert((STAGES - 1) * RUNS_PER_WAVE < 64, "in-flight copies exceed vmcnt");
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[STAGES > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st3[STAGES > 3 ? STAGE : 16];
  auto stage = [&](int sidx) -> uint8_t* {
    switch (sidx) {
      case 0: return st0;
      case 1: return st1;
      case 2: return st2;
      default: return st3;
    }
  };
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar run addresses
  const int wm0 = (wave >> 1) * WM;
  const int wn0 = (wave & 1) * WN;
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (a.N + BN - 1) / BN;
  int64_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = tmi * BM;
  const int64_t n0 = tni * BN;
  const int nkt = static_cast<int>(a.K / 128);
  const int64_t mblocks = (a.M + 15) / 16, nblocks = (a.N + 15) / 16;

  // Code runs: one contiguous 1 KB tile each, from the run's uniform base
  // (lane l copies bytes [16 l, 16 l + 16)).  Scale run: 16 lanes x 16 B,
  // lane l copying bytes 16 (l & 3) .. of the scale tile of block l / 4
  // (a per-lane address).
  const uint8_t* src[RUNS_PER_WAVE];
  int dst[RUNS_PER_WAVE];
#pragma unroll
  for (int q = 0; q < RUNS_PER_WAVE - 1; ++q) {
    const int run = wave + NW * q;
    if (run < A_RUNS) {
      int64_t mb = m0 / 16 + run;
      mb = mb < mblocks ? mb : mblocks - 1;
      src[q] = a.xq + mb * nkt * 1024;
      dst[q] = (run * 4) << 8;
    } else {
      const int blk = run - A_RUNS;
      int64_t nb = n0 / 16 + blk;
      nb = nb < nblocks ? nb : nblocks - 1;
      src[q] = a.wq + nb * nkt * 1024;
      dst[q] = A_BYTES + ((blk * 4) << 8);
    }
  }
  {
    const int side = wave < SA_WAVES ? 0 : 1;        // 0: A scales, 1: B scales
    const int part = side ? (wave - SA_WAVES) % SB_WAVES : wave;
    const int blk = part * 4 + ((lane & 15) >> 2);
    int64_t b = (side ? n0 : m0) / 16 + blk;
    const int64_t nbl = side ? nblocks : mblocks;
    b = b < nbl ? b : nbl - 1;
    src[RUNS_PER_WAVE - 1] = (side ? a.mx_ws : a.mx_xs) + b * nkt * 64 + 16 * (lane & 3);
    dst[RUNS_PER_WAVE - 1] = wave >= SA_WAVES + SB_WAVES
                                 ? A_BYTES + B_BYTES + SA_BYTES + SB_BYTES
                                 : A_BYTES + B_BYTES + side * SA_BYTES + part * 256;
  }
  auto issue = [&](int kt, uint8_t* base) {
    const uint32_t b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(base));
#pragma unroll
    for (int q = 0; q < RUNS_PER_WAVE - 1; ++q)
      dma16s(src[q] + static_cast<int64_t>(kt) * 1024, 16 * lane, b + dst[q]);
    if (lane < 16)
      dma16(src[RUNS_PER_WAVE - 1] + static_cast<int64_t>(kt) * 64,
            __builtin_amdgcn_readfirstlane(b + dst[RUNS_PER_WAVE - 1]));
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fg = lane >> 4;
  auto read_frags = [&](const uint8_t* As, i32x4 (&fa)[TM], i32x4 (&fb)[TN], int (&sa)[TM],
                        int (&sb)[TN]) {
    const uint8_t* Bs = As + A_BYTES;
    const uint8_t* Ss = As + A_BYTES + B_BYTES;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      fa[i] = *reinterpret_cast<const i32x4*>(As + ((((wm0 >> 4) + i) * 4 + fg) << 8) + (frow << 4));
      sa[i] = Ss[((wm0 >> 4) + i) * 64 + fg * 16 + frow];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      fb[j] = *reinterpret_cast<const i32x4*>(Bs + ((((wn0 >> 4) + j) * 4 + fg) << 8) + (frow << 4));
      sb[j] = Ss[SA_BYTES + ((wn0 >> 4) + j) * 64 + fg * 16 + frow];
    }
  };
  auto compute = [&](const i32x4 (&fa)[TM], const i32x4 (&fb)[TN], const int (&sa)[TM],
                     const int (&sb)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const i32x8 av = {fa[i][0], fa[i][1], fa[i][2], fa[i][3], 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const i32x8 bv = {fb[j][0], fb[j][1], fb[j][2], fb[j][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0,
                                                                     sa[i], 0, sb[j]);
      }
    }
  };

#pragma unroll
  for (int sidx = 0; sidx < STAGES; ++sidx)
    if (sidx < nkt) issue(sidx, stage(sidx));
  if (nkt >= STAGES)
    wait_vmcnt<(STAGES - 1) * RUNS_PER_WAVE>();
  else
    wait_vmcnt<0>();
  stage_barrier();
  i32x4 fa0[TM], fa1[TM], fb0[TN], fb1[TN];
  int sa0[TM], sa1[TM], sb0[TN], sb1[TN];
  read_frags(stage(0), fa0, fb0, sa0, sb0);

  auto iterate = [&](int kt, int sbuf, i32x4 (&fac)[TM], i32x4 (&fbc)[TN], int (&sac)[TM],
                     int (&sbc)[TN], i32x4 (&fan)[TM], i32x4 (&fbn)[TN], int (&san)[TM],
                     int (&sbn)[TN]) {
    if (kt + STAGES <= nkt)
      wait_vmcnt<(STAGES - 2) * RUNS_PER_WAVE>();
    else
      wait_vmcnt<0>();
    stage_barrier();
    if (kt + STAGES < nkt) issue(kt + STAGES, stage(sbuf));
    read_frags(stage((sbuf + 1) % STAGES), fan, fbn, san, sbn);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
    compute(fac, fbc, sac, sbc);
  };
  // (A branch-free copy of the steady iterations, as in the int4 kernel,
  // does not fit this kernel's registers at two waves per SIMD.)
  for (int kt0 = 0; kt0 < nkt; kt0 += 2 * STAGES) {
#pragma unroll
    for (int u = 0; u < 2 * STAGES; ++u) {
      const int kt = kt0 + u;
      if (kt < nkt) {
        if (u & 1)
          iterate(kt, u % STAGES, fa1, fb1, sa1, sb1, fa0, fb0, sa0, sb0);
        else
          iterate(kt, u % STAGES, fa0, fb0, sa0, sb0, fa1, fb1, sa1, sb1);
      }
    }
  }

  const int64_t mlane = m0 + wm0 + (lane >> 4) * 4;
  const int64_t nlane = n0 + wn0 + (lane & 15);
  const bool interior = (m0 + BM <= a.M) && (n0 + BN <= a.N);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t n = nlane + j * 16;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      f32x4 yv = acc[i][j];
      if constexpr (LRMODE != LR_NONE)
        yv = add_lowrank<LRMODE>(a, yv, m0 + wm0 + i * 16, n0 + wn0 + j * 16, lane);
      const int64_t mb = mlane + i * 16;
      if (interior) {
        float* yp = a.y + mb * a.N + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) yp[r * a.N] = yv[r];
      } else if (n < a.N) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mb + r < a.M) a.y[(mb + r) * a.N + n] = yv[r];
      }
    }
  }
}

// Small M: 16 output columns per workgroup, KW waves split K.  MB row blocks
// of 16 cover M <= 16 * MB.  Every lane loads, per 128-code K pair t, the 16
// bytes [64t + 16g, 64t + 16g + 16) of its weight row (g = lane >> 4) and of
// its activation rows; K step 0 of the pair uses the first 8 bytes and K
// step 1 the last 8, identically on both sides.
template <int MB, int KW, bool GROUPED, int LRMODE, bool AI8, bool TILED>
__global__ void __launch_bounds__(64 * KW) qgemm_skinny_kernel(GemmArgs a) {
  constexpr int CH = 8;  // K pairs loaded per batch
  __shared__ i32x4 ired[KW][MB][64];
  __shared__ f32x4 fred[GROUPED ? KW : 1][GROUPED ? MB : 1][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t row_bytes = a.K / 2;
  const int64_t npairs = (a.K + 127) / 128;
  const int g = lane >> 4;
  const int64_t nrow = n0 + (lane & 15);
  const bool n_ok = nrow < a.N;
  const bool want_y = a.y != nullptr;
  const int64_t ngroups = GROUPED ? a.K / a.group : 1;
  const int64_t pairs_per_group = GROUPED ? a.group / 128 : 1;

  // Contiguous pair range of this wave.
  const int64_t p_begin = npairs * wave / KW;
  const int64_t p_end = npairs * (wave + 1) / KW;

  // The epilogue waves load their scales and low-rank operands first, so
  // that these loads overlap the weight stream instead of following it.  The
  // scales are loaded as raw bits from clamped indices, unconditionally, and
  // converted and masked only in the epilogue: arithmetic on them here (or a
  // select of the loaded value) made the wave wait for each load in turn
  // before issuing its weight loads, about 1 us per launch.
  uint32_t sx_bits[4] = {0u, 0u, 0u, 0u};
  uint32_t sw_bits = 0u;
  LowRankPre lrp;
  if (wave < MB && want_y) {
    const int64_t mblk = wave * 16;
    const int64_t n = n0 + (lane & 15);
    const int64_t nc = n < a.N ? n : a.N - 1;
    if (!GROUPED) {
      if (a.sw_f16)
        sw_bits = reinterpret_cast<const uint16_t*>(a.sw)[nc];
      else
        sw_bits = reinterpret_cast<const uint32_t*>(a.sw)[nc];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = mblk + (lane >> 4) * 4 + r;
      sx_bits[r] = reinterpret_cast<const uint32_t*>(a.sx)[m < a.M ? m : a.M - 1];
    }
    if constexpr (LRMODE == LR_F16) load_lowrank_pre(a, mblk, n0, lane, lrp);
  }

  i32x4 acc[MB];
  f32x4 facc[GROUPED ? MB : 1];
  i32x4 full[GROUPED ? MB : 1];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = i32x4{0, 0, 0, 0};
  if constexpr (GROUPED) {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      facc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      full[b] = i32x4{0, 0, 0, 0};
    }
  }

  for (int64_t p0 = p_begin; p0 < p_end; p0 += CH) {
    uint4 wv[CH], xv[CH][MB][AI8 ? 2 : 1];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t p = p0 + c;
      if constexpr (TILED) {
        // One contiguous 1 KB block per (16-row block, K pair) and wave.
        const bool ok = p < p_end;
        wv[c] = ok ? *reinterpret_cast<const uint4*>(a.wq + (n0 / 16 * npairs + p) * 1024 + 16 * lane)
                   : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          const int64_t mb = b < (a.M + 15) / 16 ? b : (a.M + 15) / 16 - 1;
          if constexpr (AI8) {  // 2 KB int8 tile
            const uint8_t* xp = a.xq + (mb * npairs + p) * 2048 + 16 * lane;
            xv[c][b][0] = ok ? *reinterpret_cast<const uint4*>(xp) : make_uint4(0, 0, 0, 0);
            xv[c][b][AI8 ? 1 : 0] = ok ? *reinterpret_cast<const uint4*>(xp + 1024) : make_uint4(0, 0, 0, 0);
          } else {  // 1 KB packed tile, the weights' layout
            const uint8_t* xp = a.xq + (mb * npairs + p) * 1024 + 16 * lane;
            xv[c][b][0] = ok ? *reinterpret_cast<const uint4*>(xp) : make_uint4(0, 0, 0, 0);
          }
        }
      } else {
        const int64_t kb = p * 64 + g * 16;
        const bool ok = p < p_end && kb < row_bytes;
        wv[c] = (ok && n_ok) ? *reinterpret_cast<const uint4*>(a.wq + nrow * row_bytes + kb)
                             : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          const int64_t m = b * 16 + (lane & 15);
          const bool xok = ok && m < a.M;
          if constexpr (AI8) {
            const uint8_t* xp = a.xq + m * a.K + 2 * kb;  // int8 codes [2kb, 2kb + 32)
            xv[c][b][0] = xok ? *reinterpret_cast<const uint4*>(xp) : make_uint4(0, 0, 0, 0);
            xv[c][b][AI8 ? 1 : 0] = xok ? *reinterpret_cast<const uint4*>(xp + 16) : make_uint4(0, 0, 0, 0);
          } else {
            xv[c][b][0] = xok ? *reinterpret_cast<const uint4*>(a.xq + m * row_bytes + kb)
                              : make_uint4(0, 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const i32x4 w0 = (TILED && a.w_ob) ? widen_ob(wv[c].x, wv[c].y) : widen(wv[c].x, wv[c].y);
      const i32x4 w1 = (TILED && a.w_ob) ? widen_ob(wv[c].z, wv[c].w) : widen(wv[c].z, wv[c].w);
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        i32x4 x0, x1;
        if constexpr (AI8) {
          x0 = *reinterpret_cast<const i32x4*>(&xv[c][b][0]);
          x1 = *reinterpret_cast<const i32x4*>(&xv[c][b][AI8 ? 1 : 0]);
        } else {
          x0 = widen(xv[c][b][0].x, xv[c][b][0].y);
          x1 = widen(xv[c][b][0].z, xv[c][b][0].w);
        }
        acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x0, w0, acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x1, w1, acc[b], 0, 0, 0);
      }
      if constexpr (GROUPED) {
        const int64_t p = p0 + c;
        if (p < p_end && (p + 1) % pairs_per_group == 0) {
          const int64_t grp = p / pairs_per_group;
          const float sw = (want_y && n_ok) ? load_scale(a.sw, nrow * ngroups + grp, a.sw_f16) : 0.f;
#pragma unroll
          for (int b = 0; b < MB; ++b) {
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[b][r] = fmaf(static_cast<float>(acc[b][r]), sw, facc[b][r]);
            full[b] += acc[b];
            acc[b] = i32x4{0, 0, 0, 0};
          }
        }
      }
    }
  }
  if constexpr (GROUPED) {
    // A group straddling this wave's last pair and the next wave's first is
    // flushed by both waves, each with its part of the sum.
    if (p_end > p_begin && p_end % pairs_per_group != 0) {
      const int64_t grp = (p_end - 1) / pairs_per_group;
      const float sw = (want_y && n_ok) ? load_scale(a.sw, nrow * ngroups + grp, a.sw_f16) : 0.f;
#pragma unroll
      for (int b = 0; b < MB; ++b) {
#pragma unroll
        for (int r = 0; r < 4; ++r) facc[b][r] = fmaf(static_cast<float>(acc[b][r]), sw, facc[b][r]);
        full[b] += acc[b];
      }
    }
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      ired[wave][b][lane] = full[b];
      fred[wave][b][lane] = facc[b];
    }
  } else {
#pragma unroll
    for (int b = 0; b < MB; ++b) ired[wave][b][lane] = acc[b];
  }
  __syncthreads();
  if (wave < MB) {
    const int b = wave;
    i32x4 total = ired[0][b][lane];
#pragma unroll
    for (int w = 1; w < KW; ++w) total += ired[w][b][lane];
    f32x4 yv = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t mblk = b * 16;
    if (want_y) {
      f32x4 fsum = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (GROUPED) {
        fsum = fred[0][b][lane];
#pragma unroll
        for (int w = 1; w < KW; ++w) fsum += fred[w][b][lane];
      }
      float sx_pre[4];
      float sw_pre = 1.f;
      if (!GROUPED && n0 + (lane & 15) < a.N)
        sw_pre = a.sw_f16 ? __half2float(__ushort_as_half(static_cast<unsigned short>(sw_bits)))
                          : __uint_as_float(sw_bits);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = mblk + (lane >> 4) * 4 + r;
        sx_pre[r] = m < a.M ? __uint_as_float(sx_bits[r]) * (AI8 ? kInv16 : kInv256) : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        yv[r] = GROUPED ? fsum[r] * sx_pre[r] : static_cast<float>(total[r]) * (sx_pre[r] * sw_pre);
      if constexpr (LRMODE == LR_F16) {
        yv = apply_lowrank_pre(a, lrp, lane, yv);
        yv = add_lowrank<LRMODE>(a, yv, mblk, n0, lane, 32 * LR_PRE);
      } else {
        yv = add_lowrank<LRMODE>(a, yv, mblk, n0, lane);
      }
    }
    store_block(a, mblk, n0, lane, total, yv, AI8 ? 4 : 8);
  }
}

// Small M for the other 4-bit forms (tiled operands, packed codes): the
// skinny kernel's decomposition (16 output columns per workgroup, KW waves
// over contiguous 128-code steps, partials reduced through LDS) with
//   XRES:  the residual steps after the K / 128 main ones, into their own
//          accumulator; total = 8 main + residual;
//   XMX:   MXFP4 codes on the scaled FP4 instruction, scale bytes read per
//          lane beside the code bytes;
//   XASYM: asymmetric activation groups, flushed with per-row scales; the
//          zero-point term sum_g s (z - 8) wsum is a float32 loop in the
//          epilogue (K / group terms per output).
enum SkinnyMode { XRES = 1, XMX = 2, XASYM = 3 };

template <int MB, int KW, int XM, int LRMODE>
__global__ void __launch_bounds__(64 * KW) qgemm_skinny_x_kernel(GemmArgs a) {
  constexpr int CH = 8;  // steps loaded per batch
  constexpr bool FL = XM == XMX || XM == XASYM;  // float partials
  __shared__ i32x4 ired[KW][MB][64];
  __shared__ f32x4 fred[FL ? KW : 1][FL ? MB : 1][64];
  const int lane = threadIdx.x & 63;
  // Wave-uniform by construction: the branches on the step index below
  // (main or residual accumulator) must be scalar branches, because a
  // matrix instruction on the untaken side of an EXEC-masked branch would
  // still execute.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int nkt = static_cast<int>(a.K / 128);                  // code steps
  const int nsteps = nkt + (XM == XRES ? a.res_iters : 0);       // weight steps
  const int64_t nrow = n0 + (lane & 15);
  const bool n_ok = nrow < a.N;
  const bool want_y = a.y != nullptr;
  const int64_t mlast = (a.M + 15) / 16 - 1;
  const int ipg = XM == XASYM ? a.agroup / 128 : 1;              // steps per group
  const int G = XM == XASYM ? nkt / ipg : 1;

  const int p_begin = static_cast<int>(static_cast<int64_t>(nsteps) * wave / KW);
  const int p_end = static_cast<int>(static_cast<int64_t>(nsteps) * (wave + 1) / KW);

  // The epilogue waves load their scales and low-rank operands first, as
  // raw bits from clamped indices (the skinny kernel's rule), so that these
  // loads overlap the weight stream instead of following it.
  uint32_t sw_bits = 0u;
  uint32_t sx_bits[4] = {0u, 0u, 0u, 0u};
  LowRankPre lrp;
  if (wave < MB && want_y) {
    const int64_t mblk = wave * 16;
    const int64_t nc = nrow < a.N ? nrow : a.N - 1;
    if constexpr (XM != XMX) {
      if (a.sw_f16)
        sw_bits = reinterpret_cast<const uint16_t*>(a.sw)[nc];
      else
        sw_bits = reinterpret_cast<const uint32_t*>(a.sw)[nc];
    }
    if constexpr (XM == XRES) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = mblk + (lane >> 4) * 4 + r;
        sx_bits[r] = reinterpret_cast<const uint32_t*>(a.sx)[m < a.M ? m : a.M - 1];
      }
    }
    if constexpr (LRMODE == LR_F16) load_lowrank_pre(a, mblk, n0, lane, lrp);
  }

  i32x4 acc[MB], accr[XM == XRES ? MB : 1];
  f32x4 facc[FL ? MB : 1];
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    acc[b] = i32x4{0, 0, 0, 0};
    if constexpr (XM == XRES) accr[b] = i32x4{0, 0, 0, 0};
    if constexpr (FL) facc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // One batch of steps (weights, codes and, for MXFP4, their scale bytes)
  // into registers.  The first batch is issued before the asymmetric groups'
  // staging below, so that the weights are in flight during its round trip.
  uint4 wv[CH], xv[CH][MB];
  int ws_[XM == XMX ? CH : 1], xs_[XM == XMX ? CH : 1][MB];
  auto load_batch = [&](int p0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int p = p0 + c;
      const bool ok = p < p_end;
      const int pa = (XM == XRES && p >= nkt) ? p - nkt : p;     // code step
      wv[c] = ok ? *reinterpret_cast<const uint4*>(a.wq + (n0 / 16 * nsteps + p) * 1024 + 16 * lane)
                 : make_uint4(0, 0, 0, 0);
      if constexpr (XM == XMX)
        ws_[c] = ok ? a.mx_ws[(n0 / 16 * nkt + p) * 64 + (lane >> 4) * 16 + (lane & 15)] : 127;
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const int64_t mb = b < mlast ? b : mlast;
        xv[c][b] = ok ? *reinterpret_cast<const uint4*>(a.xq + (mb * nkt + pa) * 1024 + 16 * lane)
                      : make_uint4(0, 0, 0, 0);
        if constexpr (XM == XMX)
          xs_[c][b] = ok ? a.mx_xs[(mb * nkt + p) * 64 + (lane >> 4) * 16 + (lane & 15)] : 127;
      }
    }
  };
  if (p_begin < p_end) load_batch(p_begin);

  // Asymmetric groups: the rows' scales (times 1/256) and offsets
  // s (z - 8), and the columns' weight sums, staged in LDS as [group][row]
  // and [group][column] before the loop (dynamic LDS of 4 (2 * 16 MB + 16) G
  // bytes), so that neither the flushes nor the epilogue wait on memory.
  extern __shared__ __attribute__((aligned(16))) float xsh[];
  float* s_st = xsh;                         // [G][16 MB]
  float* o_st = xsh + G * 16 * MB;           // [G][16 MB]
  float* w_st = xsh + 2 * G * 16 * MB;       // [G][16]
  if constexpr (XM == XASYM) {
    for (int e = threadIdx.x; e < G * 16 * MB; e += 64 * KW) {
      const int row = e % (16 * MB), gg = e / (16 * MB);
      const bool ok = row < a.M;
      const float sv = ok ? a.sx[row * G + gg] : 0.f;
      s_st[e] = sv * kInv256;
      o_st[e] = ok ? sv * static_cast<float>(a.zx[row * G + gg] - 8) : 0.f;
    }
    for (int e = threadIdx.x; e < G * 16; e += 64 * KW) {
      const int col = e % 16, gg = e / 16;
      const int64_t n = n0 + col;
      w_st[e] = n < a.N ? static_cast<float>(a.wsum[n * G + gg]) : 0.f;
    }
    __syncthreads();
  }
  // asymmetric groups: adds acc * s[m, grp] to facc and clears acc
  auto flush = [&](int grp) {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sv = s_st[grp * 16 * MB + b * 16 + (lane >> 4) * 4 + r];
        facc[b][r] = fmaf(static_cast<float>(acc[b][r]), sv, facc[b][r]);
      }
      acc[b] = i32x4{0, 0, 0, 0};
    }
  };

  for (int p0 = p_begin; p0 < p_end; p0 += CH) {
    if (p0 != p_begin) load_batch(p0);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int p = p0 + c;
      if constexpr (XM == XMX) {
        const i32x8 bv = {static_cast<int>(wv[c].x), static_cast<int>(wv[c].y),
                          static_cast<int>(wv[c].z), static_cast<int>(wv[c].w), 0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          const i32x8 av = {static_cast<int>(xv[c][b].x), static_cast<int>(xv[c][b].y),
                            static_cast<int>(xv[c][b].z), static_cast<int>(xv[c][b].w), 0, 0, 0, 0};
          facc[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, facc[b], 4, 4, 0,
                                                                     xs_[c][b], 0, ws_[c]);
        }
      } else {
        const i32x4 w0 = widen(wv[c].x, wv[c].y);
        const i32x4 w1 = widen(wv[c].z, wv[c].w);
        const bool res_step = XM == XRES && p >= nkt;
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          const i32x4 x0 = widen(xv[c][b].x, xv[c][b].y);
          const i32x4 x1 = widen(xv[c][b].z, xv[c][b].w);
          if (res_step) {
            if constexpr (XM == XRES) {
              accr[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x0, w0, accr[b], 0, 0, 0);
              accr[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x1, w1, accr[b], 0, 0, 0);
            }
          } else {
            acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x0, w0, acc[b], 0, 0, 0);
            acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x1, w1, acc[b], 0, 0, 0);
          }
        }
        if constexpr (XM == XASYM) {
          if (p < p_end && (p + 1) % ipg == 0) flush(p / ipg);
        }
      }
    }
  }
  if constexpr (XM == XASYM) {
    // a group straddling this wave's last step and the next wave's first is
    // flushed by both waves, each with its part of the sum
    if (p_end > p_begin && p_end % ipg != 0) flush((p_end - 1) / ipg);
  }
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    if constexpr (XM == XRES)
      ired[wave][b][lane] = (acc[b] << 3) + accr[b];
    else
      ired[wave][b][lane] = acc[b];
    if constexpr (FL) fred[wave][b][lane] = facc[b];
  }
  __syncthreads();
  if (wave < MB) {
    const int b = wave;
    const int64_t mblk = b * 16;
    i32x4 total = ired[0][b][lane];
#pragma unroll
    for (int w = 1; w < KW; ++w) total += ired[w][b][lane];
    f32x4 fsum = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (FL) {
      fsum = fred[0][b][lane];
#pragma unroll
      for (int w = 1; w < KW; ++w) fsum += fred[w][b][lane];
    }
    f32x4 yv = f32x4{0.f, 0.f, 0.f, 0.f};
    if (want_y) {
      float swn = 1.f;
      if (XM != XMX && n_ok)
        swn = a.sw_f16 ? __half2float(__ushort_as_half(static_cast<unsigned short>(sw_bits)))
                       : __uint_as_float(sw_bits);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = mblk + (lane >> 4) * 4 + r;
        if constexpr (XM == XRES) {
          const float sx = m < a.M ? __uint_as_float(sx_bits[r]) * (kInv256 * 0.125f) : 0.f;
          yv[r] = static_cast<float>(total[r]) * (sx * swn);
        } else if constexpr (XM == XMX) {
          yv[r] = fsum[r];
        } else {
          const int row = b * 16 + (lane >> 4) * 4 + r;
          float corr = 0.f;
          for (int gg = 0; gg < G; ++gg)
            corr = fmaf(o_st[gg * 16 * MB + row], w_st[gg * 16 + (lane & 15)], corr);
          yv[r] = (fsum[r] - corr) * swn;
        }
      }
      if constexpr (LRMODE == LR_F16) {
        yv = apply_lowrank_pre(a, lrp, lane, yv);
        yv = add_lowrank<LRMODE>(a, yv, mblk, n0, lane, 32 * LR_PRE);
      } else {
        yv = add_lowrank<LRMODE>(a, yv, mblk, n0, lane);
      }
    }
    const int64_t n = n0 + (lane & 15);
    if (n < a.N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = mblk + (lane >> 4) * 4 + r;
        if (m < a.M) {
          if (want_y) a.y[m * a.N + n] = yv[r];
          if (XM == XRES && a.acc) a.acc[m * a.N + n] = total[r] >> 8;
        }
      }
    }
  }
}

template <int MB, int XM>
hipError_t launch_skinny_x(const GemmArgs& a, hipStream_t st) {
  constexpr int KW = 4;
  const dim3 grid(static_cast<unsigned>((a.N + 15) / 16));
  const size_t lds =
      XM == XASYM ? static_cast<size_t>(a.K / a.agroup) * (2 * 16 * MB + 16) * 4 : 0;
#define W4A4_SKX_CASE(LR)                                                                  \
  if (a.lr_mode == LR) {                                                                   \
    hipLaunchKernelGGL((qgemm_skinny_x_kernel<MB, KW, XM, LR>), grid, dim3(64 * KW), lds, \
                       st, a);                                                             \
    return hipGetLastError();                                                              \
  }
  W4A4_SKX_CASE(LR_NONE) W4A4_SKX_CASE(LR_F16) W4A4_SKX_CASE(LR_F32)
#undef W4A4_SKX_CASE
  return hipErrorInvalidValue;
}

template <int XM>
hipError_t launch_skinny_x_m(const GemmArgs& a, hipStream_t st) {
  return a.M <= 16 ? launch_skinny_x<1, XM>(a, st) : launch_skinny_x<2, XM>(a, st);
}

template <int TM, int TN, bool AI8>
hipError_t launch_tiles_a(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = 32 * TM, BN = 32 * TN;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const dim3 grid(static_cast<unsigned>(tiles));
#define W4A4_GEMM_CASE(G, LR)                                                         \
  if ((a.group > 0) == G && a.lr_mode == LR) {                                       \
    hipLaunchKernelGGL((qgemm_kernel<TM, TN, G, LR, AI8>), grid, dim3(256), 0, st, a); \
    return hipGetLastError();                                                         \
  }
  W4A4_GEMM_CASE(false, LR_NONE) W4A4_GEMM_CASE(false, LR_F16) W4A4_GEMM_CASE(false, LR_F32)
  W4A4_GEMM_CASE(true, LR_NONE) W4A4_GEMM_CASE(true, LR_F16) W4A4_GEMM_CASE(true, LR_F32)
#undef W4A4_GEMM_CASE
  return hipErrorInvalidValue;
}

template <int TM, int TN>
hipError_t launch_tiles(const GemmArgs& a, hipStream_t st) {
  return a.a_i8 ? launch_tiles_a<TM, TN, true>(a, st) : launch_tiles_a<TM, TN, false>(a, st);
}

template <int TM, int TN, int STAGES>
hipError_t launch_pipe(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = 32 * TM, BN = 32 * TN;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const dim3 grid(static_cast<unsigned>(tiles));
  // Grouped: the tile's scales for all groups in dynamic LDS.
  const size_t scale_lds =
      a.group > 0 ? static_cast<size_t>(BN) * (a.K / a.group) * (a.sw_f16 ? 2 : 4) : 0;
  if (a.ob_sa) {  // offset-binary packed codes and weights, per-channel scales
    if constexpr (TM == 4 && TN == 4 && STAGES == 4) {
      if (a.lr_mode == LR_F16)
        hipLaunchKernelGGL((qgemm_pipe_kernel<TM, TN, STAGES, false, LR_F16, true, true, false,
                                              false, false, false, true>), grid, dim3(256), 0, st, a);
      else if (a.lr_mode == LR_F32)
        hipLaunchKernelGGL((qgemm_pipe_kernel<TM, TN, STAGES, false, LR_F32, true, true, false,
                                              false, false, false, true>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((qgemm_pipe_kernel<TM, TN, STAGES, false, LR_NONE, true, true, false,
                                              false, false, false, true>), grid, dim3(256), 0, st, a);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
#define W4A4_PIPE_CASE(G, LR, T, P)                                                          \
  if ((a.group > 0) == G && a.lr_mode == LR && (a.tiled != 0) == T && (!a.a_i8) == P) {      \
    if (G && P && a.group == 128)                                                           \
      hipLaunchKernelGGL((qgemm_pipe_kernel<TM, TN, STAGES, G, LR, T, P, false, G && P>),   \
                         grid, dim3(256), scale_lds, st, a);                                \
    else                                                                                    \
      hipLaunchKernelGGL((qgemm_pipe_kernel<TM, TN, STAGES, G, LR, T, P>), grid, dim3(256), \
                         scale_lds, st, a);                                                 \
    return hipGetLastError();                                                               \
  }
#define W4A4_PIPE_CASES(T, P)                                                    \
  W4A4_PIPE_CASE(false, LR_NONE, T, P) W4A4_PIPE_CASE(false, LR_F16, T, P)       \
  W4A4_PIPE_CASE(false, LR_F32, T, P) W4A4_PIPE_CASE(true, LR_NONE, T, P)        \
  W4A4_PIPE_CASE(true, LR_F16, T, P) W4A4_PIPE_CASE(true, LR_F32, T, P)
  W4A4_PIPE_CASES(false, false) W4A4_PIPE_CASES(true, false) W4A4_PIPE_CASES(true, true)
#undef W4A4_PIPE_CASES
#undef W4A4_PIPE_CASE
  return hipErrorInvalidValue;
}

// Asymmetric activation groups: packed tiled codes, tiled weights.  Dynamic
// LDS: the row scales of every group and the row maxima.
template <int TM, int TN, int STAGES>
hipError_t launch_pipe_asym(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = 32 * TM, BN = 32 * TN;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const dim3 grid(static_cast<unsigned>(tiles));
  if (a.agroup == a.K && a.lr_mode == LR_NONE) {
    // One group per row: the symmetric kernel's 128 x 128 tile, no flush.
    // (With a low-rank term this tile would drop to one wave per SIMD.)
    constexpr int BM1 = 128, BN1 = 128;
    const dim3 grid1(static_cast<unsigned>(((a.M + BM1 - 1) / BM1) * ((a.N + BN1 - 1) / BN1)));
    hipLaunchKernelGGL((qgemm_pipe_kernel<4, 4, STAGES, false, LR_NONE, true, true, true, false,
                                          true>), grid1, dim3(256), BM1 * 4, st, a);
    return hipGetLastError();
  }
  const size_t lds = static_cast<size_t>(BM) * (a.K / a.agroup) * 4 + BM * 4;
#define W4A4_ASYM_CASE(LR, G1)                                                               \
  if (a.lr_mode == LR && (a.agroup == 128) == G1) {                                          \
    hipLaunchKernelGGL((qgemm_pipe_kernel<TM, TN, STAGES, false, LR, true, true, true, G1>), \
                       grid, dim3(256), lds, st, a);                                         \
    return hipGetLastError();                                                                \
  }
  W4A4_ASYM_CASE(LR_NONE, true) W4A4_ASYM_CASE(LR_F16, true) W4A4_ASYM_CASE(LR_F32, true)
  W4A4_ASYM_CASE(LR_NONE, false) W4A4_ASYM_CASE(LR_F16, false) W4A4_ASYM_CASE(LR_F32, false)
#undef W4A4_ASYM_CASE
  return hipErrorInvalidValue;
}

template <int MB, bool AI8, bool TILED>
hipError_t launch_skinny_a(const GemmArgs& a, hipStream_t st) {
  constexpr int KW = 4;
  const dim3 grid(static_cast<unsigned>((a.N + 15) / 16));
#define W4A4_SKINNY_CASE(G, LR)                                                              \
  if ((a.group > 0) == G && a.lr_mode == LR) {                                                \
    hipLaunchKernelGGL((qgemm_skinny_kernel<MB, KW, G, LR, AI8, TILED>), grid, dim3(64 * KW), \
                       0, st, a);                                                             \
    return hipGetLastError();                                                                \
  }
  W4A4_SKINNY_CASE(false, LR_NONE) W4A4_SKINNY_CASE(false, LR_F16) W4A4_SKINNY_CASE(false, LR_F32)
  W4A4_SKINNY_CASE(true, LR_NONE) W4A4_SKINNY_CASE(true, LR_F16) W4A4_SKINNY_CASE(true, LR_F32)
#undef W4A4_SKINNY_CASE
  return hipErrorInvalidValue;
}

template <int MB>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t st) {
  if (a.tiled)
    return a.a_i8 ? launch_skinny_a<MB, true, true>(a, st) : launch_skinny_a<MB, false, true>(a, st);
  return a.a_i8 ? launch_skinny_a<MB, true, false>(a, st) : launch_skinny_a<MB, false, false>(a, st);
}

}  // namespace

// In-GEMM residual: the 128 x 128 tile, packed tiled codes.
static hipError_t launch_pipe_res(const GemmArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(((a.M + 127) / 128) * ((a.N + 127) / 128)));
  hipLaunchKernelGGL((qgemm_pipe_kernel<4, 4, 3, false, LR_NONE, true, true, false, false, false,
                                        true>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

static hipError_t launch_qgemm_mx(const GemmArgs& a, hipStream_t st) {
  constexpr int WGM = 2;  // 8 waves (256 x 128) read less but ran no faster on square shapes
  const dim3 grid(static_cast<unsigned>(((a.M + 64 * WGM - 1) / (64 * WGM)) * ((a.N + 127) / 128)));
#define W4A4_MX_CASE(LR)                                                                      \
  if (a.lr_mode == LR) {                                                                      \
    hipLaunchKernelGGL((qgemm_mx_kernel<4, 4, 4, LR, WGM>), grid, dim3(128 * WGM), 0, st, a); \
    return hipGetLastError();                                                                 \
  }
  W4A4_MX_CASE(LR_NONE) W4A4_MX_CASE(LR_F16) W4A4_MX_CASE(LR_F32)
#undef W4A4_MX_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_qgemm(const GemmArgs& a, hipStream_t st) {
  if (a.f6) return launch_qgemm_f6(a, st);
  // Decode-sized calls of the other 4-bit forms take the skinny decomposition.
  if (a.M <= 32) {
    if (a.mx_xs) return launch_skinny_x_m<XMX>(a, st);
    if (a.res) return launch_skinny_x_m<XRES>(a, st);
    if (a.zx) return launch_skinny_x_m<XASYM>(a, st);
  }
  if (a.mx_xs) return launch_qgemm_mx(a, st);
  if (a.res) return launch_pipe_res(a, st);
  // Asymmetric groups: a 32 x 64 wave tile, so that the row scales of every
  // group fit in LDS beside two workgroups per CU.
  if (a.zx) return launch_pipe_asym<2, 4, 3>(a, st);
  // The skinny kernel flushes weight groups at 128-code granularity.
  // (offset-binary codes take the tiled kernel at any M)
  const bool skinny_ok = (a.group == 0 || a.group % 128 == 0) && !a.ob_sa;
  if (a.M <= 16 && skinny_ok) return launch_skinny<1>(a, st);
  if (a.M <= 32 && skinny_ok) return launch_skinny<2>(a, st);
  // The tiled kernels write the int32 product only when ungrouped: a grouped
  // request for acc runs the ungrouped kernel for it (the integer product
  // does not depend on the weight groups).
  if (a.group > 0 && a.acc) {
    GemmArgs ia = a;
    ia.group = 0;
    ia.y = nullptr;
    ia.lr_mode = LR_NONE;
    hipError_t e = !a.tiled ? launch_tiles<4, 4>(ia, st)
                   : ia.a_i8 ? launch_pipe<4, 4, 3>(ia, st)
                             : launch_pipe<4, 4, 4>(ia, st);
    if (e != hipSuccess) return e;
    if (!a.y) return hipSuccess;
  }
  GemmArgs ya = a;
  if (a.group > 0) ya.acc = nullptr;
  // int8 codes, whole 128-code iterations: the pipelined direct-to-LDS kernel
  // (the only one that reads tiled operands).
  if (a.tiled || (a.a_i8 && a.K % 128 == 0 && a.group % 128 == 0)) {
    // Grouped: a 64 x 32 wave tile, so that the float group accumulators fit
    // beside the integer ones at two waves per SIMD.
    // Four stages for packed codes (2 x 64 KB of LDS per CU); int8 codes
    // double the activation tile, and four of their stages would leave one
    // workgroup per CU.
    if (ya.group > 0) return launch_pipe<4, 2, 3>(ya, st);
    return ya.a_i8 ? launch_pipe<4, 4, 3>(ya, st) : launch_pipe<4, 4, 4>(ya, st);
  }
  const int64_t big_tiles = ((a.M + 255) / 256) * ((a.N + 127) / 128);
  if (a.group == 0 && a.M >= 256 && big_tiles >= 200) return launch_tiles<8, 4>(ya, st);
  return launch_tiles<4, 4>(ya, st);
}

}  // namespace w4a4
