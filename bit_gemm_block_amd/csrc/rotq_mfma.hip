// rotq_mfma.hip — block Hadamard rotation (128 <= b <= 4096) on the fp16
// matrix instruction, fused with per-token absmax int4 quantization into the
// tiled code layouts of the layer: FP6 E2M3 tiles, or packed nibble tiles
// (plain or offset-binary, with the row sums of the odd channels' codes)
// (SERQ page, "Resumen técnico" §1-2: rotate, then quantize each token on the
// fly).
//
// The 128-point part: the rotation of 16 blocks of 128 is one product
// H [128 x 128] . X^T [128 x 16] of exact fp16 operands (fp16 X, H = +-1, the
// Sylvester matrix) with float32 accumulation, 32 instructions of
// v_mfma_f32_16x16x32_f16 (22 after the compiler shares chain prefixes),
// where butterflies would take 7 VALU instructions per element.  Wave w of
// a row's workgroup takes its elements [2048 w, 2048 w + 2048) as sixteen
// blocks c of 128:
//   * operand B of K-step kc: lane 16 g + c holds x[128 c + 32 kc + 8 g, +8)
//     (one 16-byte load);
//   * operand A of output block mb, K-step kc: lane 16 g + r holds
//     H[16 mb + r][32 kc + 8 g + t], t < 8, which splits into a per-lane
//     part and signs: with i = 16 mb + r and k = 32 kc + 8 g + t, i & k
//     keeps r & t (bits 0-2), r3 & g0 (bit 3), mb0 & g1 (bit 4) and
//     mb1 & kc0, mb2 & kc1 (bits 5-6), so A = +-(mb0 ? F1 : F0) with F0, F1
//     built once per lane;
//   * output: lane 16 g + c holds y_c[16 mb + 4 g + i'], i' < 4.
//
// Larger blocks, b = 128 n with n = 2^P sub-blocks (2 <= n <= 32):
// Sylvester's construction gives H_b = H_n (x) H_128 (entry
// (128 j + e, 128 j' + e') is (-1)^(j.j') (-1)^(e.e')), so the rotation is the
// 128-point transform of every sub-block, then the n-point transform across
// the sub-blocks at each of the 128 positions.  Sub-block bits 0-3 lie in the
// lane column; for n = 32, bit 4 pairs waves 2 v and 2 v + 1, which exchange
// their products through LDS.  A lane stage is one v_fmac_f32_dpp per value,
// v += sgn * v[partner], the partner read through a lane permutation within
// each 16-lane row: xor 1 and xor 2 (quad permutations), xor 7 (half-row
// mirror), xor 8 (row rotation by 8).  (A uniform add or subtract gives both
// lanes of a pair the same linear form of their two values; the per-lane sign
// gives the low lane the sum and the high lane the difference, negated.)
// With partner masks 1, 2, 7, 8 the stages are the Walsh-Hadamard butterflies
// in the coordinates of the column index over the basis {1, 2, 7, 8}: a
// lane's sign at stage s is its s-th coordinate, the product is H_16 with its
// columns permuted by the Gram matrix of the basis, and loading sub-block
// pi(c) into column c undoes that permutation.  At the end a lane holds its
// outputs times (-1)^(sum of its coordinates); the quantizer takes that sign
// back out.  The host derives pi, the coordinates and the final signs from
// the four masks.
//
// Then x~ = RN(y / sqrt(b)) as y * rs, s = RN(max|x~| / 7), and each code is
// x~ * RN(1 / s) rounded once to an integer.  The row's absmax is reduced
// over lanes and waves.  For the tiles, lane 16 j + c must hold the 32
// consecutive codes [32 j, 32 j + 32) of block c, which lane groups
// g = 0..3 hold 8 each (mb = 2 j, 2 j + 1): a 4 x 4 transpose of 8-value
// units across the lane groups, by v_permlane32_swap (lane groups 0,1 <->
// 2,3) then v_permlane16_swap (0 <-> 1, 2 <-> 3).
#include "rotq_mfma.h"

#include <hip/hip_fp16.h>

#include "lowrank_rows.h"

namespace w4a4 {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: x + kMagic - kMagic = rint(x) for |x| < 2^22

struct RotArgs {
  const _Float16* x;  // [M, K]
  int64_t M, K;
  float rs;           // float32(1 / sqrt(b))
  float qmax;         // largest code: 7, or 127 for int8 tiles
  float sqrt_b;       // sqrt(b) when it is a power of two (the divisor fold)
  uint8_t* q;         // the code tiles
  float* scale;       // [M]
  int32_t* ob_sum;    // offset-binary packed tiles: [M] sums of the odd channels' codes
  uint8_t* mx_scale;  // MXFP4: E8M0 scale bytes, 64 per 16 x 128 tile
  int32_t* zero;      // asymmetric codes: zero points [M, K / 128] (scale: [M, K / 128])
  // Decode launches (ROLES): blocks [0, M) take row blockIdx.x, then lr_rank
  // blocks compute column j of T = X . A, then ra.blocks read the weights
  // ahead; every block has 256 threads.
  const _Float16* lr_at;
  int lr_rank;
  void* lr_t;
  ReadAhead ra;
  int64_t tile_stride;   // tiles per 16-row block (K / 128)
  int64_t rows_per_xcd;  // a multiple of 16
  uint64_t pi_tbl;    // 4 bits per lane column c: the sub-block that column c loads
  uint64_t sel_tbl;   // 4 bits per column: bit s is the column's sign at lane stage s
  uint32_t sig_tbl;   // bit c: column c holds its outputs negated after the stages
};

// Output layouts.
enum { OUT_F6 = 0, OUT_PACKED = 1, OUT_PACKED_OB = 2, OUT_MX = 3, OUT_I8 = 4, OUT_ASYM = 5 };

template <int OUT>
constexpr int64_t kTileBytes = OUT == OUT_F6 ? 1536 : OUT == OUT_I8 ? 2048 : 1024;

__device__ __forceinline__ h8 neg8(h8 v) {
  h8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = -v[t];
  return r;
}

// The +-1 operands A of the 128-point transform: F0[t] is the Hadamard sign
// of (r & t) and (r3 & g0); F1 adds (g1) for odd output blocks; N0, N1 their
// negations.
struct HFrag {
  h8 f0, f1, n0, n1;
};

__device__ __forceinline__ HFrag h128_fragments(int lane) {
  const int g = lane >> 4, r = lane & 15;
  HFrag f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int par = (__builtin_popcount(r & t & 7) + ((r >> 3) & g & 1)) & 1;
    f.f0[t] = par ? static_cast<_Float16>(-1.0f) : static_cast<_Float16>(1.0f);
    f.f1[t] = ((g >> 1) & 1) ? -f.f0[t] : f.f0[t];
  }
  f.n0 = neg8(f.f0);
  f.n1 = neg8(f.f1);
  return f;
}

// acc[mb]: lane 16 g + c holds y_c[16 mb + 4 g + i], y_c = H x_c, for the 16
// blocks whose operand B xb this lane holds.
__device__ __forceinline__ void h128_product(const HFrag& f, const h8 (&xb)[4], f4 (&acc)[8]) {
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    acc[mb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bool neg = (((mb >> 1) & kc & 1) ^ ((mb >> 2) & (kc >> 1) & 1)) != 0;
      const h8 av = (mb & 1) ? (neg ? f.n1 : f.f1) : (neg ? f.n0 : f.f0);
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, xb[kc], acc[mb], 0, 0, 0);
    }
  }
}

// Reductions over the 64 lanes of a wave without LDS round trips: within each
// 16-lane row, data-parallel moves pair each lane with lane ^ 1, lane ^ 2,
// its half-row mirror (lane ^ 7) and its row mirror (lane ^ 15), each step
// joining two disjoint groups whose lanes agree; then the 32- and 16-lane
// swaps of the value with itself join the four rows.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true));
}

template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  auto bits = [](T x) { return __builtin_bit_cast(uint32_t, x); };
  auto val = [](uint32_t x) { return __builtin_bit_cast(T, x); };
  v = op(v, val(dpp_mov<0xB1>(bits(v))));   // quad_perm [1,0,3,2]
  v = op(v, val(dpp_mov<0x4E>(bits(v))));   // quad_perm [2,3,0,1]
  v = op(v, val(dpp_mov<0x141>(bits(v))));  // row_half_mirror
  v = op(v, val(dpp_mov<0x140>(bits(v))));  // row_mirror
  const auto s32 = __builtin_amdgcn_permlane32_swap(bits(v), bits(v), false, false);
  v = op(val(s32[0]), val(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(bits(v), bits(v), false, false);
  return op(val(s16[0]), val(s16[1]));
}

// Maximum over the W waves of a row.
template <int W>
__device__ __forceinline__ float row_max(float m, float* wmax, int lane, int w) {
  m = wave_reduce(m, [](float x, float y) { return fmaxf(x, y); });
  if (W > 1) {
    if (lane == 0) wmax[w] = m;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < W; ++v) m = fmaxf(m, wmax[v]);
  }
  return m;
}

template <int W>
__device__ __forceinline__ int row_sum(int os, int* wsum, int lane, int w) {
  os = wave_reduce(os, [](int x, int y) { return x + y; });
  if (W > 1) {
    if (lane == 0) wsum[w] = os;
    __syncthreads();
    os = 0;
#pragma unroll
    for (int v = 0; v < W; ++v) os += wsum[v];
  }
  return os;
}

// Writes the codes of the 16 blocks of one product into their tiles.  cm[mb][i]
// holds the code q of y_c[16 mb + 4 g + i] in the form its tile takes: q as a
// float for FP6 (the packing instruction's input), q + 1.5 * 2^23 for the
// nibble and byte tiles (whose low nibble or byte is q in two's complement).  Returns, for
// offset-binary tiles, this lane's sum of the codes at odd channels.
// The 4 x 4 unit transpose across the lane groups.  in[mb][i] is this lane's
// value at position 16 mb + 4 g + i of its block; unit j (the 8 values of
// chunk j: mb = 2 j + v / 4, i = v % 4) goes to lane group j.  After the two
// swaps, b[s][v] is unit (this lane group) of source group s, and this lane
// holds positions [32 g, 32 g + 32) of its block, chunk offset
// 16 (v / 4) + 4 s + v % 4 in b[s][v].
__device__ __forceinline__ void unit_transpose(const float (&in)[8][4], uint32_t (&b)[4][8]) {
  uint32_t u[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 8; ++v) u[j][v] = __float_as_uint(in[2 * j + (v >> 2)][v & 3]);
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const auto s02 = __builtin_amdgcn_permlane32_swap(u[0][v], u[2][v], false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(u[1][v], u[3][v], false, false);
    const auto t01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    const auto t23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    b[0][v] = t01[0];
    b[1][v] = t01[1];
    b[2][v] = t23[0];
    b[3][v] = t23[1];
  }
}

template <int OUT>
__device__ __forceinline__ int store_codes(const float (&cm)[8][4], uint8_t* tile, int g, int rin) {
  uint32_t b[4][8];
  unit_transpose(cm, b);
  if constexpr (OUT == OUT_I8) {
    // The 2 KB int8 tile: codes [32 g + 16 h, +16) of row r are the 16 bytes
    // at ((4 h + g) 16 + r) 16, each group of 8 in the order 0,2,4,6,1,3,5,7.
    // Element e of group q of half h is chunk offset 16 h + 8 q + e, that is
    // b[2 q + e / 4][4 h + e % 4]: dword 2 q takes e = 0, 2, 4, 6 and dword
    // 2 q + 1 takes e = 1, 3, 5, 7.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t d[4];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
          const uint32_t lo = __builtin_amdgcn_perm(b[2 * q][4 * h + 2 + odd], b[2 * q][4 * h + odd], 0x0C0C0400u);
          const uint32_t hi =
              __builtin_amdgcn_perm(b[2 * q + 1][4 * h + 2 + odd], b[2 * q + 1][4 * h + odd], 0x04000C0Cu);
          d[2 * q + odd] = lo | hi;
        }
      *reinterpret_cast<uint4*>(tile + ((4 * h + g) * 16 + rin) * 16) = make_uint4(d[0], d[1], d[2], d[3]);
    }
    return 0;
  } else if constexpr (OUT == OUT_F6) {
    // lane 16 g + (row % 16) of the 1536-byte FP6 tile
    f16v lo, hi;
#pragma unroll
    for (int sg = 0; sg < 4; ++sg)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lo[4 * sg + t] = __uint_as_float(b[sg][t]);
        hi[4 * sg + t] = __uint_as_float(b[sg][4 + t]);
      }
    const auto p = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(lo, hi, 1.0f);
    const int l6 = 16 * g + rin;
    *reinterpret_cast<uint4*>(tile + 16 * l6) = make_uint4(p[0], p[1], p[2], p[3]);
    *reinterpret_cast<uint2*>(tile + 1024 + 8 * l6) = make_uint2(p[4], p[5]);
    return 0;
  } else {
    // Nibble 8 d + e of the lane's 16 bytes is chunk offset 8 d + e: dword d
    // takes B[2 (d % 2) + e / 4][4 (d / 2) + e % 4]; the 16 bytes go to
    // lane 16 g + (row % 16) of the 1 KB tile.
    uint32_t pk[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t v = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v = __builtin_amdgcn_alignbit(b[2 * (d & 1) + (e >> 2)][4 * (d >> 1) + (e & 3)], v, 4);
      pk[d] = v;
    }
    int os = 0;
    if constexpr (OUT == OUT_PACKED_OB) {
      // The codes at odd channels (the high nibbles, as int8 16 q), then the
      // low nibbles offset by 8.
      int os16 = 0;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        os16 = __builtin_amdgcn_sdot4(static_cast<int>(pk[d] & 0xF0F0F0F0u), 0x01010101, os16, false);
      os = os16 >> 4;
#pragma unroll
      for (int d = 0; d < 4; ++d) pk[d] ^= 0x08080808u;
    }
    *reinterpret_cast<uint4*>(tile + (16 * g + rin) * 16) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    return os;
  }
}

// One lane stage over the 32 values: v += sgn * v[lane ^ mask] within each
// 16-lane row.  Inline asm, since the compiler splits the permuted operand into
// a separate move; the s_nop covers the two wait states that a permuted read
// needs after the VALU write of its register.
#define W4A4_FMAC_DPP8(CTRL, V, SG)                                                 \
  asm("s_nop 1\n\t"                                                                 \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"               \
      : "+v"((V)[0]), "+v"((V)[1]), "+v"((V)[2]), "+v"((V)[3]), "+v"((V)[4]),      \
        "+v"((V)[5]), "+v"((V)[6]), "+v"((V)[7])                                    \
      : "v"(SG))

template <int S>  // partner masks 1, 2, 7, 8
__device__ __forceinline__ void lane_stage(float (&y)[32], int sel) {
  const float sg = ((sel >> S) & 1) ? -1.f : 1.f;
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    float* v = y + k;
    if constexpr (S == 0)
      W4A4_FMAC_DPP8("quad_perm:[1,0,3,2]", v, sg);
    else if constexpr (S == 1)
      W4A4_FMAC_DPP8("quad_perm:[2,3,0,1]", v, sg);
    else if constexpr (S == 2)
      W4A4_FMAC_DPP8("row_half_mirror", v, sg);
    else
      W4A4_FMAC_DPP8("row_ror:8", v, sg);
  }
}
#undef W4A4_FMAC_DPP8

// WV waves per row, each taking one chain of 16 sub-blocks, 2048 elements
// (K = 2048 WV); b = 128 * 2^P (P = 0: the 128-point transform alone).  For
// b = 4096 the sub-block bit 4 pairs waves 2 v and 2 v + 1, which exchange
// their products through LDS.  One row per workgroup, all rows launched at
// once.  (At least two waves per SIMD: the register cap keeps the
// accumulators out of the AGPRs, which would take a copy per value.)
template <int WV, int OUT, int P, bool ROLES = false>
__global__ void __launch_bounds__(ROLES ? 256 : 64 * WV, 2) rotq_mfma_kernel(RotArgs a) {
  constexpr int kLaneStages = P < 4 ? P : 4;
  constexpr bool kPair = P == 5;
  // sqrt(b) a power of two: x~ / s = y / (s sqrt(b)) with both sides exact.
  constexpr bool kFold = (P & 1) != 0;
  __shared__ float wmax[WV];
  __shared__ int wsum[WV];
  __shared__ f4 exch[kPair ? WV * 8 * 64 : 1];  // each wave's products, for the pair stage
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  int64_t row;
  if constexpr (ROLES) {
    // Decode launch: the roles after the M rotation blocks (whole workgroups,
    // so no barrier is split), then one row per block.
    __shared__ float role_lds[64];
    if (static_cast<int64_t>(blockIdx.x) >= a.M) {
      const int e = static_cast<int>(blockIdx.x - a.M);
      if (e < a.lr_rank)
        lowrank_rows_body<16>(a.x, a.lr_at, a.M, a.K, a.lr_rank, a.lr_t, 1, e, role_lds);
      else
        read_ahead_role(a.ra, e - a.lr_rank, blockIdx.x, reinterpret_cast<uint32_t*>(role_lds));
      return;
    }
    row = blockIdx.x;
    if (w >= WV) {
      // Waves past the row's: take part in the row's barriers, then leave.
      constexpr int kBarriers = (kPair ? 1 : 0) + (WV > 1 ? 1 : 0) + (OUT == OUT_PACKED_OB && WV > 1 ? 1 : 0);
#pragma unroll
      for (int k = 0; k < kBarriers; ++k) __syncthreads();
      return;
    }
  } else {
    // Workgroup b runs on XCD b % 8 (round robin); each XCD takes a range of
    // whole 16-row blocks, so that every line of a code tile is written from
    // one L2.
    row = (blockIdx.x % 8) * a.rows_per_xcd + blockIdx.x / 8;
    if (row >= a.M) return;
  }
  const int pc = static_cast<int>((a.pi_tbl >> (4 * c)) & 15u);
  const _Float16* src = a.x + row * a.K + 2048 * w + 128 * pc + 8 * g;

  h8 xb[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) xb[kc] = *reinterpret_cast<const h8*>(src + 32 * kc);
  f4 acc[8];
  h128_product(h128_fragments(lane), xb, acc);
  const int sel = static_cast<int>((a.sel_tbl >> (4 * c)) & 15u);
  float y[32];  // y[4 mb + i]

  // The stages across sub-blocks.  The first one after the products is
  // ordinary code, which waits on the matrix results; the inline asm after it
  // reads registers that ordinary VALU code wrote.
  if constexpr (kPair) {
    // bit 4: the even wave of the pair takes the sum, the odd one the
    // difference (even minus odd): own * (+-1) + other
    const float so = (w & 1) ? -1.f : 1.f;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) exch[(w * 8 + mb) * 64 + lane] = acc[mb];
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const f4 o = exch[((w ^ 1) * 8 + mb) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[4 * mb + i] = __builtin_fmaf(acc[mb][i], so, o[i]);
    }
    lane_stage<0>(y, sel);
  } else if constexpr (P >= 1) {
    const float sg = (sel & 1) ? -1.f : 1.f;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = acc[mb][i];
        y[4 * mb + i] = __builtin_fmaf(
            __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)), sg,
            v);  // quad_perm [1,0,3,2]: lane ^ 1
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) y[4 * mb + i] = acc[mb][i];
  }
  if constexpr (kLaneStages > 1) lane_stage<1>(y, sel);
  if constexpr (kLaneStages > 2) lane_stage<2>(y, sel);
  if constexpr (kLaneStages > 3) lane_stage<3>(y, sel);

  if constexpr (OUT == OUT_MX) {
    // MXFP4 (the butterfly kernel's rule): after the unit transpose a lane
    // holds one 32-element block, positions [32 g, 32 g + 32) of sub-block
    // 16 w + c.  e = max(floor(log2(max|x~|)) - 2, -127), max|x~| =
    // RN(max|y| rs); each element x~ 2^-e (exact) to E2M1 by the hardware
    // conversion, with the sign of the quotient.  The lane's sign sgn goes
    // into the multiplier.
    float yv[8][4];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) yv[mb][i] = y[4 * mb + i];
    uint32_t bt[4][8];
    unit_transpose(yv, bt);
    float bm = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int v = 0; v < 8; ++v) bm = fmaxf(bm, fabsf(__uint_as_float(bt[s4][v])));
    const float amax = bm * a.rs;
    const int e = max(static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF) - 129, -127);
    const float sgn = ((a.sig_tbl >> c) & 1u) ? -1.f : 1.f;
    const float srs = sgn * a.rs;
    const float mul = ldexpf(kFold ? srs : 1.f, -e);  // exact: a power of two
    // element o (chunk offset) is bt[(o / 4) % 4][4 (o / 16) + o % 4]; elements
    // 2 k and 2 k + 1 go to byte k of the 16 (low nibble first)
    auto q2 = [&](int o) {
      const int s4 = (o >> 2) & 3, v = 4 * (o >> 4) + (o & 3);
      const float x0 = __uint_as_float(bt[s4][v]), x1 = __uint_as_float(bt[s4][v + 1]);
      return kFold ? float2{x0 * mul, x1 * mul} : float2{(x0 * srs) * mul, (x1 * srs) * mul};
    };
    uint32_t pk[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float2 e0 = q2(8 * d), e1 = q2(8 * d + 2), e2 = q2(8 * d + 4), e3 = q2(8 * d + 6);
      uint32_t v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, e0.x, e0.y, 1.0f, 0);
      v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, e1.x, e1.y, 1.0f, 1);
      v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, e2.x, e2.y, 1.0f, 2);
      pk[d] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, e3.x, e3.y, 1.0f, 3);
    }
    const int rin = static_cast<int>(row & 15);
    const int64_t blk = (row >> 4) * a.tile_stride + 16 * w + c;  // sub-block 16 w + c
    *reinterpret_cast<uint4*>(a.q + blk * 1024 + (16 * g + rin) * 16) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    a.mx_scale[blk * 64 + g * 16 + rin] = static_cast<uint8_t>(e + 127);
    return;
  }

  if constexpr (OUT == OUT_ASYM) {
    // Asymmetric codes of each (row, block of 128) (the butterfly kernel's
    // rule, b = 128): the group is sub-block 16 w + c, which the four lane
    // groups of column c hold, 32 values each.  s = RN((hi - lo) / 15),
    // z = rint(RN(-lo / s)), q = clamp(rint(x~ / s) + z, 0, 15) with the
    // correctly rounded quotient (a large z makes its last bits matter),
    // stored as q - 8; a group without spread spans [min(c, 0), max(c, 0)].
    float ymax = y[0], ymin = y[0];
#pragma unroll
    for (int k = 1; k < 32; ++k) {
      ymax = fmaxf(ymax, y[k]);
      ymin = fminf(ymin, y[k]);
    }
    auto join = [](float v, auto op) {  // over the lanes c, c + 16, c + 32, c + 48
      const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      v = op(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
      const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      return op(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    };
    ymax = join(ymax, [](float p, float q) { return fmaxf(p, q); });
    ymin = join(ymin, [](float p, float q) { return fminf(p, q); });
    float lo = ymin * a.rs, hi = ymax * a.rs;
    if (hi == lo) {
      lo = fminf(lo, 0.f);
      hi = fmaxf(hi, 0.f);
    }
    const float s = __fdiv_rn(hi - lo, 15.f);
    const bool live = s > 0.f;
    const float zf = live ? rintf(__fdiv_rn(-lo, s)) : 0.f;
    const int64_t si = row * (a.K / 128) + 16 * w + c;
    if (g == 0) {
      a.scale[si] = s;
      a.zero[si] = static_cast<int>(zf);
    }
    const float rc = live ? __frcp_rn(s) : 0.f;
    float cm[8][4];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xt = y[4 * mb + i] * a.rs;
        float q = xt * rc;
        q = __builtin_fmaf(__builtin_fmaf(-q, s, xt), rc, q);
        q = __builtin_fmaf(__builtin_fmaf(-q, s, xt), rc, q);
        // rint(q) + z is exact whenever it lands near [0, 15]; farther out
        // the clamp decides.  (q - 8) + 1.5 * 2^23 has q - 8 in its low nibble.
        const float qc = __builtin_amdgcn_fmed3f(rintf(q) + zf, 0.f, 15.f);
        cm[mb][i] = qc + (kMagic - 8.f);
      }
    const int64_t blk = (row >> 4) * a.tile_stride + 16 * w + c;
    store_codes<OUT_PACKED>(cm, a.q + blk * 1024, g, static_cast<int>(row & 15));
    return;
  }

  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) m = fmaxf(m, fabsf(y[k]));
  m = row_max<WV>(m, wmax, lane, w);

  // s = RN(max|x~| / 7) (x~ = RN(y rs) is monotone in |y|); each code is
  // x~ * RN(1 / s) rounded once to an integer (one fma with 1.5 * 2^23, the
  // same instruction for every layout), without the refinement to the
  // correctly rounded quotient: the exact product is within one unit in the
  // last place of the quotient (|q| < 8), below the float32 rounding that the
  // transform's own sums leave in x~, and the quantizer takes one or two
  // instructions per value instead of six.  |q| < 7 (1 + 2^-23), so no clamp.
  // A lane holds its values times sgn; the reciprocal times sgn takes it out
  // (exactly: rounding is symmetric).
  const float amax = m * a.rs;
  const float s = __fdiv_rn(amax, a.qmax);
  if (threadIdx.x == 0) a.scale[row] = s;
  const float sgn = ((a.sig_tbl >> c) & 1u) ? -1.f : 1.f;
  const float rc = s == 0.f ? 0.f : __frcp_rn((kFold ? s * a.sqrt_b : s) * sgn);
  float cm[8][4];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float xt = kFold ? y[4 * mb + i] : y[4 * mb + i] * a.rs;
      const float t = __builtin_fmaf(xt, rc, kMagic);  // 1.5 * 2^23 + code
      cm[mb][i] = OUT == OUT_F6 ? t - kMagic : t;
    }
  const int64_t blk = (row >> 4) * a.tile_stride + 16 * w + c;  // sub-block 16 w + c
  const int os = store_codes<OUT>(cm, a.q + blk * kTileBytes<OUT>, g, static_cast<int>(row & 15));
  if constexpr (OUT == OUT_PACKED_OB) {
    const int tot = row_sum<WV>(os, wsum, lane, w);
    if (threadIdx.x == 0) a.ob_sum[row] = tot;
  }
}

int parity(int v) { return __builtin_popcount(static_cast<unsigned>(v)) & 1; }

// Load permutation, per-stage signs and final signs of the lane stages with
// partner masks 1, 2, 7, 8 (the first `stages` of them, which span the low
// `stages` bits of the column index).
void derive_kron_tables(int stages, RotArgs* a) {
  static constexpr int kMask[4] = {1, 2, 7, 8};
  const int n = 1 << stages;
  int coord[16] = {};
  for (int v = 0; v < n; ++v) {
    int i = 0;
    for (int s = 0; s < stages; ++s)
      if ((v >> s) & 1) i ^= kMask[s];
    coord[i] = v;  // the masks are a basis of [0, n), so each i is hit once
  }
  a->pi_tbl = a->sel_tbl = 0;
  a->sig_tbl = 0;
  for (int c = 0; c < 16; ++c) {
    const int lo = c & (n - 1), hi = c & ~(n - 1);
    int pj = 0;
    for (int j = 0; j < n; ++j) {  // (-1)^(coord(i).coord(lo)) = (-1)^(i.j) for every i
      bool ok = true;
      for (int i = 0; i < n && ok; ++i) ok = parity(coord[i] & coord[lo]) == parity(i & j);
      if (ok) {
        pj = j;
        break;
      }
    }
    a->pi_tbl |= static_cast<uint64_t>(hi | pj) << (4 * c);
    a->sel_tbl |= static_cast<uint64_t>(coord[lo]) << (4 * c);
    a->sig_tbl |= static_cast<uint32_t>(parity(coord[lo])) << c;
  }
}

// The tables for 0-4 stages, derived once.
void kron_tables(int stages, RotArgs* a) {
  struct Tables {
    uint64_t pi[5], sel[5];
    uint32_t sig[5];
  };
  static const Tables t = [] {
    Tables r{};
    for (int n = 0; n < 5; ++n) {
      RotArgs x{};
      derive_kron_tables(n, &x);
      r.pi[n] = x.pi_tbl;
      r.sel[n] = x.sel_tbl;
      r.sig[n] = x.sig_tbl;
    }
    return r;
  }();
  a->pi_tbl = t.pi[stages];
  a->sel_tbl = t.sel[stages];
  a->sig_tbl = t.sig[stages];
}

RotArgs base_args(const _Float16* x, int64_t M, int64_t K, int log2b, uint8_t* q, float* scale,
                  int32_t* ob_sum) {
  RotArgs a{};
  a.x = x;
  a.M = M;
  a.K = K;
  a.rs = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(int64_t{1} << log2b)));
  a.sqrt_b = static_cast<float>(int64_t{1} << (log2b / 2));
  a.q = q;
  a.scale = scale;
  a.ob_sum = ob_sum;
  a.tile_stride = K / 128;
  a.rows_per_xcd = ((M + 15) / 16 + 7) / 8 * 16;
  return a;
}

}  // namespace

bool rotq_mfma_ok(int64_t M, int64_t K, int log2b) {
  const int64_t step = log2b == 12 ? 4096 : 2048;
  return M > 0 && K % step == 0 && K >= step && K <= 16384 && log2b >= 7 && log2b <= 12;
}

hipError_t launch_rotq_mfma(const _Float16* x, int64_t M, int64_t K, int log2b, RotMfmaOut out_kind,
                            int qmax, uint8_t* q, float* scale, int32_t* i32, uint8_t* mx_scale,
                            hipStream_t st) {
  if (!rotq_mfma_ok(M, K, log2b)) return hipErrorInvalidValue;
  if ((out_kind == ROT_OUT_MX) != (mx_scale != nullptr) ||
      (i32 && out_kind != ROT_OUT_PACKED && out_kind != ROT_OUT_ASYM) ||
      (out_kind == ROT_OUT_ASYM && (!i32 || log2b != 7)) ||
      (qmax != 7 && !(qmax == 127 && out_kind == ROT_OUT_I8)))
    return hipErrorInvalidValue;
  RotArgs a = base_args(x, M, K, log2b, q, scale, out_kind == ROT_OUT_PACKED ? i32 : nullptr);
  a.mx_scale = mx_scale;
  a.zero = out_kind == ROT_OUT_ASYM ? i32 : nullptr;
  a.qmax = static_cast<float>(qmax);
  const int p = log2b - 7;  // log2 of the sub-blocks per rotation block
  kron_tables(p < 4 ? p : 4, &a);
  const int WV = static_cast<int>(K / 2048);
  const dim3 grid(static_cast<unsigned>(8 * a.rows_per_xcd));
  const int out = out_kind == ROT_OUT_MX     ? OUT_MX
                  : out_kind == ROT_OUT_F6   ? OUT_F6
                  : out_kind == ROT_OUT_I8   ? OUT_I8
                  : out_kind == ROT_OUT_ASYM ? OUT_ASYM
                  : a.ob_sum                 ? OUT_PACKED_OB
                                             : OUT_PACKED;
#define W4A4_ROT(WW, OO)                                                                          \
  switch (p) {                                                                                     \
    case 0: hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 0>), grid, dim3(64 * WW), 0, st, a); break; \
    case 1: hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 1>), grid, dim3(64 * WW), 0, st, a); break; \
    case 2: hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 2>), grid, dim3(64 * WW), 0, st, a); break; \
    case 3: hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 3>), grid, dim3(64 * WW), 0, st, a); break; \
    case 4: hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 4>), grid, dim3(64 * WW), 0, st, a); break; \
    default:                                                                                       \
      if constexpr (WW % 2 == 0)                                                                   \
        hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 5>), grid, dim3(64 * WW), 0, st, a);          \
      else                                                                                         \
        return hipErrorInvalidValue;                                                               \
      break;                                                                                       \
  }                                                                                                \
  return hipGetLastError();
#define W4A4_ROT_P0(WW, OO)                                                                  \
  hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 0>), grid, dim3(64 * WW), 0, st, a);           \
  return hipGetLastError();
#define W4A4_ROT_W(WW)                        \
  case WW:                                     \
    if (out == OUT_F6) {                       \
      W4A4_ROT(WW, OUT_F6)                    \
    } else if (out == OUT_PACKED) {            \
      W4A4_ROT(WW, OUT_PACKED)                \
    } else if (out == OUT_PACKED_OB) {         \
      W4A4_ROT(WW, OUT_PACKED_OB)             \
    } else if (out == OUT_I8) {                \
      W4A4_ROT(WW, OUT_I8)                    \
    } else if (out == OUT_ASYM) {              \
      W4A4_ROT_P0(WW, OUT_ASYM)               \
    } else {                                   \
      W4A4_ROT(WW, OUT_MX)                    \
    }
  switch (WV) {
    W4A4_ROT_W(1) W4A4_ROT_W(2) W4A4_ROT_W(3) W4A4_ROT_W(4) W4A4_ROT_W(5) W4A4_ROT_W(6)
    W4A4_ROT_W(7) W4A4_ROT_W(8)
    default:
      return hipErrorInvalidValue;
  }
#undef W4A4_ROT_W
#undef W4A4_ROT_P0
#undef W4A4_ROT
}

bool rotq_mfma_roles_ok(int64_t M, int64_t K, int log2b) {
  const int64_t step = log2b == 12 ? 4096 : 2048;
  return M > 0 && M <= 64 && K % step == 0 && K >= step && K <= 8192 && log2b >= 7 && log2b <= 12;
}

hipError_t launch_rotq_mfma_roles(const _Float16* x, int64_t M, int64_t K, int log2b, bool f6,
                                  uint8_t* q, float* scale, const _Float16* lr_at, int lr_rank,
                                  void* lr_t, const ReadAhead& ra, hipStream_t st) {
  if (!rotq_mfma_roles_ok(M, K, log2b) || (lr_rank > 0 && M > 16) || ra.blocks % 8 != 0)
    return hipErrorInvalidValue;
  RotArgs a = base_args(x, M, K, log2b, q, scale, nullptr);
  a.lr_at = lr_at;
  a.lr_rank = lr_rank;
  a.lr_t = lr_t;
  a.ra = ra;
  a.qmax = 7.f;
  const int p = log2b - 7;
  kron_tables(p < 4 ? p : 4, &a);
  const int WV = static_cast<int>(K / 2048);
  const dim3 grid(static_cast<unsigned>(M + lr_rank + ra.blocks));
#define W4A4_ROLES(WW, OO)                                                                            \
  switch (p) {                                                                                        \
    case 0: hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 0, true>), grid, dim3(256), 0, st, a); break; \
    case 1: hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 1, true>), grid, dim3(256), 0, st, a); break; \
    case 2: hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 2, true>), grid, dim3(256), 0, st, a); break; \
    case 3: hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 3, true>), grid, dim3(256), 0, st, a); break; \
    case 4: hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 4, true>), grid, dim3(256), 0, st, a); break; \
    default:                                                                                          \
      if constexpr (WW % 2 == 0)                                                                      \
        hipLaunchKernelGGL((rotq_mfma_kernel<WW, OO, 5, true>), grid, dim3(256), 0, st, a);           \
      else                                                                                            \
        return hipErrorInvalidValue;                                                                  \
      break;                                                                                          \
  }                                                                                                   \
  return hipGetLastError();
#define W4A4_ROLES_W(WW)   \
  case WW:                  \
    if (f6) {               \
      W4A4_ROLES(WW, OUT_F6) \
    } else {                \
      W4A4_ROLES(WW, OUT_PACKED) \
    }
  switch (WV) {
    W4A4_ROLES_W(1) W4A4_ROLES_W(2) W4A4_ROLES_W(3) W4A4_ROLES_W(4)
    default:
      return hipErrorInvalidValue;
  }
#undef W4A4_ROLES_W
#undef W4A4_ROLES
}

}  // namespace w4a4
