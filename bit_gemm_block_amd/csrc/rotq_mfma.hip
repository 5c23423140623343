// rotq_mfma.hip — block Hadamard rotation with b = 128 on the fp16 matrix
// instruction, fused with per-token absmax int4 quantization into the tiled
// code layouts of the layer: FP6 E2M3 tiles, or packed nibble tiles (plain or
// offset-binary, with the row sums of the odd channels' codes) (SERQ page,
// "Resumen técnico" §1-2: rotate, then quantize each token on the fly).
//
// With b = 128 the rotation of a row is 128-point transforms of its blocks,
// y_c = H x_c (H the Sylvester matrix, entries +-1).  Sixteen blocks at a
// time are one product H [128 x 128] . X^T [128 x 16] of exact fp16 operands
// (fp16 X, H = +-1) with float32 accumulation, 32 instructions of
// v_mfma_f32_16x16x32_f16, where the butterflies would take 7 VALU
// instructions per element.  Everything after the transform is the
// quantizer of the butterfly kernel: x~ = RN(y / sqrt(b)) as y * rs,
// s = RN(max|x~| / 7), each code rint of the correctly rounded quotient
// x~ / s (reciprocal plus two refinement steps; exact for every scale fp16
// input can produce), so the two kernels differ only where the float32
// sums of the transform round differently.
//
// A workgroup takes one row; wave w takes its elements [2048 w, 2048 w + 2048)
// as sixteen blocks c of 128:
//   * operand B of K-step kc: lane 16 g + c holds x[128 c + 32 kc + 8 g, +8)
//     (one 16-byte load);
//   * operand A of output block mb, K-step kc: lane 16 g + r holds
//     H[16 mb + r][32 kc + 8 g + t], t < 8, which splits into a per-lane
//     part and signs: with i = 16 mb + r and k = 32 kc + 8 g + t, i & k
//     keeps r & t (bits 0-2), r3 & g0 (bit 3), mb0 & g1 (bit 4) and
//     mb1 & kc0, mb2 & kc1 (bits 5-6), so A = +-(mb0 ? F1 : F0) with F0, F1
//     built once per lane;
//   * output: lane 16 g + c holds y_c[16 mb + 4 g + i'], i' < 4.
// The row's absmax is reduced over lanes and waves.  For the tiles, lane
// 16 j + c must hold the 32 consecutive codes [32 j, 32 j + 32) of block c,
// which lane groups g = 0..3 hold 8 each (mb = 2 j, 2 j + 1): a 4 x 4
// transpose of 8-value units across the lane groups, by v_permlane32_swap
// (lane groups 0,1 <-> 2,3) then v_permlane16_swap (0 <-> 1, 2 <-> 3).
#include "w4a4_internal.h"

#include <hip/hip_fp16.h>

namespace w4a4 {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: x + kMagic - kMagic = rint(x) for |x| < 2^22

struct Rot128Args {
  const _Float16* x;  // [M, K]
  int64_t M, K;
  float rs;           // float32(1 / sqrt(128))
  uint8_t* q;         // the code tiles
  float* scale;       // [M]
  int32_t* ob_sum;    // offset-binary packed tiles: [M] sums of the odd channels' codes
  int64_t tile_stride;  // tiles per 16-row block (K / 128)
  int64_t rows_per_xcd;  // a multiple of 16
};

// Output layouts.
enum { OUT_F6 = 0, OUT_PACKED = 1, OUT_PACKED_OB = 2 };

__device__ __forceinline__ h8 neg8(h8 v) {
  h8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = -v[t];
  return r;
}

template <int W, int OUT>  // W waves per row: K = 2048 W
__global__ void __launch_bounds__(64 * W) rotq128_kernel(Rot128Args a) {
  __shared__ float wmax[W];
  __shared__ int wsum[W];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  // Workgroup b runs on XCD b % 8 (round robin); each XCD takes a range of
  // whole 16-row blocks, so that every line of a code tile is written from
  // one L2.
  const int64_t row = (blockIdx.x % 8) * a.rows_per_xcd + blockIdx.x / 8;
  if (row >= a.M) return;
  const _Float16* src = a.x + row * a.K + 2048 * w + 128 * c + 8 * g;

  h8 xb[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) xb[kc] = *reinterpret_cast<const h8*>(src + 32 * kc);

  // F0[t] = H sign of (r & t) and (r3 & g0); F1 adds (g1) for odd mb.
  const int r = lane & 15;
  h8 f0, f1;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int par = (__builtin_popcount(r & t & 7) + ((r >> 3) & g & 1)) & 1;
    f0[t] = par ? static_cast<_Float16>(-1.0f) : static_cast<_Float16>(1.0f);
    f1[t] = ((g >> 1) & 1) ? -f0[t] : f0[t];
  }
  const h8 n0 = neg8(f0), n1 = neg8(f1);

  f4 acc[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    acc[mb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bool neg = (((mb >> 1) & kc & 1) ^ ((mb >> 2) & (kc >> 1) & 1)) != 0;
      const h8 av = (mb & 1) ? (neg ? n1 : f1) : (neg ? n0 : f0);
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, xb[kc], acc[mb], 0, 0, 0);
    }
  }

  // Row absmax of y (x~ = RN(y rs) is monotone in |y|).
  float m = 0.f;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(acc[mb][i]));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (W > 1) {
    if (lane == 0) wmax[w] = m;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < W; ++v) m = fmaxf(m, wmax[v]);
  }

  // Scale and codes, as the butterfly kernel's quantizer (fp16 input keeps
  // every scale inside the range where the refined reciprocal is exact).
  const float amax = m * a.rs;
  const float s = __fdiv_rn(amax, 7.0f);
  if (threadIdx.x == 0) a.scale[row] = s;
  const float rc = s == 0.f ? 0.f : __frcp_rn(s);
  // cm holds q + 1.5 * 2^23 for the code q: minus that constant it is q as a
  // float (the FP6 packing instruction's input), and its low nibble is q in
  // two's complement.
  float cm[8][4];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float xt = acc[mb][i] * a.rs;
      float q = xt * rc;
      q = __builtin_fmaf(__builtin_fmaf(-q, s, xt), rc, q);
      q = __builtin_fmaf(__builtin_fmaf(-q, s, xt), rc, q);
      cm[mb][i] = q + kMagic;
    }

  // Unit j of this lane (the 8 codes of chunk j: mb = 2 j + v / 4, i' = v % 4)
  // goes to lane group j.  After the two swaps, B[s][v] is unit (this lane
  // group) of source group s.
  uint32_t u[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 8; ++v) u[j][v] = __float_as_uint(cm[2 * j + (v >> 2)][v & 3]);
  uint32_t b[4][8];
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
  // This lane now holds codes [32 g, 32 g + 32) of block 16 w + c of the
  // row; chunk offset 16 (v / 4) + 4 s + v % 4 is B[s][v].
  const int64_t blk = (row >> 4) * a.tile_stride + 16 * w + c;  // tile of block 16 w + c
  const int rin = static_cast<int>(row & 15);
  if constexpr (OUT == OUT_F6) {
    // lane 16 g + (row % 16) of the 1536-byte FP6 tile
    f16v lo, hi;
#pragma unroll
    for (int sg = 0; sg < 4; ++sg)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lo[4 * sg + t] = __uint_as_float(b[sg][t]) - kMagic;
        hi[4 * sg + t] = __uint_as_float(b[sg][4 + t]) - kMagic;
      }
    const auto p = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(lo, hi, 1.0f);
    uint8_t* tile = a.q + blk * 1536;
    const int l6 = 16 * g + rin;
    *reinterpret_cast<uint4*>(tile + 16 * l6) = make_uint4(p[0], p[1], p[2], p[3]);
    *reinterpret_cast<uint2*>(tile + 1024 + 8 * l6) = make_uint2(p[4], p[5]);
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
    if constexpr (OUT == OUT_PACKED_OB) {
      // Row sum of the codes at odd channels (the high nibbles, as int8 16 q),
      // then the low nibbles offset by 8.
      int os16 = 0;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        os16 = __builtin_amdgcn_sdot4(static_cast<int>(pk[d] & 0xF0F0F0F0u), 0x01010101, os16, false);
      int os = os16 >> 4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) os += __shfl_xor(os, o);
      if (W > 1) {
        if (lane == 0) wsum[w] = os;
        __syncthreads();
        os = 0;
#pragma unroll
        for (int v = 0; v < W; ++v) os += wsum[v];
      }
      if (threadIdx.x == 0) a.ob_sum[row] = os;
#pragma unroll
      for (int d = 0; d < 4; ++d) pk[d] ^= 0x08080808u;
    }
    *reinterpret_cast<uint4*>(a.q + blk * 1024 + (16 * g + rin) * 16) =
        make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

}  // namespace

bool rotq128_ok(int64_t M, int64_t K) {
  return M > 64 && K % 2048 == 0 && K >= 2048 && K <= 16384;
}

hipError_t launch_rotq128(const _Float16* x, int64_t M, int64_t K, bool f6, uint8_t* q,
                          float* scale, int32_t* ob_sum, hipStream_t st) {
  Rot128Args a;
  a.x = x;
  a.M = M;
  a.K = K;
  a.rs = static_cast<float>(1.0 / __builtin_sqrt(128.0));
  a.q = q;
  a.scale = scale;
  a.ob_sum = ob_sum;
  a.tile_stride = K / 128;
  a.rows_per_xcd = ((M + 15) / 16 + 7) / 8 * 16;
  const dim3 grid(static_cast<unsigned>(8 * a.rows_per_xcd));
  const int out = f6 ? OUT_F6 : ob_sum ? OUT_PACKED_OB : OUT_PACKED;
  switch (K / 2048) {
#define W4A4_R128(WW)                                                                        \
  case WW:                                                                                   \
    if (out == OUT_F6)                                                                       \
      hipLaunchKernelGGL((rotq128_kernel<WW, OUT_F6>), grid, dim3(64 * WW), 0, st, a);       \
    else if (out == OUT_PACKED)                                                              \
      hipLaunchKernelGGL((rotq128_kernel<WW, OUT_PACKED>), grid, dim3(64 * WW), 0, st, a);   \
    else                                                                                     \
      hipLaunchKernelGGL((rotq128_kernel<WW, OUT_PACKED_OB>), grid, dim3(64 * WW), 0, st, a); \
    return hipGetLastError();
    W4A4_R128(1) W4A4_R128(2) W4A4_R128(3) W4A4_R128(4) W4A4_R128(5) W4A4_R128(6)
    W4A4_R128(7) W4A4_R128(8)
#undef W4A4_R128
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace w4a4
