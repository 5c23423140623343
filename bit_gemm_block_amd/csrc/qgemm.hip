// qgemm.hip — int4 x int4 GEMM on gfx950 int8 matrix cores, with the
// dequantizing epilogue and the low-rank term (SERQ page, "Resumen técnico"
// §2-3: a 4-bit product in the linear layer plus a single low-rank
// compensation matrix added to it).
//
//   acc[m, n] = sum_k qx[m, k] * qw[n, k]          (exact int32)
//   y[m, n]   = sx[m] * sum_j sw[n, j] * acc_j[m, n] + (T . B)[m, n]
//
// Both operands are packed int4, K-contiguous ([rows, K/2] bytes).  There is
// no int4 matrix instruction on CDNA4, so codes are widened to int8 in
// registers right before v_mfma_i32_16x16x64_i8.  A nibble moved to the top
// of its byte is a valid signed int8 equal to 16*q, so the widening is one
// AND (high nibbles) or one shift+AND (low nibbles) per 8 codes, and the
// accumulator holds 256 * acc, which stays below 2^31 for K <= 65536
// (256 * 64 * K).  Low and high nibbles of a dword feed different int8
// lanes of the instruction, i.e. the K order inside one instruction is
// permuted; A and B use the same permutation, so the dot products are exact.
//
// Tiling: a 256-thread workgroup owns a BM x BN output tile; its four waves
// form a 2 x 2 grid of (BM/2) x (BN/2) wave tiles.  K advances 128 codes
// (64 bytes per row, two MFMA K steps) per iteration through double-buffered
// LDS tiles.
#include "w4a4_internal.h"

#include <hip/hip_fp16.h>

namespace w4a4 {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int BK_BYTES = 64;  // 128 int4 codes per row per K step

__device__ __forceinline__ float load_scale(const void* p, int64_t i, int f16) {
  if (f16) return __half2float(reinterpret_cast<const __half*>(p)[i]);
  return reinterpret_cast<const float*>(p)[i];
}

// Widen 16 packed nibbles (two dwords) into one MFMA operand of 16 int8
// values 16*q: low nibbles of p0, high nibbles of p0, then the same for p1.
__device__ __forceinline__ i32x4 widen(uint32_t p0, uint32_t p1) {
  return i32x4{static_cast<int32_t>((p0 << 4) & 0xF0F0F0F0u), static_cast<int32_t>(p0 & 0xF0F0F0F0u),
               static_cast<int32_t>((p1 << 4) & 0xF0F0F0F0u), static_cast<int32_t>(p1 & 0xF0F0F0F0u)};
}

// LDS tile rows hold 64 bytes (128 codes).  Lane group g (lanes 16g..16g+15)
// of an MFMA reads one 16-byte chunk: its first 8 bytes are codes
// [16g, 16g+16) of K step 0 (codes 0..63 of the row) and its last 8 bytes the
// same slice of K step 1 (codes 64..127), so that each K step is a contiguous
// range of 64 codes.  Chunks are XOR-swizzled by row to spread LDS banks.
//
// Physical byte offset of 16-byte chunk c of tile row r.
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * BK_BYTES + ((c ^ ((r >> 2) & 3)) << 4);
}
// Physical byte offset of logical 8-byte piece p (bytes [8p, 8p+8)) of row r.
__device__ __forceinline__ int piece_off(int r, int p) {
  return tile_off(r, p & 3) + ((p >> 2) << 3);
}

template <int BM, int BN, bool GROUPED>
__global__ void __launch_bounds__(256) qgemm_kernel(GemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int A_UNITS = BM * BK_BYTES / 16 / 256;  // 16-byte loads per thread
  constexpr int B_UNITS = BN * BK_BYTES / 16 / 256;
  static_assert(A_UNITS >= 1 && B_UNITS >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * BK_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * BK_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave >> 1) * WM;
  const int wn0 = (wave & 1) * WN;

  const int64_t tiles_n = (a.N + BN - 1) / BN;
  const int64_t tile = blockIdx.x;
  const int64_t m0 = (tile / tiles_n) * BM;
  const int64_t n0 = (tile % tiles_n) * BN;
  const int64_t K = a.K;
  const int64_t row_bytes = K / 2;
  const int nkt = static_cast<int>((K + 127) / 128);
  const int ksteps = static_cast<int>(K / 64);

  uint4 ra[A_UNITS], rb[B_UNITS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i) {
      const int u = tid + 256 * i;
      const int r = u >> 2, c = u & 3;
      const int64_t m = m0 + r;
      const int64_t kb = static_cast<int64_t>(kt) * BK_BYTES + c * 16;
      if (m < a.M && kb < row_bytes)
        ra[i] = *reinterpret_cast<const uint4*>(a.xq + m * row_bytes + kb);
      else
        ra[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_UNITS; ++i) {
      const int u = tid + 256 * i;
      const int r = u >> 2, c = u & 3;
      const int64_t n = n0 + r;
      const int64_t kb = static_cast<int64_t>(kt) * BK_BYTES + c * 16;
      if (n < a.N && kb < row_bytes)
        rb[i] = *reinterpret_cast<const uint4*>(a.wq + n * row_bytes + kb);
      else
        rb[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i) {
      const int u = tid + 256 * i;
      const int r = u >> 2, p = (u & 3) * 2;
      *reinterpret_cast<uint2*>(&As[buf][piece_off(r, p)]) = make_uint2(ra[i].x, ra[i].y);
      *reinterpret_cast<uint2*>(&As[buf][piece_off(r, p + 1)]) = make_uint2(ra[i].z, ra[i].w);
    }
#pragma unroll
    for (int i = 0; i < B_UNITS; ++i) {
      const int u = tid + 256 * i;
      const int r = u >> 2, p = (u & 3) * 2;
      *reinterpret_cast<uint2*>(&Bs[buf][piece_off(r, p)]) = make_uint2(rb[i].x, rb[i].y);
      *reinterpret_cast<uint2*>(&Bs[buf][piece_off(r, p + 1)]) = make_uint2(rb[i].z, rb[i].w);
    }
  };

  i32x4 acc[TM][TN];
  float facc[GROUPED ? TM : 1][GROUPED ? TN : 1][4];
  i32x4 full[GROUPED ? TM : 1][GROUPED ? TN : 1];  // full-K sum (for the acc output)
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
  if constexpr (GROUPED) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        full[i][j] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < 4; ++r) facc[i][j][r] = 0.f;
      }
  }
  const bool want_y = a.y != nullptr;  // scales are only read when y is written
  const int gsteps = GROUPED ? a.group / 64 : 1;
  const int64_t ngroups = GROUPED ? K / a.group : 1;

  gload(0);
  lstore(0);
  __syncthreads();

  const int frow = lane & 15;  // fragment row within a 16-row block
  const int fchk = lane >> 4;  // 16-byte chunk of the 64-byte tile row

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);

    uint4 fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[i] = *reinterpret_cast<const uint4*>(&As[buf][tile_off(wm0 + i * 16 + frow, fchk)]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[j] = *reinterpret_cast<const uint4*>(&Bs[buf][tile_off(wn0 + j * 16 + frow, fchk)]);

#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kstep = kt * 2 + h;
      if (kstep < ksteps) {
        i32x4 opa[TM], opb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) opa[i] = h ? widen(fa[i].z, fa[i].w) : widen(fa[i].x, fa[i].y);
#pragma unroll
        for (int j = 0; j < TN; ++j) opb[j] = h ? widen(fb[j].z, fb[j].w) : widen(fb[j].x, fb[j].y);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(opa[i], opb[j], acc[i][j], 0, 0, 0);

        if constexpr (GROUPED) {
          if ((kstep + 1) % gsteps == 0) {
            const int64_t grp = (kstep + 1) / gsteps - 1;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const int64_t n = n0 + wn0 + j * 16 + frow;
              const float sw =
                  (want_y && n < a.N) ? load_scale(a.sw, n * ngroups + grp, a.sw_f16) : 0.f;
#pragma unroll
              for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  facc[i][j][r] = fmaf(static_cast<float>(acc[i][j][r]), sw, facc[i][j][r]);
                full[i][j] += acc[i][j];
                acc[i][j] = i32x4{0, 0, 0, 0};
              }
            }
          }
        }
      }
    }

    if (kt + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  Output fragment (i, j) of lane holds rows 4*(lane>>4)+r, column lane&15.
  const int ecol = lane & 15;
  const int erow = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t n = n0 + wn0 + j * 16 + ecol;
    if (n >= a.N) continue;
    const float swn = (GROUPED || !want_y) ? 1.f : load_scale(a.sw, n, a.sw_f16);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm0 + i * 16 + erow + r;
        if (m >= a.M) continue;
        const int32_t total = GROUPED ? full[GROUPED ? i : 0][GROUPED ? j : 0][r] : acc[i][j][r];
        if (a.acc) a.acc[m * a.N + n] = total >> 8;
        if (a.y) {
          float val;
          if constexpr (GROUPED)
            val = facc[i][j][r] * (a.sx[m] * 0.00390625f);
          else
            val = static_cast<float>(total) * (a.sx[m] * swn * 0.00390625f);
          if (a.rank > 0) {
            float lr = 0.f;
            const float* trow = a.t + m * a.rank;
            for (int q = 0; q < a.rank; ++q)
              lr = fmaf(trow[q], load_scale(a.B, static_cast<int64_t>(q) * a.N + n, a.b_f16), lr);
            val += lr;
          }
          a.y[m * a.N + n] = val;
        }
      }
    }
  }
}

template <int BM, int BN>
hipError_t launch_tile(const GemmArgs& a, hipStream_t st) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (a.group > 0)
    hipLaunchKernelGGL((qgemm_kernel<BM, BN, true>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                       st, a);
  else
    hipLaunchKernelGGL((qgemm_kernel<BM, BN, false>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                       st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qgemm(const GemmArgs& a, hipStream_t st) { return launch_tile<128, 128>(a, st); }

}  // namespace w4a4
