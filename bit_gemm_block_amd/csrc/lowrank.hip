// lowrank.hip — T = X . A, the first factor of the single low-rank
// compensation term of SERQ (SERQ page, "Resumen técnico" §2 item 2), on the
// unrotated activations.  A is stored transposed, At [rank, K], so both
// operands are contiguous along the contraction like the int4 weights.
//
// fp16 inputs: v_mfma_f32_16x16x32_f16 with float32 accumulation.  A
// workgroup owns 16 rows of X and NCB blocks of 16 columns of T; its KW waves
// split K and their partial 16x16 tiles are summed in LDS in a fixed order.
// T is written as an fp16 pair (t_hi = fp16(T), t_lo = fp16(T - t_hi)) so
// that the GEMM epilogue can form T . B with two fp16 MFMAs at about 22 bits
// of precision.
//
// fp32 inputs: LDS-tiled float32 FMA, T written as float32.
#include "w4a4_internal.h"
#include "gemm_common.h"
#include "lowrank_rows.h"

namespace w4a4 {
namespace {


template <int NCB, int KW, int PF>
__global__ void __launch_bounds__(64 * KW) lowrank_f16_kernel(const _Float16* __restrict__ x,
                                                             const _Float16* __restrict__ at,
                                                             int64_t M, int64_t K, int rank,
                                                             void* __restrict__ t, int pair_out) {
  __shared__ f32x4 red[KW][NCB][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int c0 = blockIdx.y * NCB * 16;  // first column of T
  const int64_t mrow = m0 + (lane & 15);
  const int koff = (lane >> 4) * 8;
  const bool row_ok = mrow < M;

  f32x4 acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each wave owns a contiguous range of 32-wide K chunks and issues the
  // loads of PF chunks before their matrix instructions, so that a short
  // range costs one memory latency rather than one per chunk.
  const int64_t nchunks = K / 32;
  const int64_t c_begin = nchunks * wave / KW;
  const int64_t c_end = nchunks * (wave + 1) / KW;
  const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t cb = c_begin; cb < c_end; cb += PF) {
    half8 xa[PF], ab[PF][NCB];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const bool ok = cb + u < c_end;
      const int64_t k = (cb + u) * 32 + koff;
      xa[u] = ok && row_ok ? *reinterpret_cast<const half8*>(x + mrow * K + k) : zero8;
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const int j = c0 + c * 16 + (lane & 15);
        ab[u][c] = ok && j < rank
                       ? *reinterpret_cast<const half8*>(at + static_cast<int64_t>(j) * K + k)
                       : zero8;
      }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u)
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[u], ab[u][c], acc[c], 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < NCB; ++c) red[wave][c][lane] = acc[c];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      f32x4 s = red[0][c][lane];
#pragma unroll
      for (int w = 1; w < KW; ++w) s += red[w][c][lane];
      // Output fragment: rows 4*(lane>>4)+i, column lane&15.
      const int j = c0 + c * 16 + (lane & 15);
      if (j < rank) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = m0 + (lane >> 4) * 4 + i;
          if (m < M) {
            if (pair_out) {
              const _Float16 hi = static_cast<_Float16>(s[i]);
              const _Float16 lo = static_cast<_Float16>(s[i] - static_cast<float>(hi));
              static_cast<_Float16*>(t)[m * rank + j] = hi;
              static_cast<_Float16*>(t)[M * rank + m * rank + j] = lo;
            } else {
              static_cast<float*>(t)[m * rank + j] = s[i];
            }
          }
        }
      }
    }
  }
}

// Prefill sizes (fp16, rank <= 16 NCB <= 32, K a multiple of 512): one
// workgroup of eight waves per 16 rows of X, fed by direct-to-LDS copies.
// Stage s holds channels [512 s, 512 s + 512) of the 16 rows of X and of the
// 16 NCB rows of At, each row one contiguous 1 KB run (the register-loaded
// kernel above reads 16 rows x 64 bytes per load instruction, and At once per
// 16 rows of X, which bounded it at about 7 TB/s from the L2); rows lie
// 1040 bytes apart in LDS, so that the fragment reads of 16 rows fall in
// distinct banks.  Three stages are in flight.  Wave w multiplies K steps
// [2 w, 2 w + 2) of every stage; the waves' partial tiles are summed in LDS
// (over the first stage buffer) in a fixed order.  (Eight waves issue the
// copies of a stage faster than four: 22.4 -> 20.4 us at K = 14336.)  Rows past M and columns past rank read the last valid
// row (their results are not stored).
template <int NCB>
__global__ void __launch_bounds__(512) lowrank_stage_kernel(const _Float16* __restrict__ x,
                                                            const _Float16* __restrict__ at,
                                                            int64_t M, int64_t K, int rank,
                                                            void* __restrict__ t, int pair_out) {
  constexpr int ROWS = 16 + 16 * NCB;  // X rows, then At rows
  constexpr int RS = 1040;             // LDS bytes per row
  constexpr int STAGE = ROWS * RS;
  constexpr int NW = 8;                // waves
  constexpr int CPW = ROWS / NW;       // copies per wave per stage
  constexpr int STAGES = 3;
  static_assert(ROWS % NW == 0 && (STAGES - 1) * CPW < 64, "copies per wave");
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[STAGE];
  auto stage = [&](int sidx) -> uint8_t* { return sidx == 0 ? st0 : sidx == 1 ? st1 : st2; };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int nst = static_cast<int>(K / 512);

  // Copy q of this wave: stage row wave + NW q.
  const uint8_t* src[CPW];
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int row = wave + NW * q;
    const _Float16* p;
    if (row < 16) {
      const int64_t m = m0 + row < M ? m0 + row : M - 1;
      p = x + m * K;
    } else {
      const int j = row - 16 < rank ? row - 16 : rank - 1;
      p = at + static_cast<int64_t>(j) * K;
    }
    src[q] = reinterpret_cast<const uint8_t*>(p) + 16 * lane;
  }
  auto issue = [&](int s, uint8_t* buf) {
    const uint32_t b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf));
#pragma unroll
    for (int q = 0; q < CPW; ++q) dma16(src[q] + static_cast<int64_t>(s) * 1024, b + (wave + NW * q) * RS);
  };

  f32x4 acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r = lane & 15, g = lane >> 4;
  auto compute = [&](const uint8_t* buf) {
#pragma unroll
    for (int u = 0; u < 16 / NW; ++u) {
      const int off = ((16 / NW) * wave + u) * 64 + 16 * g;
      const half8 xa = *reinterpret_cast<const half8*>(buf + r * RS + off);
      half8 ab[NCB];
#pragma unroll
      for (int c = 0; c < NCB; ++c) ab[c] = *reinterpret_cast<const half8*>(buf + (16 + 16 * c + r) * RS + off);
#pragma unroll
      for (int c = 0; c < NCB; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, ab[c], acc[c], 0, 0, 0);
    }
  };
  // Stage s: once it has landed and the barrier has retired every wave's
  // reads of stage s - 1, that buffer takes stage s + 2.
  auto iterate = [&](int s, int sbuf, bool steady) {
    if (steady || s + 2 <= nst)
      wait_vmcnt<CPW>();
    else
      wait_vmcnt<0>();
    stage_barrier();
    if (steady || s + 2 < nst) issue(s + 2, stage((sbuf + 2) % 3));
    compute(stage(sbuf));
  };
  issue(0, st0);
  if (nst > 1) issue(1, st1);
  int s0 = 0;
  for (; s0 + 6 <= nst; s0 += 3) {
    iterate(s0, 0, true);
    iterate(s0 + 1, 1, true);
    iterate(s0 + 2, 2, true);
  }
#pragma unroll
  for (int u = 0; u < 6; ++u)
    if (s0 + u < nst) iterate(s0 + u, u % 3, false);

  f32x4 (*red)[NCB][64] = reinterpret_cast<f32x4 (*)[NCB][64]>(st0);
  __syncthreads();  // every wave's last reads of the stages
#pragma unroll
  for (int c = 0; c < NCB; ++c) red[wave][c][lane] = acc[c];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      f32x4 sum = red[0][c][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += red[w][c][lane];
      const int j = c * 16 + (lane & 15);
      if (j < rank) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = m0 + (lane >> 4) * 4 + i;
          if (m < M) {
            if (pair_out) {
              const _Float16 hi = static_cast<_Float16>(sum[i]);
              const _Float16 lo = static_cast<_Float16>(sum[i] - static_cast<float>(hi));
              static_cast<_Float16*>(t)[m * rank + j] = hi;
              static_cast<_Float16*>(t)[M * rank + m * rank + j] = lo;
            } else {
              static_cast<float*>(t)[m * rank + j] = sum[i];
            }
          }
        }
      }
    }
  }
}

// Few rows (M <= MR), fp16: one workgroup per column j of T (body in
// lowrank_rows.h).
template <int MR>
__global__ void __launch_bounds__(256) lowrank_rows_kernel(const _Float16* __restrict__ x,
                                                          const _Float16* __restrict__ at,
                                                          int64_t M, int64_t K, int rank,
                                                          void* __restrict__ t, int pair_out) {
  __shared__ float red[4 * MR];
  lowrank_rows_body<MR>(x, at, M, K, rank, t, pair_out, blockIdx.x, red);
}

constexpr int TR = 16;  // rows of X per workgroup (fp32 path)
constexpr int TC = 64;  // columns of T per workgroup
constexpr int KC = 64;  // K chunk

__global__ void __launch_bounds__(256) lowrank_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ at, int64_t M,
                                                         int64_t K, int rank,
                                                         float* __restrict__ t) {
  __shared__ float xs[TR][KC + 1];
  __shared__ float as[TC][KC + 1];
  const int tid = threadIdx.x;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * TR;
  const int c0 = blockIdx.y * TC;
  const int col = tid % TC;
  const int rg = (tid / TC) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < K; k0 += KC) {
    for (int e = tid; e < TR * KC; e += 256) {
      const int i = e / KC, k = e % KC;
      const int64_t m = r0 + i;
      xs[i][k] = m < M ? x[m * K + k0 + k] : 0.f;
    }
    for (int e = tid; e < TC * KC; e += 256) {
      const int c = e / KC, k = e % KC;
      as[c][k] = (c0 + c) < rank ? at[static_cast<int64_t>(c0 + c) * K + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < KC; ++k) {
      const float av = as[col][k];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(xs[rg + q][k], av, acc[q]);
    }
    __syncthreads();
  }
  if (c0 + col < rank) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = r0 + rg + q;
      if (m < M) t[m * rank + c0 + col] = acc[q];
    }
  }
}

template <int NCB>
hipError_t launch_f16(const _Float16* x, const _Float16* at, int64_t M, int64_t K, int rank,
                      void* t, int pair, hipStream_t st) {
  const int64_t row_tiles = (M + 15) / 16;
  const int col_groups = (rank + NCB * 16 - 1) / (NCB * 16);
  const dim3 grid(static_cast<unsigned>(row_tiles), static_cast<unsigned>(col_groups));
  constexpr int PF = NCB >= 4 ? 2 : 8 / NCB;
  if constexpr (NCB <= 4) {
    // Sixteen waves split K, so that every wave has a short range whose
    // loads are all in flight at once (with four waves the 4096-row
    // projection was a chain of eight dependent load batches per wave).
    hipLaunchKernelGGL((lowrank_f16_kernel<NCB, 16, PF>), grid, dim3(1024), 0, st, x, at, M, K,
                       rank, t, pair);
    return hipGetLastError();
  } else {
    hipLaunchKernelGGL((lowrank_f16_kernel<NCB, 4, PF>), grid, dim3(256), 0, st, x, at, M, K,
                       rank, t, pair);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_lowrank_project(const void* x, bool x_f16, const void* at, int64_t M, int64_t K,
                                  int rank, void* t, bool pair_out, hipStream_t st) {
  if (x_f16) {
    const _Float16* xh = static_cast<const _Float16*>(x);
    const _Float16* ah = static_cast<const _Float16*>(at);
    const int pair = pair_out ? 1 : 0;
    const int64_t row_tiles = (M + 15) / 16;
    const int blocks = (rank + 15) / 16;
    if (M <= 8) {
      hipLaunchKernelGGL((lowrank_rows_kernel<8>), dim3(rank), dim3(256), 0, st, xh, ah, M, K,
                         rank, t, pair);
      return hipGetLastError();
    }
    if (M <= 16) {
      hipLaunchKernelGGL((lowrank_rows_kernel<16>), dim3(rank), dim3(256), 0, st, xh, ah, M, K,
                         rank, t, pair);
      return hipGetLastError();
    }
    // Prefill sizes: the staged kernel.
    if (row_tiles >= 64 && rank <= 32 && K % 512 == 0) {
      const dim3 grid(static_cast<unsigned>(row_tiles));
      if (rank <= 16)
        hipLaunchKernelGGL((lowrank_stage_kernel<1>), grid, dim3(512), 0, st, xh, ah, M, K, rank, t, pair);
      else
        hipLaunchKernelGGL((lowrank_stage_kernel<2>), grid, dim3(512), 0, st, xh, ah, M, K, rank, t, pair);
      return hipGetLastError();
    }
    // Few row tiles: one 16-column block per workgroup for parallelism.
    // Many row tiles: all columns in one workgroup so X is read once.
    if (row_tiles < 64 || blocks == 1) return launch_f16<1>(xh, ah, M, K, rank, t, pair, st);
    if (blocks <= 2) return launch_f16<2>(xh, ah, M, K, rank, t, pair, st);
    if (blocks <= 4) return launch_f16<4>(xh, ah, M, K, rank, t, pair, st);
    if (blocks <= 8) return launch_f16<8>(xh, ah, M, K, rank, t, pair, st);
    return launch_f16<16>(xh, ah, M, K, rank, t, pair, st);
  }
  const dim3 grid(static_cast<unsigned>((M + TR - 1) / TR), static_cast<unsigned>((rank + TC - 1) / TC));
  hipLaunchKernelGGL(lowrank_f32_kernel, grid, dim3(256), 0, st, static_cast<const float*>(x),
                     static_cast<const float*>(at), M, K, rank, static_cast<float*>(t));
  return hipGetLastError();
}

}  // namespace w4a4
