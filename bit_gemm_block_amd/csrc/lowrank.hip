// lowrank.hip — T = X . A, the first factor of the single low-rank
// compensation term of SERQ (SERQ page, "Resumen técnico" §2 item 2), on the
// unrotated activations.  float32 accumulation; X and A are fp16 or fp32.
//
// A workgroup owns 16 rows of X and 64 columns of A.  K is walked in chunks
// of 64: the X chunk [16 x 64] and the A chunk [64 x 64] are staged in LDS as
// float32 and every thread accumulates 4 outputs (4 rows of one column).
#include "w4a4_internal.h"

namespace w4a4 {
namespace {

constexpr int TR = 16;  // rows of X per workgroup
constexpr int TC = 64;  // columns of A per workgroup
constexpr int KC = 64;  // K chunk

template <typename T>
__global__ void __launch_bounds__(256) lowrank_project_kernel(const T* __restrict__ x,
                                                             const T* __restrict__ A, int64_t M,
                                                             int64_t K, int rank,
                                                             float* __restrict__ t) {
  __shared__ float xs[TR][KC + 1];
  __shared__ float as[KC][TC + 1];
  const int tid = threadIdx.x;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * TR;
  const int c0 = blockIdx.y * TC;
  const int col = tid % TC;
  const int rg = (tid / TC) * 4;  // first of this thread's 4 rows
  float acc[4] = {0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < K; k0 += KC) {
    for (int e = tid; e < TR * KC; e += 256) {
      const int i = e / KC, k = e % KC;
      const int64_t m = r0 + i;
      xs[i][k] = m < M ? static_cast<float>(x[m * K + k0 + k]) : 0.f;
    }
    for (int e = tid; e < KC * TC; e += 256) {
      const int k = e / TC, c = e % TC;
      as[k][c] = (c0 + c) < rank ? static_cast<float>(A[(k0 + k) * rank + c0 + c]) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < KC; ++k) {
      const float av = as[k][col];
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

}  // namespace

hipError_t launch_lowrank_project(const void* x, bool x_f16, const void* A, int64_t M, int64_t K,
                                  int rank, float* t, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((M + TR - 1) / TR), static_cast<unsigned>((rank + TC - 1) / TC));
  if (x_f16)
    hipLaunchKernelGGL(lowrank_project_kernel<_Float16>, grid, dim3(256), 0, st,
                       static_cast<const _Float16*>(x), static_cast<const _Float16*>(A), M, K, rank,
                       t);
  else
    hipLaunchKernelGGL(lowrank_project_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(A), M, K, rank, t);
  return hipGetLastError();
}

}  // namespace w4a4
