// lowrank_rows.h — device body of T[:, j] = X . A[:, j] for few rows (M <= MR),
// fp16 operands, used by the low-rank kernel and by the fused decode prologue
// of the rotation kernel.  First factor of the single low-rank compensation
// term of SERQ (SERQ page, "Resumen técnico" §2 item 2), on the unrotated X.
//
// Needs exactly 256 threads (four waves).  They read, at channel
// 8 (64 w + l) + 2048 c, the 16 bytes of every row of X and of row j of At ([rank, K]), so that every
// load instruction is one contiguous 1 KB run, and accumulate x . a with fp16
// pair dot products in float32.  Partial sums are reduced across lanes, then
// across the four waves in a fixed order.  T is written as float32 [M, rank]
// or, with pair_out, as the fp16 pair t_hi [M, rank] followed by
// t_lo = fp16(T - t_hi) [M, rank].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

template <int MR>
__device__ __forceinline__ void lowrank_rows_body(const _Float16* __restrict__ x,
                                                  const _Float16* __restrict__ at, int64_t M,
                                                  int64_t K, int rank, void* __restrict__ t,
                                                  int pair_out, int j, float* red /* [4][MR] */) {
  typedef _Float16 half8v __attribute__((ext_vector_type(8)));
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const _Float16* arow = at + static_cast<int64_t>(j) * K;
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;
#pragma unroll 2
  for (int64_t k = 8 * tid; k < K; k += 2048) {
    const half8v av = *reinterpret_cast<const half8v*>(arow + k);
    half8v xv[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m)
      xv[m] = m < M ? *reinterpret_cast<const half8v*>(x + m * K + k)
                    : half8v{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < MR; ++m) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const half2v xa = {xv[m][2 * p], xv[m][2 * p + 1]};
        const half2v aa = {av[2 * p], av[2 * p + 1]};
        acc[m] = __builtin_amdgcn_fdot2(xa, aa, acc[m], false);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float v = acc[m];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    acc[m] = v;
  }
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m) red[wave * MR + m] = acc[m];
  }
  __syncthreads();
  if (tid < MR && tid < M) {
    const float sum = (red[tid] + red[MR + tid]) + (red[2 * MR + tid] + red[3 * MR + tid]);
    const int64_t m = tid;
    if (pair_out) {
      const _Float16 hi = static_cast<_Float16>(sum);
      const _Float16 lo = static_cast<_Float16>(sum - static_cast<float>(hi));
      static_cast<_Float16*>(t)[m * rank + j] = hi;
      static_cast<_Float16*>(t)[M * rank + m * rank + j] = lo;
    } else {
      static_cast<float*>(t)[m * rank + j] = sum;
    }
  }
}

}  // namespace w4a4
