// offq.hip — weight group sums for asymmetric activation groups.
//
// With per-group zero points z on the activations (OffQ page,
// "Metodología" steps 2-3: the zero point of a per-group asymmetric
// quantizer absorbs the constant offset the all-ones Hadamard row creates),
// the product over a group is sum_k (q - z) qw = sum_k q qw - z sum_k qw.
// The second factor, sum_k qw over the group, depends on the weights only and
// is computed once, offline, by this kernel.
#include "w4a4_internal.h"

namespace w4a4 {
namespace {

// One wave per (row n, group g); every lane reads 4 packed bytes (8 codes)
// per step and the wave reduces by shuffles.
__global__ void __launch_bounds__(256) weight_group_sums_kernel(const uint8_t* wq, int tiled,
                                                                int64_t N, int64_t K, int group,
                                                                int32_t* out) {
  const int64_t G = K / group;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (item >= N * G) return;  // whole waves leave together
  const int lane = threadIdx.x & 63;
  const int64_t n = item / G, g = item % G;
  const int64_t nkt = K / 128;
  const int64_t j1 = (g + 1) * (group / 2);
  int sum = 0;
  for (int64_t j = g * (group / 2) + 4 * lane; j < j1; j += 256) {
    // Packed byte j of row n: row-major, or in the 1 KB tile (n / 16, j / 64)
    // at ((j % 64) / 16 * 16 + n % 16) * 16 + j % 16.  Four bytes from a
    // multiple of 4 stay inside one 16-byte piece.
    const int64_t off = tiled ? ((n >> 4) * nkt + (j >> 6)) * 1024 +
                                    ((((j & 63) >> 4) * 16 + (n & 15)) << 4) + (j & 15)
                              : n * (K / 2) + j;
    const uint32_t d = *reinterpret_cast<const uint32_t*>(wq + off);
#pragma unroll
    for (int t = 0; t < 8; ++t) sum += static_cast<int32_t>(d << (28 - 4 * t)) >> 28;
  }
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) out[n * G + g] = sum;
}

}  // namespace

hipError_t launch_weight_group_sums(const uint8_t* wq, bool tiled, int64_t N, int64_t K, int group,
                                    int32_t* out, hipStream_t st) {
  const int64_t items = N * (K / group);
  const dim3 grid(static_cast<unsigned>((items + 3) / 4));
  hipLaunchKernelGGL(weight_group_sums_kernel, grid, dim3(256), 0, st, wq, tiled ? 1 : 0, N, K,
                     group, out);
  return hipGetLastError();
}

}  // namespace w4a4
