// offq.hip — weight-side preparation: group sums for asymmetric activation
// groups, and the conversion to offset-binary tiled weights.
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

// Offset-binary weights: one wave per (padded) row n.  Every byte of the
// row's tile pieces gets its nibbles swapped, the new low nibble XOR 8 (the
// odd channel's code + 8 below the even channel's signed code), and the
// codes at even channels (the old low nibbles) are summed for the row.  Each
// lane reads and writes only its own 16-byte pieces, so out may equal wq.
__global__ void __launch_bounds__(256) weights_to_ob_kernel(const uint8_t* wq, int64_t rows,
                                                            int64_t K, uint8_t* out) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (n >= rows) return;  // whole waves leave together
  const int lane = threadIdx.x & 63;
  const int64_t nkt = K / 128;
  int sum = 0;
  for (int64_t p = lane; p < nkt * 4; p += 64) {
    const int64_t kt = p >> 2;
    const int g = static_cast<int>(p & 3);
    const int64_t off = ((n >> 4) * nkt + kt) * 1024 + ((g * 16 + (n & 15)) << 4);
    const uint4 v = *reinterpret_cast<const uint4*>(wq + off);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t x = w[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) sum += static_cast<int32_t>(x << (28 - 8 * i)) >> 28;
      w[t] = ((x & 0x0F0F0F0Fu) << 4) | (((x >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u);
    }
    *reinterpret_cast<uint4*>(out + off) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) reinterpret_cast<int32_t*>(out + rows * (K / 2))[n] = sum;
}

}  // namespace

hipError_t launch_weights_to_ob(const uint8_t* wq, int64_t rows, int64_t K, uint8_t* out,
                                hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  hipLaunchKernelGGL(weights_to_ob_kernel, grid, dim3(256), 0, st, wq, rows, K, out);
  return hipGetLastError();
}

hipError_t launch_weight_group_sums(const uint8_t* wq, bool tiled, int64_t N, int64_t K, int group,
                                    int32_t* out, hipStream_t st) {
  const int64_t items = N * (K / group);
  const dim3 grid(static_cast<unsigned>((items + 3) / 4));
  hipLaunchKernelGGL(weight_group_sums_kernel, grid, dim3(256), 0, st, wq, tiled ? 1 : 0, N, K,
                     group, out);
  return hipGetLastError();
}

}  // namespace w4a4
