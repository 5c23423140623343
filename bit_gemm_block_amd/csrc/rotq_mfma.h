// rotq_mfma.h — block Hadamard rotation on the fp16 matrix instruction, fused
// with per-token absmax int4 quantization into the tiled code layouts (FP6
// tiles, or packed tiles, plain or offset-binary with the row sums of the odd
// channels' codes) (SERQ page, "Resumen técnico" §1-2).  Both forms take fp16
// rows, one float32 scale per row, and more than 64 rows; every other form of
// the rotation runs the butterfly kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

// b = 2^log2b with 128 <= b <= 4096 (the transform of 16 sub-blocks of 128
// at a time, then for b > 128 the Kronecker factor across them): K a multiple
// of 2048 (of 4096 for b = 4096) up to 16384.
bool rotq_mfma_ok(int64_t M, int64_t K, int log2b);
hipError_t launch_rotq_mfma(const _Float16* x, int64_t M, int64_t K, int log2b, bool f6,
                            uint8_t* q, float* scale, int32_t* ob_sum, hipStream_t st);

}  // namespace w4a4
