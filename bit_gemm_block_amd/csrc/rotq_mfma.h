// rotq_mfma.h — block Hadamard rotation on the fp16 matrix instruction, fused
// with the activation quantizer into the tiled code layouts: per-token absmax
// int4 codes with one float32 scale per row in FP6 tiles, packed tiles
// (plain, or offset-binary with the row sums of the odd channels' codes) or
// int8 tiles (SERQ page, "Resumen técnico" §1-2; 8-bit codes for the W4A8
// layer), MXFP4 codes with their E8M0 scale tiles (SERQ page,
// "Metodología" item 2), or asymmetric codes per block of 128 (OffQ page,
// "Metodología" steps 2-3).  For fp16 rows; every other form of the rotation
// runs the butterfly kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_roles.h"

namespace w4a4 {

// b = 2^log2b with 128 <= b <= 4096 (the transform of 16 sub-blocks of 128
// at a time, then for b > 128 the Kronecker factor across them): K a multiple
// of 2048 (of 4096 for b = 4096) up to 16384.
bool rotq_mfma_ok(int64_t M, int64_t K, int log2b);
// Outputs: FP6 tiles, packed tiles (offset-binary, with the row sums in i32,
// when i32 is given) or int8 tiles (qmax 7 or 127), each with one float32
// scale per row; MXFP4 codes in packed tiles with their E8M0 scale tiles
// (mx_scale; scale unused); or, for b = 128, asymmetric codes of every
// (row, block of 128) in packed tiles with float32 scales (scale) and int32
// zero points (i32), [M, K / 128] each.
enum RotMfmaOut { ROT_OUT_F6, ROT_OUT_PACKED, ROT_OUT_I8, ROT_OUT_MX, ROT_OUT_ASYM };
hipError_t launch_rotq_mfma(const _Float16* x, int64_t M, int64_t K, int log2b, RotMfmaOut out_kind,
                            int qmax, uint8_t* q, float* scale, int32_t* i32, uint8_t* mx_scale,
                            hipStream_t st);

// Decode launches (1 <= M <= 64, K up to 8192), FP6 or packed tiles with one
// float32 scale per row: the rotation blocks take one row each, followed by
// lr_rank blocks computing column j of T = X . A (fp16, M <= 16; T as the
// fp16 pair) and ra.blocks blocks reading the weights ahead, all of 256
// threads.
bool rotq_mfma_roles_ok(int64_t M, int64_t K, int log2b);
hipError_t launch_rotq_mfma_roles(const _Float16* x, int64_t M, int64_t K, int log2b, bool f6,
                                  uint8_t* q, float* scale, const _Float16* lr_at, int lr_rank,
                                  void* lr_t, const ReadAhead& ra, hipStream_t st);

}  // namespace w4a4
