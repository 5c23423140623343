// Internal launch interface between the C-ABI host layer (api.cpp) and the
// HIP kernels (rotq.hip, qgemm.hip, lowrank.hip).  Shapes reaching these
// launchers have already been validated by the host layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

// ---- rotation + quantization (rotq.hip) -----------------------------------
struct RotqPlan {
  int L = 0;             // lanes per segment
  int R = 0;             // elements per lane
  int segs_per_row = 0;  // K / (L * R)
  int rows_per_wg = 0;
  int threads = 0;       // block size (multiple of 64)
  int lds_bytes = 0;
  int nslots = 0;        // cross-segment reduction slots per workgroup
};

// Chooses the segment shape for (K, b, group), with at least min_r elements
// per lane; returns false if none fits.
bool rotq_plan(int64_t M, int64_t K, int log2b, int64_t gsz, int max_lds, RotqPlan* plan,
               int min_r = 8);

// ROTQ_QUANT_I8 writes one int8 code per byte, each group of 8 elements in
// the order 0,2,4,6,1,3,5,7 (the K order of the GEMM's nibble widening): the
// activation operand format the fused layer hands to the GEMM.  The _TILED
// modes write the same bytes in 16-row x 128-code tiles (see include/w4a4.h,
// W4A4_WEIGHTS_TILED and W4A4_CODES_I8_TILED).
enum RotqMode {
  ROTQ_ROTATE = 0,
  ROTQ_QUANT = 1,
  ROTQ_QUANT_I8 = 2,
  ROTQ_QUANT_TILED = 3,
  ROTQ_QUANT_I8_TILED = 4,
  // FP6 E2M3 codes in 16-row x 128-code tiles of 1536 bytes (see
  // include/w4a4.h, W4A4_CODES_F6_TILED); needs a plan with R >= 16.
  ROTQ_QUANT_F6 = 5
};

// x: [M, K] (f16 if x_f16 else f32).  mode ROTATE writes xrot [M, K] f32;
// mode QUANT writes q [M, K/2] (QUANT_I8: q [M, K]) and one scale per group of
// gsz elements (gsz == K: per row) as f32 or f16 (scale_f16).
// Options: the code range (qmax), and optional extra work in the same launch
// (decode prologue): the low-rank
// projection t = x . A for M <= 16 and fp16 inputs (lr_rank workgroups,
// written as the fp16 pair), and a read of the GEMM's weight operand in
// pf_units units of pf_unit bytes (the last one pf_last bytes) by pf_blocks
// workgroups (a multiple of 8), so that the GEMM finds it in cache.
struct RotqExtras {
  int qmax = 7;  // 127: 8-bit activation codes (int8 code modes only)
  // Asymmetric uint4 codes (packed modes, float32 scales): one scale and one
  // int32 zero point per group of gsz elements, zero points written here;
  // the nibbles hold q - 8.
  int32_t* asym_zero = nullptr;
  // Tiled weights only: residual codes of channels [0, res_r) in
  // ceil(res_r / 128) extra tiles after each row block's K / 128 tiles.
  int res_r = 0;
  // MXFP4 (packed modes): E2M1 codes and one E8M0 byte per 32 elements,
  // written here ([M, K/32] row-major, or in 64-byte tiles with the tiled
  // codes: byte (g * 16 + r) of tile (row block, t) is block 4 t + g of row r).
  uint8_t* mx_scale = nullptr;
  // Offset-binary packed codes (packed tiled mode): every byte XOR 0x08, and
  // the sum of each row's codes at odd channels written here ([rows] int32).
  int32_t* ob_sum = nullptr;
  const void* lr_at = nullptr;
  int lr_rank = 0;
  void* lr_t = nullptr;
  const uint8_t* pf = nullptr;
  int64_t pf_unit = 0;
  int64_t pf_units = 0;
  int64_t pf_last = 0;
  int pf_blocks = 0;
};

hipError_t launch_rotq(const void* x, bool x_f16, int64_t M, int64_t K,
                       int log2b, int mode, int64_t gsz, bool scale_f16,
                       float* xrot, uint8_t* q, void* scale,
                       const RotqPlan& plan, hipStream_t st,
                       const RotqExtras* extras = nullptr);

// ---- int4 GEMM (qgemm.hip) -------------------------------------------------
// Low-rank epilogue kinds: none; fp16 (t = fp16 pair t_hi [M, r] followed by
// t_lo [M, r], B = Bt [N, r] fp16); fp32 (t = [M, r], B = Bt [N, r] fp32).
enum LowRankMode { LR_NONE = 0, LR_F16 = 1, LR_F32 = 2 };

struct GemmArgs {
  const uint8_t* xq;     // [M, K/2] packed, or [M, K] int8 when a_i8
  const float* sx;       // [M]
  const uint8_t* wq;     // [N, K/2]
  const void* sw;        // [N] or [N, K/group]
  int sw_f16;
  int group;             // 0 = per channel, else multiple of 64
  int64_t M, N, K;
  float* y;              // [M, N] or null
  int32_t* acc;          // [M, N] or null
  const void* t;         // X.A as described by lr_mode, or null
  const void* B;         // Bt [N, rank], or null
  int lr_mode;           // LowRankMode
  int rank;
  int a_i8;              // activation codes as int8 (ROTQ_QUANT_I8 layout)
  int tiled;             // int8 codes and weights both in the 16 x 128 tiled layouts
  // Asymmetric activation groups (zx non-null; packed tiled codes holding
  // q - 8, tiled weights, per-channel weight scales, no acc): sx is
  // [M, K/agroup], zx [M, K/agroup] the zero points, wsum [N, K/agroup] the
  // weight codes summed over each group.
  const int32_t* zx;
  const int32_t* wsum;
  int agroup;
  // In-GEMM residual (res non-zero; packed tiled codes, tiled weights whose
  // row blocks hold K / 128 + res_iters tiles, no groups, no low-rank term):
  // the last res_iters (>= 0) iterations multiply the first 128 * res_iters
  // code columns again, by the residual tiles, at 1/8 the weight of the main
  // sum; acc holds 8 sum_k + sum_{k<r}.
  int res;
  int res_iters;
  // MXFP4 (mx_xs non-null): xq and wq hold E2M1 codes in the packed tiled
  // layout, mx_xs and mx_ws their E8M0 scales in 64-byte tiles; sx, sw unused.
  const uint8_t* mx_xs;
  const uint8_t* mx_ws;
  // Offset-binary operands.  w_ob: the tiled weights are in the offset-binary
  // layout.  ob_sa non-null: the packed tiled codes are too (every byte XOR
  // 0x08), ob_sa [M] and ob_sb [N] being the sums of the activation codes at
  // odd and of the weight codes at even channels; the accumulator then holds
  // 16 sum_k qx qw + 128 (ob_sa[m] + ob_sb[n]).
  int w_ob;
  const int32_t* ob_sa;
  const int32_t* ob_sb;
  // FP6 E2M3 operands (xq and wq in the FP6 tiled layouts): launch_qgemm
  // hands the call to launch_qgemm_f6.
  int f6;
};

hipError_t launch_qgemm(const GemmArgs& a, hipStream_t st);

// ---- int4 GEMM on the FP6 matrix instruction (qgemm_f6.hip) -----------------
// xq and wq in the FP6 tiled layouts (W4A4_CODES_F6_TILED and
// W4A4_WEIGHTS_TILED_F6), K a multiple of 128, weight groups multiples of 128;
// sx, sw, y, acc, the low-rank term and group as in GemmArgs.
hipError_t launch_qgemm_f6(const GemmArgs& a, hipStream_t st);

// ---- the layer (api.cpp) ----------------------------------------------------
// w4a4_qlinear_forward (qmax 7) and w4a8_qlinear_forward (qmax 127) with the
// given workspace: validation, planning and launches; returns a w4a4_status.
int qlinear_impl(const void* x, int x_dtype, const uint8_t* wq, int w_layout,
                 const void* w_scale, int w_scale_dtype, int64_t M, int64_t N, int64_t K,
                 int64_t had_block, int64_t w_group, const void* At, const void* Bt,
                 int64_t rank, float* y, void* workspace, size_t ws_bytes, void* stream,
                 int qmax);
// Records e as the HIP error behind a W4A4_ERR_HIP and returns that status.
int hip_status(hipError_t e);

// ---- weight group sums (offq.hip) ------------------------------------------
// out[n, g] = sum of the signed weight codes of row n over K-group g
// (group a multiple of 8 dividing K); wq row-major [N, K/2] or tiled.
hipError_t launch_weight_group_sums(const uint8_t* wq, bool tiled, int64_t N, int64_t K,
                                    int group, int32_t* out, hipStream_t st);

// Tiled int4 weights -> offset-binary tiled weights followed by the per-row
// sums of the codes at even channels (rows a multiple of 16, K of 128).
hipError_t launch_weights_to_ob(const uint8_t* wq, int64_t rows, int64_t K, uint8_t* out,
                                hipStream_t st);

// ---- low-rank projection (lowrank.hip) -------------------------------------
// t = x [M, K] . At[rank, K]^T.  fp16 inputs: pair_out writes the fp16 pair
// (t_hi [M, rank], then t_lo [M, rank]) into t, otherwise float32 [M, rank].
// fp32 inputs always write float32.
hipError_t launch_lowrank_project(const void* x, bool x_f16, const void* at,
                                  int64_t M, int64_t K, int rank, void* t,
                                  bool pair_out, hipStream_t st);

}  // namespace w4a4
