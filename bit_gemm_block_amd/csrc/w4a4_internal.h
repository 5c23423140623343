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

// Chooses the segment shape for (K, b, group); returns false if none fits.
bool rotq_plan(int64_t K, int log2b, int64_t gsz, int max_lds, RotqPlan* plan);

enum RotqMode { ROTQ_ROTATE = 0, ROTQ_QUANT = 1 };

// x: [M, K] (f16 if x_f16 else f32).  mode ROTATE writes xrot [M, K] f32;
// mode QUANT writes q [M, K/2] and one scale per group of gsz elements
// (gsz == K: per row) as f32 or f16 (scale_f16).
hipError_t launch_rotq(const void* x, bool x_f16, int64_t M, int64_t K,
                       int log2b, int mode, int64_t gsz, bool scale_f16,
                       float* xrot, uint8_t* q, void* scale,
                       const RotqPlan& plan, hipStream_t st);

// ---- int4 GEMM (qgemm.hip) -------------------------------------------------
struct GemmArgs {
  const uint8_t* xq;     // [M, K/2]
  const float* sx;       // [M]
  const uint8_t* wq;     // [N, K/2]
  const void* sw;        // [N] or [N, K/group]
  int sw_f16;
  int group;             // 0 = per channel, else multiple of 64
  int64_t M, N, K;
  float* y;              // [M, N] or null
  int32_t* acc;          // [M, N] or null
  const float* t;        // [M, rank] (X.A) or null
  const void* B;         // [rank, N] or null
  int b_f16;
  int rank;
};

hipError_t launch_qgemm(const GemmArgs& a, hipStream_t st);

// ---- low-rank projection (lowrank.hip) -------------------------------------
hipError_t launch_lowrank_project(const void* x, bool x_f16, const void* A,
                                  int64_t M, int64_t K, int rank, float* t,
                                  hipStream_t st);

}  // namespace w4a4
