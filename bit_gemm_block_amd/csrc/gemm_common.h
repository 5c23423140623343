// gemm_common.h — device helpers shared by the GEMM kernels: operand vector
// types, scale loads, the low-rank epilogue term, the XCD-aware tile order,
// and the direct-to-LDS copies with their waits and barrier.
#pragma once
#include "w4a4_internal.h"

#include <hip/hip_fp16.h>

namespace w4a4 {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float load_scale(const void* p, int64_t i, int f16) {
  if (f16) return __half2float(reinterpret_cast<const __half*>(p)[i]);
  return reinterpret_cast<const float*>(p)[i];
}

// Adds the low-rank term of one 16x16 output block to its dequantized values.
// Fragment layout of a 16x16 MFMA result: lane holds rows 4*(lane>>4)+i of
// column lane&15.
template <int LRMODE>
__device__ __forceinline__ f32x4 add_lowrank(const GemmArgs& a, f32x4 v, int64_t mblk, int64_t nblk,
                                             int lane, int c_begin = 0) {
  if constexpr (LRMODE == LR_F16) {
    const int64_t mr = mblk + (lane & 15);  // operand row (A side)
    const int64_t nr = nblk + (lane & 15);  // operand row of Bt (B side)
    const int koff = (lane >> 4) * 8;
    const _Float16* th = static_cast<const _Float16*>(a.t);
    const _Float16* tl = th + a.M * a.rank;
    const _Float16* bt = static_cast<const _Float16*>(a.B);
    const half8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int c = c_begin; c < a.rank; c += 32) {
      const int j = c + koff;
      const bool jok = j < a.rank;
      const half8 hi = (jok && mr < a.M) ? *reinterpret_cast<const half8*>(th + mr * a.rank + j) : z;
      const half8 lo = (jok && mr < a.M) ? *reinterpret_cast<const half8*>(tl + mr * a.rank + j) : z;
      const half8 bb = (jok && nr < a.N) ? *reinterpret_cast<const half8*>(bt + nr * a.rank + j) : z;
      v = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, bb, v, 0, 0, 0);
      v = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, bb, v, 0, 0, 0);
    }
  } else if constexpr (LRMODE == LR_F32) {
    const int64_t n = nblk + (lane & 15);
    if (n < a.N) {
      const float* t = static_cast<const float*>(a.t);
      const float* bt = static_cast<const float*>(a.B) + n * a.rank;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = mblk + (lane >> 4) * 4 + i;
        if (m < a.M) {
          float s = 0.f;
          for (int q = 0; q < a.rank; ++q) s = fmaf(t[m * a.rank + q], bt[q], s);
          v[i] += s;
        }
      }
    }
  }
  return v;
}

// Maps a workgroup index to an output tile: consecutive workgroup indices go
// to different XCDs (round robin), so the tiles of one XCD are taken as one
// contiguous range of a grouped ordering (groups of GM tile rows, tile
// columns fastest inside a group) and land as a compact block.
__device__ __forceinline__ void tile_of(int64_t bid, int64_t tiles_m, int64_t tiles_n, int64_t* tm,
                                        int64_t* tn) {
  const int64_t T = tiles_m * tiles_n;
  int64_t L = bid;
  if ((T & 7) == 0) L = (bid & 7) * (T >> 3) + (bid >> 3);
  constexpr int64_t GM = 4;
  const int64_t per_group = GM * tiles_n;
  const int64_t g = L / per_group;
  const int64_t first_m = g * GM;
  const int64_t gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int64_t r = L % per_group;
  *tm = first_m + r % gsize;
  *tn = r / gsize;
}

// s_waitcnt immediate that waits for vmcnt <= n only (expcnt and lgkmcnt at
// their maximum); vmcnt is split over bits [3:0] and [15:14].
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

// 16 bytes per lane from global memory straight into LDS: lane l writes
// [lds_base + 16 l, lds_base + 16 l + 16).  Issued from asm so that the
// compiler does not treat the copy as an LDS store it must wait for before
// every LDS read; the kernel waits for the copies itself (wait_vmcnt).  The
// asm writes no register, so nothing it produces can be consumed early.
__device__ __forceinline__ void dma16(const uint8_t* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

// 4 bytes per lane straight into LDS: lane l writes [lds_base + 4 l, +4).
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

// The same copy from a wave-uniform base address (SGPR pair) plus a 32-bit
// per-lane offset: the per-iteration address arithmetic stays scalar.
__device__ __forceinline__ void dma16s(const uint8_t* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_base)
               : "memory", "m0");
}

// Workgroup barrier that also waits for this wave's own LDS reads: no wave
// passes it while another may still read a stage that is about to be
// refilled.  Written as asm with a memory clobber so that the compiler keeps
// LDS accesses on their side of it and adds no wait for the in-flight
// direct-to-LDS copies (each stage is its own LDS array, so it can tell the
// stage being read from the stages being filled).
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace
}  // namespace w4a4
