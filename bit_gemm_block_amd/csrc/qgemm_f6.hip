// qgemm_f6.hip — the int4 x int4 GEMM of the W4A4 layer (SERQ page, "Resumen
// técnico" §2-3) on the FP6 matrix instruction of gfx950.
//
// Every 4-bit code q in [-7, 7] is an exact FP6 E2M3 value (sign, two
// exponent bits with bias 1, three mantissa bits: 1 = 1.0 x 2^0,
// 3 = 1.5 x 2^1, 7 = 1.75 x 2^2, ...).  v_mfma_scale_f32_16x16x128_f8f6f4
// with both operand formats E2M3 and unit scales therefore multiplies the
// codes exactly and adds the products in float32, and every partial sum is
// an integer of magnitude at most 49 K <= 49 * 16384 < 2^24, so the float32
// accumulator holds sum_k qx[m,k] qw[n,k] exactly: the same integer as the
// int32 accumulation of the int8 instruction.  The FP6 instruction takes 128
// codes per issue where the int8 one takes 64 at the same issue cost, and
// the operands arrive in the instruction's own format (no widening in
// registers).
//
// Operand layout (codes and weights alike, K a multiple of 128): rows in
// blocks of 16, K in steps of 128; the (row block b, step t) tile is 1536
// bytes at (b * (K / 128) + t) * 1536.  Lane l = 16 g + r of the instruction
// takes row r and codes [128 t + 32 g, +32) as 192 bits: their E2M3 fields,
// field p (bits [6p, 6p + 6)) holding code 128 t + 32 g + p / 2 + 16 (p % 2),
// the order of the packing instruction that writes them.  Bytes
// [16 l, 16 l + 16) of the tile are the lane's first four dwords, bytes
// [1024 + 8 l, +8) its last two, so that one wave fills a tile with 1 KB
// copies and reads each half with one conflict-free LDS instruction.
//
// Decomposition as in the int8 pipelined kernel: a workgroup of 2 NWM waves
// owns a (16 TM NWM) x (32 TN) output tile as an NWM x 2 grid of
// (16 TM) x (16 TN) wave tiles, and K advances one 128-code step per
// iteration through a ring of STAGES LDS buffers filled by direct
// global-to-LDS copies of 1 KB issued ahead of their use.  With eight waves
// (NWM = 4) one workgroup fills a CU: a 256 x 128 tile reads 25% fewer
// operand bytes per product than two 128 x 128 ones, and four stages keep
// more iterations of copies in flight to cover stages whose lines miss the
// L2; with 64 x 128 wave tiles (TN = 8) the 256 x 256 tile reads a third
// fewer than 256 x 128.  Weight groups (multiples of 128 codes) are flushed into a float
// accumulator, y = sx sum_g sw_g acc_g, with the group scales of the tile's
// columns staged in LDS before the loop.
#include "w4a4_internal.h"
#include "gemm_common.h"

#include <hip/hip_fp16.h>

#include <type_traits>

namespace w4a4 {
namespace {

constexpr int kF6Tile = 1536;  // bytes of one 16-row x 128-code operand tile
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// One FP6 operand (six dwords) from the two halves of a tile in LDS.
__device__ __forceinline__ i32x8 read_f6(const uint8_t* tile, int lane) {
  const i32x4 p = *reinterpret_cast<const i32x4*>(tile + 16 * lane);
  const i32x2 q = *reinterpret_cast<const i32x2*>(tile + 1024 + 8 * lane);
  const i32x4 q4 = __builtin_shufflevector(q, q, 0, 1, -1, -1);
  return __builtin_shufflevector(p, q4, 0, 1, 2, 3, 4, 5, -1, -1);
}

// 16 x 16 x 128 product of two E2M3 operands (unit scales: E8M0 127).
__device__ __forceinline__ f32x4 mfma_f6(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 2, 2, 0, 127, 0, 127);
}

template <int TM, int TN, int NWM, int STAGES, bool GROUPED, int LRMODE>
__global__ void __launch_bounds__(128 * NWM) qgemm_f6_kernel(GemmArgs a) {
  constexpr int NW = 2 * NWM;  // waves
  constexpr int WM = TM * 16, WN = TN * 16;
  constexpr int BM = NWM * WM, BN = 2 * WN;
  constexpr int A_BYTES = BM / 16 * kF6Tile, B_BYTES = BN / 16 * kF6Tile;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int RUN = 1024;  // bytes of one wave copy (16 per lane)
  static_assert(A_BYTES % RUN == 0 && B_BYTES % RUN == 0, "whole copies per operand");
  constexpr int A_COPIES = A_BYTES / RUN;
  constexpr int COPIES = STAGE / RUN;
  // Copy c goes to wave c % NW.  When the waves do not share the copies
  // evenly, the waves short of one repeat their first copy into a spare 1 KB
  // at the end of the stage buffer, so that every wave issues CPW copies and
  // waits for the same counts.
  constexpr int EXTRA = COPIES % NW;
  constexpr int CPW = COPIES / NW + (EXTRA ? 1 : 0);
  constexpr int STAGE_LDS = STAGE + (EXTRA ? RUN : 0);
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  static_assert((STAGES - 1) * CPW < 64, "in-flight copies exceed vmcnt");
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE_LDS];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE_LDS];
  __shared__ __attribute__((aligned(16))) uint8_t st2[STAGES > 2 ? STAGE_LDS : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st3[STAGES > 3 ? STAGE_LDS : 16];
  auto stage = [&](int sidx) -> uint8_t* {
    switch (sidx) {
      case 0: return st0;
      case 1: return st1;
      case 2: return st2;
      default: return st3;
    }
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar copy bases
  const int wm0 = (wave >> 1) * WM;
  const int wn0 = (wave & 1) * WN;
  // Wait until at most n stages of this wave's copies are in flight.
  auto wait_stages = [&](auto n) { wait_vmcnt<decltype(n)::value * CPW>(); };
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (a.N + BN - 1) / BN;
  int64_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = tmi * BM;
  const int64_t n0 = tni * BN;
  const int nkt = static_cast<int>(a.K / 128);
  const int64_t mblocks = (a.M + 15) / 16, nblocks = (a.N + 15) / 16;
  const int64_t panel = static_cast<int64_t>(nkt) * kF6Tile;  // bytes per row block

  // Copy q of this wave fills LDS bytes [1024 c, 1024 c + 1024) of the stage,
  // c = wave + NW q: lane l copies 16 bytes of the tile that byte
  // 1024 c + 16 l falls in (c past the last copy: copy q = 0's bytes again,
  // into the spare 1 KB).  The base is the operand panel of the tile's first row block
  // (wave-uniform); the per-lane offset reaches the lane's tile, row blocks
  // past the end repeating the last one.
  const uint8_t* base[CPW];
  uint32_t voff[CPW];
  int dst[CPW];
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const bool spare = wave + NW * q >= COPIES;
    const int c = spare ? wave : wave + NW * q;
    const bool is_a = c < A_COPIES;
    const int byte = (is_a ? c : c - A_COPIES) * RUN + 16 * lane;
    const int t = byte / kF6Tile, o = byte % kF6Tile;
    const int64_t first = (is_a ? m0 : n0) / 16;
    const int64_t last = (is_a ? mblocks : nblocks) - 1;
    const int64_t blk = first + t < last ? first + t : last;
    base[q] = (is_a ? a.xq : a.wq) + first * panel;
    voff[q] = static_cast<uint32_t>((blk - first) * panel + o);
    dst[q] = spare ? STAGE : c * RUN;
  }
  auto issue = [&](int kt, uint8_t* buf) {
    const uint32_t b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf));
#pragma unroll
    for (int q = 0; q < CPW; ++q)
      dma16s(base[q] + static_cast<int64_t>(kt) * kF6Tile, voff[q], b + dst[q]);
  };

  f32x4 acc[TM][TN];
  f32x4 facc[GROUPED ? TM : 1][GROUPED ? TN : 1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (GROUPED) facc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  const int iters_per_group = GROUPED ? a.group / 128 : 1;
  const int64_t ngroups = GROUPED ? a.K / a.group : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t gsc[];  // group scales [group][column]
  const int frow = lane & 15;

  auto read_frags = [&](const uint8_t* S, i32x8 (&fa)[TM], i32x8 (&fb)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = read_f6(S + ((wm0 >> 4) + i) * kF6Tile, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = read_f6(S + A_BYTES + ((wn0 >> 4) + j) * kF6Tile, lane);
  };
  // Iteration kt: one instruction per 16 x 16 block.  A weight group's first
  // iteration starts from a zero accumulator; its last adds the group's
  // float value, times the column scale, to facc.
  auto compute = [&](int kt, const i32x8 (&fa)[TM], const i32x8 (&fb)[TN]) {
    const bool first = GROUPED && kt % iters_per_group == 0;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = mfma_f6(fa[i], fb[j], first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i][j]);
    if constexpr (GROUPED) {
      if ((kt + 1) % iters_per_group == 0) {
        const int64_t grp = (kt + 1) / iters_per_group - 1;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = wn0 + j * 16 + frow;
          const float sw = a.sw_f16
                               ? __half2float(reinterpret_cast<const __half*>(gsc)[grp * BN + col])
                               : reinterpret_cast<const float*>(gsc)[grp * BN + col];
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[i][j][r] = fmaf(acc[i][j][r], sw, facc[i][j][r]);
        }
      }
    }
  };

  // Group scales of the tile's columns, [group][column], staged before any
  // copy is in flight (loaded inside the loop they would wait for the copies).
  if constexpr (GROUPED) {
    const int esz = a.sw_f16 ? 2 : 4;
    for (int e = tid; e < BN * ngroups; e += 128 * NWM) {
      const int col = e % BN;
      const int64_t grp = e / BN;
      int64_t n = n0 + col;
      n = n < a.N ? n : a.N - 1;
      if (esz == 2)
        reinterpret_cast<__half*>(gsc)[e] = reinterpret_cast<const __half*>(a.sw)[n * ngroups + grp];
      else
        reinterpret_cast<float*>(gsc)[e] = reinterpret_cast<const float*>(a.sw)[n * ngroups + grp];
    }
    __syncthreads();
  }

  // One fragment set per iteration, read right before its instructions, when
  // the accumulators take too many registers for a second set: weight groups
  // (group and float accumulators) and 64 x 128 wave tiles.
  constexpr bool SB = GROUPED || TM * TN > 16;
  if constexpr (!SB) {
    // Prologue: the first STAGES stages in flight, stage 0 visible, its
    // fragments read.
#pragma unroll
    for (int sidx = 0; sidx < STAGES; ++sidx)
      if (sidx < nkt) issue(sidx, stage(sidx));
    if (nkt >= STAGES)
      wait_stages(std::integral_constant<int, STAGES - 1>{});
    else
      wait_vmcnt<0>();
    stage_barrier();
    i32x8 fa0[TM], fa1[TM], fb0[TN], fb1[TN];
    read_frags(stage(0), fa0, fb0);

    // Iteration kt (buffer kt % STAGES): once stage kt + 1 has landed and the
    // barrier has retired every wave's reads of stage kt, that buffer is
    // refilled with stage kt + STAGES and stage kt + 1's fragments are read
    // into the other register set; stage kt's instructions run meanwhile.
    auto iterate = [&](int kt, int sbuf, i32x8 (&fac)[TM], i32x8 (&fbc)[TN], i32x8 (&fan)[TM],
                       i32x8 (&fbn)[TN], bool steady) {
      // The reads are unconditional (on the last iteration they read a stale,
      // in-bounds buffer) so that no branch joins between them and the matrix
      // instructions.
      if (steady || kt + STAGES <= nkt)
        wait_stages(std::integral_constant<int, STAGES - 2>{});
      else
        wait_vmcnt<0>();
      stage_barrier();
      if (steady || kt + STAGES < nkt) issue(kt + STAGES, stage(sbuf));
      read_frags(stage((sbuf + 1) % STAGES), fan, fbn);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the instructions
      compute(kt, fac, fbc);
    };
    // Blocks of 2 * STAGES iterations (so that buffer index and register set
    // are compile-time constants in each unrolled copy) while every iteration
    // refills a stage; the remaining iterations, fewer than 3 * STAGES, run
    // unrolled with checks.
    int kt0 = 0;
    for (; kt0 + 3 * STAGES <= nkt; kt0 += 2 * STAGES) {
#pragma unroll
      for (int u = 0; u < 2 * STAGES; ++u) {
        if (u & 1)
          iterate(kt0 + u, u % STAGES, fa1, fb1, fa0, fb0, true);
        else
          iterate(kt0 + u, u % STAGES, fa0, fb0, fa1, fb1, true);
      }
    }
#pragma unroll
    for (int u = 0; u < 3 * STAGES; ++u) {
      const int kt = kt0 + u;
      if (kt < nkt) {
        if (u & 1)
          iterate(kt, u % STAGES, fa1, fb1, fa0, fb0, false);
        else
          iterate(kt, u % STAGES, fa0, fb0, fa1, fb1, false);
      }
    }
  } else {
    // One fragment set, read right before the instructions (the other waves
    // of the SIMD cover the read latency).  Prologue: stages 0 .. STAGES - 2
    // in flight.
#pragma unroll
    for (int sidx = 0; sidx < STAGES - 1; ++sidx)
      if (sidx < nkt) issue(sidx, stage(sidx));
    // Iteration kt: once stage kt has landed and the barrier has retired
    // every wave's reads of stage kt - 1, that buffer takes stage
    // kt + STAGES - 1; stage kt's fragments are read and multiplied.
    auto iterate = [&](int kt, int sbuf, bool steady) {
      if (steady || kt + STAGES - 1 <= nkt)
        wait_stages(std::integral_constant<int, STAGES - 2>{});
      else
        wait_vmcnt<0>();
      stage_barrier();
      if (steady || kt + STAGES - 1 < nkt)
        issue(kt + STAGES - 1, stage((sbuf + STAGES - 1) % STAGES));
      i32x8 fa[TM], fb[TN];
      read_frags(stage(sbuf), fa, fb);
      compute(kt, fa, fb);
    };
    int kt0 = 0;
    for (; kt0 + 2 * STAGES <= nkt; kt0 += STAGES) {
#pragma unroll
      for (int u = 0; u < STAGES; ++u) iterate(kt0 + u, u, true);
    }
#pragma unroll
    for (int u = 0; u < 2 * STAGES; ++u) {
      const int kt = kt0 + u;
      if (kt < nkt) iterate(kt, u % STAGES, false);
    }
  }

  // Epilogue: y = acc * (sx * sw) (per channel) or facc * sx (groups), plus
  // the low-rank term; acc (int32) on request, per channel only.
  const bool interior = (m0 + BM <= a.M) && (n0 + BN <= a.N);
  const bool want_y = a.y != nullptr;
  const int64_t mlane = m0 + wm0 + (lane >> 4) * 4;
  const int64_t nlane = n0 + wn0 + (lane & 15);
  float sxr[TM][4], swr[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    f32x4 sv = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t mf = mlane + i * 16;  // a multiple of 4: x_scale + mf is 16-byte aligned
    if (want_y) {
      if (mf + 3 < a.M) {
        sv = *reinterpret_cast<const f32x4*>(a.sx + mf);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mf + r < a.M) sv[r] = a.sx[mf + r];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sxr[i][r] = sv[r];
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t n = nlane + j * 16;
    swr[j] = (GROUPED || !want_y || n >= a.N) ? 1.f : load_scale(a.sw, n, a.sw_f16);
  }

  // fp16 low-rank term: the first 32 ranks of the wave's Bt rows are loaded
  // before the stores, and each row block's T pair once (further ranks go
  // through add_lowrank, with the same instructions in the same order).
  constexpr bool LRP = LRMODE == LR_F16;
  const half8 lr_z = {0, 0, 0, 0, 0, 0, 0, 0};
  const int lr_koff = (lane >> 4) * 8;
  const bool lr_kok = want_y && lr_koff < a.rank;
  half8 lr_b[LRP ? TN : 1];
  if constexpr (LRP) {
    const _Float16* bt = static_cast<const _Float16*>(a.B);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t nr = n0 + wn0 + j * 16 + (lane & 15);
      lr_b[j] = (lr_kok && nr < a.N) ? *reinterpret_cast<const half8*>(bt + nr * a.rank + lr_koff)
                                     : lr_z;
    }
  }

  auto emit = [&](auto fast) {
    constexpr bool FAST = decltype(fast)::value;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      half8 lr_hi = lr_z, lr_lo = lr_z;
      if constexpr (LRP) {
        const int64_t mr = m0 + wm0 + i * 16 + (lane & 15);
        if (lr_kok && mr < a.M) {
          const _Float16* th = static_cast<const _Float16*>(a.t);
          lr_hi = *reinterpret_cast<const half8*>(th + mr * a.rank + lr_koff);
          lr_lo = *reinterpret_cast<const half8*>(th + (a.M + mr) * a.rank + lr_koff);
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = nlane + j * 16;
        f32x4 yv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (GROUPED)
            yv[r] = facc[i][j][r] * sxr[i][r];
          else
            yv[r] = acc[i][j][r] * (sxr[i][r] * swr[j]);
        }
        if constexpr (LRP) {
          if (want_y) {
            yv = __builtin_amdgcn_mfma_f32_16x16x32_f16(lr_lo, lr_b[j], yv, 0, 0, 0);
            yv = __builtin_amdgcn_mfma_f32_16x16x32_f16(lr_hi, lr_b[j], yv, 0, 0, 0);
            if (a.rank > 32)
              yv = add_lowrank<LRMODE>(a, yv, m0 + wm0 + i * 16, n0 + wn0 + j * 16, lane, 32);
          }
        } else if constexpr (LRMODE != LR_NONE) {
          if (want_y) yv = add_lowrank<LRMODE>(a, yv, m0 + wm0 + i * 16, n0 + wn0 + j * 16, lane);
        }
        const int64_t mb = mlane + i * 16;
        if constexpr (FAST) {
          float* yp = a.y + mb * a.N + n;
#pragma unroll
          for (int r = 0; r < 4; ++r) yp[r * a.N] = yv[r];
        } else if (n < a.N) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (mb + r < a.M) {
              if (want_y) a.y[(mb + r) * a.N + n] = yv[r];
              if (!GROUPED && a.acc)
                a.acc[(mb + r) * a.N + n] = static_cast<int32_t>(acc[i][j][r]);
            }
          }
        }
      }
    }
  };
  if (interior && want_y && (GROUPED || !a.acc))
    emit(std::true_type{});
  else
    emit(std::false_type{});
}

template <int TM, int TN, int NWM, int STAGES>
hipError_t launch_f6(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = 16 * TM * NWM, BN = 32 * TN;
  const dim3 grid(static_cast<unsigned>(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN)));
  size_t shm = 0;
  if (a.group > 0) shm = static_cast<size_t>(BN) * (a.K / a.group) * (a.sw_f16 ? 2 : 4);
#define W4A4_F6_CASE(G, LR)                                                                  \
  if ((a.group > 0) == G && a.lr_mode == LR) {                                             \
    hipLaunchKernelGGL((qgemm_f6_kernel<TM, TN, NWM, STAGES, G, LR>), grid,                \
                       dim3(128 * NWM), shm, st, a);                                       \
    return hipGetLastError();                                                              \
  }
  W4A4_F6_CASE(false, LR_NONE) W4A4_F6_CASE(false, LR_F16) W4A4_F6_CASE(false, LR_F32)
  if constexpr (TM * TN <= 16) {  // grouped wave tiles of at most 64 x 64 (registers)
    W4A4_F6_CASE(true, LR_NONE) W4A4_F6_CASE(true, LR_F16) W4A4_F6_CASE(true, LR_F32)
  }
#undef W4A4_F6_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qgemm_f6(const GemmArgs& a, hipStream_t st) {
  // The tiled kernels write the int32 product only when ungrouped: a grouped
  // request for acc runs the ungrouped kernel for it (the integer product
  // does not depend on the weight groups).
  if (a.group > 0 && a.acc) {
    GemmArgs ia = a;
    ia.group = 0;
    ia.y = nullptr;
    ia.lr_mode = LR_NONE;
    hipError_t e = launch_f6<4, 4, 4, 4>(ia, st);
    if (e != hipSuccess || !a.y) return e;
  }
  GemmArgs ya = a;
  if (a.group > 0) {
    ya.acc = nullptr;
    // Eight waves (256 x 128 tiles), as many stages of 37 KB as fit beside
    // the staged group scales in the 160 KB of LDS.
    const size_t shm = size_t{128} * (a.K / a.group) * (a.sw_f16 ? 2 : 4);
    if (3 * 37888 + shm <= 163840) return launch_f6<4, 4, 4, 3>(ya, st);
    return launch_f6<4, 4, 4, 2>(ya, st);
  }
  // Per-channel scales, largest tile first:
  // * eight waves of 64 x 128 (256 x 256 tiles, one workgroup per CU, three
  //   stages of 48 KB) when the tiles fill at least 90% of their rounds on
  //   the 256 CUs: a third fewer operand bytes per product than 256 x 128
  //   (4096 x 28672 x 4096: 19% faster, 4096 x 4096 x 14336: 11%,
  //   4096 x 4096 x 4096: 7%; 384 tiles, 1.5 rounds: 3% slower);
  // * eight waves of 64 x 64 (256 x 128 tiles, four stages) for long K or
  //   many tiles;
  // * two four-wave 128 x 128 workgroups per CU (three stages) otherwise
  //   (the 2048- and 4096-row products with K = 4096: 3-5% faster).
  constexpr int64_t kCUs = 256;  // MI355X
  const int64_t tiles8 = ((a.M + 255) / 256) * ((a.N + 127) / 128);
  const int64_t tiles16 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  const int64_t rounds16 = (tiles16 + kCUs - 1) / kCUs;
  if (tiles16 >= kCUs && 10 * tiles16 >= 9 * rounds16 * kCUs)
    return launch_f6<4, 8, 4, 3>(ya, st);
  if (a.K >= 8192 || tiles8 >= 2048) return launch_f6<4, 4, 4, 4>(ya, st);
  return launch_f6<4, 4, 2, 3>(ya, st);
}

}  // namespace w4a4
