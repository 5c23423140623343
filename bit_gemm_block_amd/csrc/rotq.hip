// rotq.hip — block Hadamard rotation fused with symmetric int4 quantization.
//
// The rotation is the OffQ offsetting transform (OffQ page, "Metodología",
// steps 2-3): every contiguous block of b channels of a row is multiplied by
// the Sylvester Hadamard matrix (first row all ones) scaled by 1/sqrt(b).
// The quantizer is the per-token (or per weight group) symmetric int4 absmax
// quantizer of SERQ's 4-bit path (SERQ page, "Resumen técnico" §1-2), or its
// 8-bit form (qmax 127) for the activations of W4A8 layers (DynamicPTQ page,
// "Metodología" §2).
//
// Work decomposition.  A row of K elements is cut into segments of S = L*R
// elements; L consecutive lanes own a segment and every lane keeps R float32
// values in registers.  The fast Walsh-Hadamard transform runs in three
// passes, each on register-resident data with compile-time butterfly pairs:
//   1. load pass: the row is read with coalesced 16-byte loads (V = 8 fp16 or
//      4 fp32 elements per load); element bits [0, log2 V) are in registers
//      (fp16: bit 0 is transformed while widening, one v_fma_mix_f32 per value);
//   2. column pass: after a trip through LDS a lane holds, for a few fixed
//      columns of the [L][R] view of the segment, all values of the row
//      bits the block spans; element bits [log2 R, log2 b) are transformed;
//   3. row pass: after a second trip a lane holds one row of R contiguous
//      elements; element bits [log2 V, min(log2 b, log2 R)) are transformed.
// The row pass layout is also the output layout: R contiguous codes per lane
// pack into R/2 contiguous bytes.  LDS rows are XOR-swizzled at float4
// granularity so that row reads (ds_read_b128) and column reads (ds_read_b32)
// are free of bank conflicts for R = 64.
//
// Residual (weights, tiled; SERQ page, "Metodología" items 2-3): for the
// first r channels (the salient ones, permuted to the front offline) the
// kernel also writes the 4-bit residual q_r = clamp(rint(e / (s/8)), -8, 7),
// e = RN(x~ - RN(s q)), taken against the stored scale, into res_pad / 128
// extra tiles that follow each row block's K / 128 code tiles.
//
// MXFP4 mode (SERQ page, "Metodología" item 2, read as the OCP
// microscaling format): every 32 consecutive elements share the scale 2^e,
// e = max(floor(log2(max|x~|)) - 2, -127), stored as the byte e + 127; each
// element is x~ 2^-e (exact) rounded to the nearest E2M1 value
// {0, .5, 1, 1.5, 2, 3, 4, 6} with ties to the even encoding and saturation
// at 6, the quotient's sign (negative zero included) in bit 3.  The
// rounding is the hardware's packed conversion (two quotients per
// instruction, scale 1), which follows exactly this rule.
//
// Asymmetric mode (OffQ page, "Metodología" steps 2-3): one scale and zero
// point per token and Hadamard block, s = (max - min) / 15,
// z = rint(-min / s) (an integer, not clamped), q = clamp(rint(x~ / s) + z,
// 0, 15), with a group of equal values c taking the range spanned by c and
// 0.  The stored nibble is q - 8 in two's complement (q with its top bit
// flipped), so that the codes feed the same signed int8 widening as the
// symmetric ones.
//
// Quantization is exact with respect to the float32 rule
// q = clamp(rint(fl(x~ / s)), -7, 7) with x~ = RN(y * rs): the quotient is
// formed as x~ * RN(1/s) and refined twice by Markstein's step (residual
// r = x~ - q s by fma, then q' = RN(q + r RN(1/s))); once q is within one ulp
// of x~ / s, the refined value is the correctly rounded quotient.  Quotients
// of magnitude >= 1/4 keep every intermediate normal for 2^-100 <= s <= 2^100,
// and smaller ones give code 0 whatever their last bits; scales outside that
// range take the IEEE division.  The clamp is applied only where it can act,
// under float16 scales below 2^-14; with a float32 or normal float16 scale
// every rounded quotient already lies in [-qmax, qmax].  When rs is a power
// of two the quotient is formed as y / (s / rs), the same real number.
#include "w4a4_internal.h"
#include "lowrank_rows.h"
#include "decode_roles.h"
#include "rotq_mfma.h"

#include <hip/hip_fp16.h>
#include <type_traits>

#pragma clang fp contract(off)

namespace w4a4 {
namespace {

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v >> 1); }

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct Piece;
template <> struct Piece<float> {
  static constexpr int V = 4;
  __device__ static void load(const float* p, float* out) {
    const float4 f = *reinterpret_cast<const float4*>(p);
    out[0] = f.x; out[1] = f.y; out[2] = f.z; out[3] = f.w;
  }
};
template <> struct Piece<_Float16> {
  static constexpr int V = 8;
  __device__ static void load(const _Float16* p, float* out) {
    const half8 h = *reinterpret_cast<const half8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = static_cast<float>(h[i]);
  }
};

// First butterfly stage straight from a pair of fp16 values packed in one
// dword (element 2i in the low half, 2i + 1 in the high half): v_fma_mix_f32
// widens its fp16 operands exactly and rounds once, so lo * 1 + hi and
// hi * (-1) + lo equal the float32 sum and difference of the widened values.
__device__ __forceinline__ float mix_sum(uint32_t w) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(w));
  return r;
}
__device__ __forceinline__ float mix_dif(uint32_t w) {
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(w));
  return r;
}

// Butterflies on register-index bits [LO, HI) of v: for every pair
// (r, r | 2^st) with bit st of r clear, (a, b) -> (a + b, a - b).  The stage
// range is a compile-time constant so that all stages form one straight-line
// block in which the register allocator renames instead of copying.
template <int LO, int HI, int N>
__device__ __forceinline__ void fwht_stages(float (&v)[N]) {
#pragma unroll
  for (int st = LO; st < HI; ++st) {
#pragma unroll
    for (int r = 0; r < N; ++r) {
      if ((r & (1 << st)) == 0) {
        const float a = v[r], b = v[r | (1 << st)];
        v[r] = a + b;
        v[r | (1 << st)] = a - b;
      }
    }
  }
}

// Stages [LO, hi) for a run-time hi in [LO, HI]: one uniform branch picks a
// fully unrolled stage sequence.
template <int LO, int HI, int N>
__device__ __forceinline__ void fwht_bits_upto(float (&v)[N], int hi) {
  if constexpr (HI > LO) {
    if (hi >= HI) {
      fwht_stages<LO, HI>(v);
    } else {
      fwht_bits_upto<LO, HI - 1>(v, hi);
    }
  }
}

struct RotqKArgs {
  const void* x;
  int64_t M;
  int K;
  int log2b;
  float rs;          // float32(1 / sqrt(b))
  int mode;          // RotqMode
  int gsz;           // elements per scale group (K = one scale per row)
  int scale_f16;
  float fqmax;       // largest code: 7 (int4) or 127 (int8 activations)
  int asym;          // asymmetric uint4 codes with zero points (packed modes)
  int32_t* zero;     // asym: zero points, laid out like the scales
  int mx;            // MXFP4: E2M1 codes, one E8M0 scale byte per 32 elements
  int res_r;         // residual codes for channels [0, res_r) (tiled weights)
  int res_pad;       // res_r rounded up to 128 (0: no residual)
  int64_t tile_stride;  // 128-code tiles per 16-row block of the tiled output
  uint8_t* mx_scale;    // MXFP4 scale bytes: [M, K/32], or tiled (64 B per 16 x 128 tile)
  int32_t* ob_sum;      // offset-binary packed codes: per-row sums of the odd channels' codes
  float* xrot;
  uint8_t* q;
  void* scale;
  int segs_per_row;
  int rows_per_wg;
  int nslots;
  // Extra block roles after the rotation blocks (all zero/null when unused):
  int nrot_blocks;        // blocks [0, nrot_blocks) rotate and quantize
  const void* lr_at;      // then lr_rank blocks: column j of T = X . A (fp16, M <= 16)
  int lr_rank;
  void* lr_t;
  ReadAhead ra;           // then ra.blocks blocks read the weights ahead (decode_roles.h)
};

// Order-preserving map of float32 onto uint32 (unsigned compare = float
// compare), for LDS atomic max of signed values, and its inverse.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_val(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Swizzled float offset of element (i, j) of a segment stored as [L][R].
template <int R>
__device__ __forceinline__ int lds_off(int i, int j) {
  constexpr int R4 = R / 4;
  return i * R + ((((j >> 2) ^ (i & (R4 - 1)))) << 2) + (j & 3);
}

// Quantizer variants fixed at compile time.  QV_ANY: every mode and role,
// the quotient form chosen at run time.  QV_FOLD / QV_PLAIN: symmetric codes
// with float32 scales (no clamp needed), no extra roles, no MXFP4,
// asymmetric or residual output, the quotient taken as y / (s / rs) (rs a
// power of two) or as (y rs) / s.  The kernel then carries only the code it
// runs: with fp16 input not even the IEEE-division fallback.
enum QuantVariant { QV_ANY = 0, QV_FOLD = 1, QV_PLAIN = 2 };

// LB >= 0: the Hadamard block is 2^LB, fixed at compile time, so that each
// butterfly pass is one unrolled sequence instead of a run-time choice among
// all of them.  With both (4096 x 4096 fp16 activations, b = 4096): 2255
// instructions instead of 3531, 10.0 us instead of 10.6 on MI355X.
template <typename TIn, int L, int R, int QV = QV_ANY, int LB = -1>
__global__ void __launch_bounds__(256) rotq_kernel(RotqKArgs a) {
  constexpr int V = Piece<TIn>::V;
  constexpr int S = L * R;
  constexpr int LOGR = ilog2(R);
  constexpr int LOGV = ilog2(V);
  constexpr int PPL = R / V;  // 16-byte pieces per lane
  constexpr int R4 = R / 4;
  static_assert(R >= 8 && R <= 64 && (R % V) == 0, "segment shape");

  extern __shared__ float lds[];
  if (QV == QV_ANY && static_cast<int>(blockIdx.x) >= a.nrot_blocks) {
    // Decode prologue roles (whole workgroups, so no barrier is split).
    const int e = static_cast<int>(blockIdx.x) - a.nrot_blocks;
    if (e < a.lr_rank) {
      if constexpr (sizeof(TIn) == 2)
        lowrank_rows_body<16>(static_cast<const _Float16*>(a.x),
                              static_cast<const _Float16*>(a.lr_at), a.M, a.K, a.lr_rank, a.lr_t,
                              1, e, lds);
    } else {
      read_ahead_role(a.ra, e - a.lr_rank, blockIdx.x, reinterpret_cast<uint32_t*>(lds));
    }
    return;
  }
  const int tid = threadIdx.x;
  const int segs_wg = a.segs_per_row * a.rows_per_wg;
  const int seg_wg = tid / L;
  const int lam = tid % L;
  const bool on = seg_wg < segs_wg;
  const int row_wg = on ? seg_wg / a.segs_per_row : 0;
  const int seg_row = on ? seg_wg % a.segs_per_row : 0;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * a.rows_per_wg + row_wg;
  const bool valid = on && row < a.M;
  float* seg = lds + static_cast<size_t>(on ? seg_wg : 0) * S;
  uint32_t* slots = reinterpret_cast<uint32_t*>(lds + static_cast<size_t>(segs_wg) * S);
  if (tid < a.nslots) slots[tid] = 0u;

  const int k0 = seg_row * S;
  float v[R];

  // 1. Coalesced load and the in-piece butterflies.
  // fp16 input with b >= 2: the first stage is fused into the widening.
  const int log2b = LB >= 0 ? LB : a.log2b;
  const bool mix0 = sizeof(TIn) == 2 && log2b >= 1;
  if (valid) {
    const TIn* src = reinterpret_cast<const TIn*>(a.x) + row * a.K + k0;
    if (mix0) {
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
        const uint4 w = *reinterpret_cast<const uint4*>(src + (j * L + lam) * V);
        const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int u = 0; u < V / 2; ++u) {
          v[j * V + 2 * u] = mix_sum(wd[u]);
          v[j * V + 2 * u + 1] = mix_dif(wd[u]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < PPL; ++j) Piece<TIn>::load(src + (j * L + lam) * V, &v[j * V]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = 0.f;
  }
  if (mix0)
    fwht_bits_upto<1, LOGV>(v, log2b);
  else
    fwht_bits_upto<0, LOGV>(v, log2b);
  if (on) {
#pragma unroll
    for (int j = 0; j < PPL; ++j) {
      const int e = (j * L + lam) * V;
      const int i = e >> LOGR;
      const int c4 = (e & (R - 1)) >> 2;
#pragma unroll
      for (int u = 0; u < V / 4; ++u) {
        float4 f = make_float4(v[j * V + 4 * u], v[j * V + 4 * u + 1], v[j * V + 4 * u + 2],
                               v[j * V + 4 * u + 3]);
        *reinterpret_cast<float4*>(seg + i * R + (((c4 + u) ^ (i & (R4 - 1))) << 2)) = f;
      }
    }
  }
  __syncthreads();

  // 2. Column pass over element bits [log2 R, log2 b).
  const int cb = min(log2b - LOGR, LOGR);
  if (cb > 0) {
    if (on) {
      const int cmask = (1 << cb) - 1;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int g = (r >> cb) * L + lam;
        const int i = ((g >> LOGR) << cb) + (r & cmask);
        v[r] = seg[lds_off<R>(i, g & (R - 1))];
      }
      fwht_bits_upto<0, LOGR>(v, cb);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int g = (r >> cb) * L + lam;
        const int i = ((g >> LOGR) << cb) + (r & cmask);
        seg[lds_off<R>(i, g & (R - 1))] = v[r];
      }
    }
    __syncthreads();
  }
  // Blocks larger than R^2 (segments spanning several waves): further column
  // passes over element bits [lo, lo + LOGR), lo = 2 LOGR, 3 LOGR, ...  In the
  // [L][R] view these are bits [o, o + cb2) of the row index i, o = lo - LOGR;
  // a lane holds the 2^cb2 values of (R >> cb2) (column, other row bits)
  // combinations.
  if constexpr (L >= 128) {
  for (int lo = 2 * LOGR; lo < log2b; lo += LOGR) {
    const int cb2 = min(log2b - lo, LOGR);
    const int o = lo - LOGR;
    if (on) {
      const int cmask = (1 << cb2) - 1;
      const int omask = (1 << o) - 1;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int g = (r >> cb2) * L + lam;
        const int rest = g >> LOGR;
        const int i = ((rest >> o) << (o + cb2)) | ((r & cmask) << o) | (rest & omask);
        v[r] = seg[lds_off<R>(i, g & (R - 1))];
      }
      fwht_bits_upto<0, LOGR>(v, cb2);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int g = (r >> cb2) * L + lam;
        const int rest = g >> LOGR;
        const int i = ((rest >> o) << (o + cb2)) | ((r & cmask) << o) | (rest & omask);
        seg[lds_off<R>(i, g & (R - 1))] = v[r];
      }
    }
    __syncthreads();
  }
  }

  // 3. Row pass: lane lam holds elements [lam * R, lam * R + R) of the segment.
  if (on) {
#pragma unroll
    for (int c4 = 0; c4 < R4; ++c4) {
      const float4 f =
          *reinterpret_cast<const float4*>(seg + lam * R + ((c4 ^ (lam & (R4 - 1))) << 2));
      v[4 * c4] = f.x; v[4 * c4 + 1] = f.y; v[4 * c4 + 2] = f.z; v[4 * c4 + 3] = f.w;
    }
  }
  fwht_bits_upto<LOGV, LOGR>(v, log2b);

  const int kfirst = k0 + lam * R;  // first element of this lane's run

  if (QV == QV_ANY && a.mode == ROTQ_ROTATE) {
    if (valid) {
      float* dst = a.xrot + row * a.K + kfirst;
#pragma unroll
      for (int c4 = 0; c4 < R4; ++c4)
        *reinterpret_cast<float4*>(dst + 4 * c4) =
            make_float4(v[4 * c4] * a.rs, v[4 * c4 + 1] * a.rs, v[4 * c4 + 2] * a.rs,
                        v[4 * c4 + 3] * a.rs);
    }
    return;
  }

  const int gsz = a.gsz;
  // Lanes sharing one scale: shuffles inside a wave, then an LDS atomic max
  // when the group spans several waves or segments.
  const int span_lanes = (gsz < S ? gsz : S) / R;
  const int span_wave = span_lanes < 64 ? span_lanes : 64;
  const bool cross = gsz > S || span_lanes > 64;
  const int slot = row_wg * (a.K / gsz) + kfirst / gsz;
  const bool leader = valid && (kfirst % gsz) == 0;
  const int64_t si = row * (a.K / gsz) + kfirst / gsz;
  // code[r] holds the bits of q + 1.5 * 2^23 for the code q of element r: its
  // low bits are q in two's complement (low nibble = q & 0xF, low byte =
  // q & 0xFF), and the float minus 1.5 * 2^23 is q.
  uint32_t code[R];
  uint32_t rpk[R / 8];  // packed residual codes (weights with a residual)
  const bool res_lane = QV == QV_ANY && kfirst < a.res_pad;
  if (QV == QV_ANY && a.mx) {
    // 4m. block maxima over 32 elements: in-lane for R >= 32, else over the
    // 32 / R lanes that hold one block.
    constexpr int NB = R >= 32 ? R / 32 : 1;   // blocks per lane
    constexpr int BL = R >= 32 ? 32 : R;        // elements of a block in this lane
    float bm[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      float m = 0.f;
#pragma unroll
      for (int u = 0; u < BL; ++u) m = fmaxf(m, fabsf(v[c * BL + u]));
      if constexpr (R < 32) {
#pragma unroll
        for (int o = 1; o < 32 / R; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
      }
      bm[c] = m;
    }
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      // e from the exponent field of RN(max|y| rs) = max|x~|: floor(log2)
      // for normals; subnormals and 0 land on the clamp.
      const float amax = bm[c] * a.rs;
      const int e = max(static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF) - 129, -127);
      const int kb = kfirst + c * BL;           // first element of this lane's part
      if (valid && (kb & 31) == 0) {
        uint8_t* sp;
        if (a.mode == ROTQ_QUANT_TILED)
          sp = a.mx_scale + ((row >> 4) * (a.K / 128) + (kb >> 7)) * 64 + ((kb & 127) >> 5) * 16 +
               (row & 15);
        else
          sp = a.mx_scale + row * (a.K / 32) + (kb >> 5);
        *sp = static_cast<uint8_t>(e + 127);
      }
#pragma unroll
      for (int u = 0; u < BL; u += 2) {
        const float p0 = ldexpf(v[c * BL + u] * a.rs, -e);
        const float p1 = ldexpf(v[c * BL + u + 1] * a.rs, -e);
        const uint32_t pr = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, p0, p1, 1.0f, 0);
        code[c * BL + u] = pr & 0xFu;
        code[c * BL + u + 1] = (pr >> 4) & 0xFu;
      }
    }
  } else if (QV == QV_ANY && a.asym) {
    // 4a. min and max of the group (of y; x~ = RN(y * rs) is monotone in y).
    float ymax = v[0], ymin = v[0];
#pragma unroll
    for (int r = 1; r < R; ++r) {
      ymax = fmaxf(ymax, v[r]);
      ymin = fminf(ymin, v[r]);
    }
    for (int o = 1; o < span_wave; o <<= 1) {
      ymax = fmaxf(ymax, __shfl_xor(ymax, o));
      ymin = fminf(ymin, __shfl_xor(ymin, o));
    }
    if (cross) {
      const int half = a.nslots / 2;
      if (valid && (lam & (span_wave - 1)) == 0) {
        atomicMax(&slots[slot], order_key(ymax));
        atomicMax(&slots[half + slot], order_key(-ymin));
      }
      __syncthreads();
      if (on) {
        ymax = order_val(slots[slot]);
        ymin = -order_val(slots[half + slot]);
      }
    }
    // 5a. Scale and zero point; a group without spread spans [min(c,0), max(c,0)].
    float lo = ymin * a.rs, hi = ymax * a.rs;
    if (hi == lo) {
      lo = fminf(lo, 0.f);
      hi = fmaxf(hi, 0.f);
    }
    const float s = __fdiv_rn(hi - lo, 15.f);
    const bool live = s > 0.f;
    const int zi = live ? static_cast<int>(rintf(__fdiv_rn(-lo, s))) : 0;
    if (leader) {
      reinterpret_cast<float*>(a.scale)[si] = s;
      a.zero[si] = zi;
    }
    // 6a. Codes q = clamp(rint(x~ / s) + z, 0, 15), stored as q - 8.  Zero
    // scale: q = 0.  Quotients here can exceed the magic-number range, so
    // rint is the rounding instruction.
    if (!live) {
#pragma unroll
      for (int r = 0; r < R; ++r) code[r] = 8u;
    } else if (s >= 0x1p-100f && s <= 0x1p100f) {
      const float rc = __frcp_rn(s);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float xt = v[r] * a.rs;
        float q = xt * rc;
        q = __builtin_fmaf(__builtin_fmaf(-q, s, xt), rc, q);
        q = __builtin_fmaf(__builtin_fmaf(-q, s, xt), rc, q);
        const int qi = static_cast<int>(rintf(q)) + zi;
        code[r] = static_cast<uint32_t>(min(max(qi, 0), 15)) ^ 8u;
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float xt = v[r] * a.rs;
        const int qi = static_cast<int>(rintf(__fdiv_rn(xt, s))) + zi;
        code[r] = static_cast<uint32_t>(min(max(qi, 0), 15)) ^ 8u;
      }
    }
  } else {
    // 4. absmax of the scale group (max |y|; the rotated value is y * rs).
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) m = fmaxf(m, fabsf(v[r]));
    for (int o = 1; o < span_wave; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (cross) {
      if (valid && (lam & (span_wave - 1)) == 0) atomicMax(&slots[slot], __float_as_uint(m));
      __syncthreads();
      if (on) m = __uint_as_float(slots[slot]);
    }

    // 5. Scale: s = max|x~| / 7 with max|x~| = RN(max|y| * rs).
    const float amax = m * a.rs;
    const float s = __fdiv_rn(amax, a.fqmax);
    float s_eff = s;
    __half s_h = __float2half_rn(s);
    if (a.scale_f16) s_eff = __half2float(s_h);
    if (leader) {
      if (a.scale_f16)
        reinterpret_cast<__half*>(a.scale)[si] = s_h;
      else
        reinterpret_cast<float*>(a.scale)[si] = s;
    }

    // 6. Codes.  A zero scale (an all-zero group) takes the reciprocal 0, so every
    // quotient and code is 0.  The rint is the magic-number addition: the low
    // mantissa bits of q + 1.5 * 2^23 are rint(q) in two's complement.
    // The specialized variants (float32 scales) on fp16 input never need the
    // IEEE division: every value of the transform is a multiple of 2^-24, so
    // a non-zero |x~| is at least 2^-24 / 64 and a non-zero scale above
    // 2^-33, and |x~| <= 64 * 65504 keeps the scale below 2^20.
    constexpr bool kInRange = QV != QV_ANY && std::is_same<TIn, _Float16>::value;
    if (kInRange || s_eff == 0.f || (s_eff >= 0x1p-100f && s_eff <= 0x1p100f)) {
      // When rs is a power of two (b = 4^k) the product y * rs is exact, so the
      // quotient x~ / s is the same real number as y / (s / rs), with s / rs
      // exact too, and both round alike.  An x~ that would underflow gives a
      // quotient below 2^-26 in magnitude either way, that is code 0.
      // The clamp to [-qmax, qmax] is needed only for a float16 scale below
      // 2^-14: otherwise |x~| <= RN(max|y| rs) and s_eff is that maximum over
      // qmax rounded to float32 or to a normal float16, so |q| <= qmax (1 + 2^-11),
      // below qmax + 1/2, for every finite input.  (The clamped form keeps
      // the multiply by rs.)
      const bool clamp = a.scale_f16 && s_eff < 0x1p-14f;
      const bool fold = !clamp && (__float_as_uint(a.rs) & 0x807FFFFFu) == 0u;
      const float sd = fold ? s_eff * __fdiv_rn(1.f, a.rs) : s_eff;
      const float rc = s_eff == 0.f ? 0.f : __frcp_rn(sd);
      auto quantize = [&](auto folded, auto clamped) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float xt = decltype(folded)::value ? v[r] : v[r] * a.rs;
          float q = xt * rc;
          q = __builtin_fmaf(__builtin_fmaf(-q, sd, xt), rc, q);
          q = __builtin_fmaf(__builtin_fmaf(-q, sd, xt), rc, q);
          const float u = q + kMagic;
          code[r] = __float_as_uint(decltype(clamped)::value
                                        ? __builtin_amdgcn_fmed3f(u, kMagic - a.fqmax, kMagic + a.fqmax)
                                        : u);
        }
      };
      if constexpr (QV == QV_FOLD) {
        quantize(std::true_type{}, std::false_type{});
      } else if constexpr (QV == QV_PLAIN) {
        quantize(std::false_type{}, std::false_type{});
      } else {
        if (clamp)
          quantize(std::false_type{}, std::true_type{});
        else if (fold)
          quantize(std::true_type{}, std::false_type{});
        else
          quantize(std::false_type{}, std::false_type{});
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float xt = v[r] * a.rs;
        float qf = rintf(__fdiv_rn(xt, s_eff));
        qf = fminf(fmaxf(qf, -a.fqmax), a.fqmax);
        code[r] = __float_as_uint(qf + kMagic);
      }
    }
    // 7. Residual codes of the first res_r channels, packed like the codes.
    if (res_lane) {
      const float t = s_eff * 0.125f;  // the residual step s / 8
#pragma unroll
      for (int d = 0; d < R / 8; ++d) {
        uint32_t acc = 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = 8 * d + u;
          int qr = 0;
          if (kfirst + r < a.res_r && t > 0.f) {
            const int q = static_cast<int>(code[r] << 28) >> 28;
            const float xt = v[r] * a.rs;
            const float e = xt - s_eff * static_cast<float>(q);
            qr = static_cast<int>(rintf(__fdiv_rn(e, t)));
            qr = min(max(qr, -8), 7);
          }
          acc = __builtin_amdgcn_alignbit(static_cast<uint32_t>(qr), acc, 4);
        }
        rpk[d] = acc;
      }
    }
  }
  // Packed nibbles (packed modes): element 8d+t in nibble t of dword d.
  const bool packed_mode = a.mode == ROTQ_QUANT || a.mode == ROTQ_QUANT_TILED;
  uint32_t pk[R / 8];
  if (packed_mode) {
#pragma unroll
    for (int d = 0; d < R / 8; ++d) {
      uint32_t acc = 0u;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_alignbit(code[8 * d + t], acc, 4);
      pk[d] = acc;
    }
  }
  // 8. Offset-binary codes: the sum of the row's codes at odd channels (the
  // high nibbles of the packed bytes, kfirst being even), reduced like the
  // absmax.  Each dword's high nibbles are 4 int8 values 16 q.
  if (a.ob_sum) {
    int os16 = 0;
#pragma unroll
    for (int d = 0; d < R / 8; ++d)
      os16 = __builtin_amdgcn_sdot4(static_cast<int>(pk[d] & 0xF0F0F0F0u), 0x01010101, os16, false);
    int os = os16 >> 4;
    for (int o = 1; o < span_wave; o <<= 1) os += __shfl_xor(os, o);
    if (cross) {
      uint32_t* ssum = slots + a.nslots / 2;
      if (valid && (lam & (span_wave - 1)) == 0) atomicAdd(&ssum[slot], static_cast<uint32_t>(os));
      __syncthreads();
      if (on) os = static_cast<int>(ssum[slot]);
    }
    if (leader) a.ob_sum[row] = os;
  }
  if (a.mode == ROTQ_QUANT_F6) {
    // FP6 E2M3 tiles: chunk c of 32 consecutive codes (k = kfirst + 32 c) is
    // one lane of the matrix instruction, lane 16 ((k % 128) / 32) + rin of
    // tile (rblk, k / 128).  The packing instruction converts the exact
    // integer values (scale 1) and interleaves its two 16-value halves:
    // field 2u holds code u, field 2u + 1 code 16 + u.  With R = 16 a chunk
    // spans two lanes, the even one holding its first half.
    if constexpr (R >= 16) {
      constexpr int NCH = R >= 32 ? R / 32 : 1;
      const int64_t rblk6 = row >> 4, rin6 = row & 15;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        f32x16 lo, hi;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if constexpr (R >= 32) {
            lo[u] = __uint_as_float(code[32 * c + u]) - kMagic;
            hi[u] = __uint_as_float(code[32 * c + 16 + u]) - kMagic;
          } else {
            const float own = __uint_as_float(code[u]) - kMagic;
            const float other = __shfl_xor(own, 1);
            lo[u] = (lam & 1) ? other : own;
            hi[u] = (lam & 1) ? own : other;
          }
        }
        const auto p = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(lo, hi, 1.0f);
        if (valid && (R >= 32 || (lam & 1) == 0)) {
          const int64_t k = kfirst + 32 * c;
          uint8_t* tile = a.q + (rblk6 * a.tile_stride + (k >> 7)) * 1536;
          const int l6 = static_cast<int>(((k & 127) >> 5) * 16 + rin6);
          *reinterpret_cast<uint4*>(tile + 16 * l6) = make_uint4(p[0], p[1], p[2], p[3]);
          *reinterpret_cast<uint2*>(tile + 1024 + 8 * l6) = make_uint2(p[4], p[5]);
        }
      }
    }
    return;
  }
  if (!valid) return;
  const bool tiled = a.mode == ROTQ_QUANT_TILED || a.mode == ROTQ_QUANT_I8_TILED;
  const int64_t nkit = a.K / 128;               // 128-code K iterations per row
  const int64_t tstride = a.tile_stride;        // tiles per row block of the output
  const int64_t rblk = row >> 4, rin = row & 15;  // 16-row block, row inside it
  if (packed_mode) {
    const uint32_t obx = a.ob_sum ? 0x08080808u : 0u;  // offset-binary low nibbles
#pragma unroll
    for (int d = 0; d < R / 8; ++d) pk[d] ^= obx;
    if (!tiled) {
      uint8_t* dst = a.q + ((row * a.K + kfirst) >> 1);
      if constexpr (R == 8) {
        *reinterpret_cast<uint32_t*>(dst) = pk[0];
      } else if constexpr (R == 16) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pk[0], pk[1]);
      } else {
#pragma unroll
        for (int d = 0; d < R / 8; d += 4)
          *reinterpret_cast<uint4*>(dst + 4 * d) = make_uint4(pk[d], pk[d + 1], pk[d + 2], pk[d + 3]);
      }
    } else {
      // Packed byte j of the row sits in the 1 KB block (rblk, j / 64) at
      // ((j % 64) / 16 * 16 + rin) * 16 + j % 16.
#pragma unroll
      for (int c = 0; c < (R >= 32 ? R / 32 : 1); ++c) {
        const int64_t j = (kfirst >> 1) + c * 16;
        uint8_t* dst = a.q + (rblk * tstride + (j >> 6)) * 1024 + ((((j & 63) >> 4) * 16 + rin) << 4) +
                       (j & 15);
        if constexpr (R == 8) {
          *reinterpret_cast<uint32_t*>(dst) = pk[0];
        } else if constexpr (R == 16) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(pk[0], pk[1]);
        } else {
          *reinterpret_cast<uint4*>(dst) = make_uint4(pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]);
        }
      }
    }
    if (tiled && res_lane) {
      // Residual: packed byte jj of the residual region sits in tile
      // (rblk, nkit + jj / 64) at the same in-tile place as a code byte.
#pragma unroll
      for (int c = 0; c < (R >= 32 ? R / 32 : 1); ++c) {
        const int64_t jj = (kfirst >> 1) + c * 16;
        uint8_t* dst = a.q + (rblk * tstride + nkit + (jj >> 6)) * 1024 +
                       ((((jj & 63) >> 4) * 16 + rin) << 4) + (jj & 15);
        if constexpr (R == 8) {
          *reinterpret_cast<uint32_t*>(dst) = rpk[0];
        } else if constexpr (R == 16) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(rpk[0], rpk[1]);
        } else {
          *reinterpret_cast<uint4*>(dst) = make_uint4(rpk[4 * c], rpk[4 * c + 1], rpk[4 * c + 2], rpk[4 * c + 3]);
        }
      }
    }
  } else {
    // One int8 code per byte, each group of 8 elements stored in the order
    // 0,2,4,6,1,3,5,7: the K order in which the GEMM widens packed weights.
    uint32_t pb[R / 4];
#pragma unroll
    for (int d = 0; d < R / 8; ++d) {
      uint32_t e = 0u, o = 0u;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        e = __builtin_amdgcn_alignbit(code[8 * d + 2 * t], e, 8);
        o = __builtin_amdgcn_alignbit(code[8 * d + 2 * t + 1], o, 8);
      }
      pb[2 * d] = e;
      pb[2 * d + 1] = o;
    }
    if (!tiled) {
      uint8_t* dst = a.q + row * a.K + kfirst;
      if constexpr (R == 8) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pb[0], pb[1]);
      } else {
#pragma unroll
        for (int d = 0; d < R / 4; d += 4)
          *reinterpret_cast<uint4*>(dst + 4 * d) = make_uint4(pb[d], pb[d + 1], pb[d + 2], pb[d + 3]);
      }
    } else {
      // Code k of the row sits in the 2 KB block (rblk, k / 128) at
      // (((k % 32) / 16 * 4 + (k % 128) / 32) * 16 + rin) * 16 + k % 16.
#pragma unroll
      for (int c = 0; c < (R >= 16 ? R / 16 : 1); ++c) {
        const int64_t k = kfirst + c * 16;
        uint8_t* dst = a.q + (rblk * tstride + (k >> 7)) * 2048 +
                       ((((((k & 31) >> 4) << 2) + ((k & 127) >> 5)) * 16 + rin) << 4) + (k & 15);
        if constexpr (R == 8) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(pb[0], pb[1]);
        } else {
          *reinterpret_cast<uint4*>(dst) = make_uint4(pb[4 * c], pb[4 * c + 1], pb[4 * c + 2], pb[4 * c + 3]);
        }
      }
    }
  }
}

struct Shape { int L, R; };
// Preference order: larger segments first, then more registers per lane.
constexpr Shape kMenu[] = {{64, 64}, {32, 64}, {64, 32}, {16, 64}, {32, 32}, {64, 16}, {8, 64},
                           {16, 32}, {32, 16}, {8, 32},  {16, 16}, {8, 16},  {8, 8}};
// Few rows: segments spread over up to four waves so that a row's transform
// is shared by more lanes (blocks above R^2 take extra column passes).
constexpr Shape kWideMenu[] = {{256, 16}, {128, 16}, {128, 32}, {256, 8}};
constexpr int64_t kWideRows = 64;  // at most this many rows use the wide menu

template <typename TIn>
hipError_t launch_typed(const RotqKArgs& ka, const RotqPlan& p, int64_t M, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(ka.nrot_blocks + ka.lr_rank + ka.ra.blocks));
  // The low-rank and read-ahead roles are written for 256 threads (their K
  // and byte strides, and the four-wave reduction); the rotation blocks leave
  // threads past the plan's count idle.
  const dim3 block((ka.lr_rank > 0 || ka.ra.blocks > 0) ? 256 : p.threads);
  // Specialized quantizer for symmetric codes with float32 scales, fp16 input,
  // no extra roles and no MXFP4, asymmetric or residual output, on the
  // segment shapes of more than 64 rows.
  const bool plain = std::is_same<TIn, _Float16>::value && ka.mode != ROTQ_ROTATE && !ka.mx &&
                     !ka.asym && ka.res_pad == 0 && !ka.scale_f16 && ka.lr_rank == 0 &&
                     ka.ra.blocks == 0;
  if (plain) {
    uint32_t rsb;
    __builtin_memcpy(&rsb, &ka.rs, 4);
    const bool fold = (rsb & 0x807FFFFFu) == 0u;
    // the blocks of the prefill workloads (4096 and 128) fixed at compile time
#define W4A4_ROTQ_QV(LL, RR)                                                                  \
  if (p.L == LL && p.R == RR) {                                                             \
    if (fold && ka.log2b == 12)                                                             \
      hipLaunchKernelGGL((rotq_kernel<TIn, LL, RR, QV_FOLD, 12>), grid, block, p.lds_bytes, st, ka); \
    else if (fold)                                                                          \
      hipLaunchKernelGGL((rotq_kernel<TIn, LL, RR, QV_FOLD>), grid, block, p.lds_bytes, st, ka); \
    else if (ka.log2b == 7)                                                                 \
      hipLaunchKernelGGL((rotq_kernel<TIn, LL, RR, QV_PLAIN, 7>), grid, block, p.lds_bytes, st, ka); \
    else                                                                                    \
      hipLaunchKernelGGL((rotq_kernel<TIn, LL, RR, QV_PLAIN>), grid, block, p.lds_bytes, st, ka); \
    return hipGetLastError();                                                               \
  }
    if constexpr (std::is_same<TIn, _Float16>::value) {
      W4A4_ROTQ_QV(64, 64) W4A4_ROTQ_QV(32, 64) W4A4_ROTQ_QV(64, 32) W4A4_ROTQ_QV(16, 64)
      W4A4_ROTQ_QV(32, 32)
    }
#undef W4A4_ROTQ_QV
  }
#define W4A4_ROTQ_CASE(LL, RR)                                                        \
  if (p.L == LL && p.R == RR) {                                                     \
    hipLaunchKernelGGL((rotq_kernel<TIn, LL, RR>), grid, block, p.lds_bytes, st, ka); \
    return hipGetLastError();                                                       \
  }
  W4A4_ROTQ_CASE(64, 64) W4A4_ROTQ_CASE(32, 64) W4A4_ROTQ_CASE(64, 32) W4A4_ROTQ_CASE(16, 64)
  W4A4_ROTQ_CASE(32, 32) W4A4_ROTQ_CASE(64, 16) W4A4_ROTQ_CASE(8, 64) W4A4_ROTQ_CASE(16, 32)
  W4A4_ROTQ_CASE(32, 16) W4A4_ROTQ_CASE(8, 32) W4A4_ROTQ_CASE(16, 16) W4A4_ROTQ_CASE(8, 16)
  W4A4_ROTQ_CASE(8, 8) W4A4_ROTQ_CASE(256, 16) W4A4_ROTQ_CASE(128, 16) W4A4_ROTQ_CASE(128, 32)
  W4A4_ROTQ_CASE(256, 8)
#undef W4A4_ROTQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace

namespace {

bool try_shape(const Shape& sh, bool wide, int64_t K, int log2b, int64_t gsz, int max_lds,
               RotqPlan* plan) {
  const int64_t b = int64_t{1} << log2b;
  const int64_t S = static_cast<int64_t>(sh.L) * sh.R;
  if (K % S != 0 || b > S) return false;
  if (!wide && b > static_cast<int64_t>(sh.R) * sh.R) return false;
  if (gsz != K && (gsz < sh.R || (gsz & (gsz - 1)) != 0 || K % gsz != 0)) return false;
  const int64_t segs_per_row = K / S;
  if (segs_per_row * sh.L > 256) return false;
  const int64_t span_lanes = (gsz < S ? gsz : S) / sh.R;
  const int64_t slots_per_row = (gsz > S || span_lanes > 64) ? K / gsz : 0;
  // Two slot arrays: the maxima, and the negated minima of the asymmetric
  // mode.
  const int64_t row_bytes = K * 4 + slots_per_row * 8;
  int64_t rows = 256 / (segs_per_row * sh.L);
  if (rows < 1) rows = 1;
  while (rows > 1 && rows * row_bytes > max_lds) --rows;
  if (rows * row_bytes > max_lds) return false;
  const int64_t threads = ((rows * segs_per_row * sh.L + 63) / 64) * 64;
  if (threads > 256 || 2 * rows * slots_per_row > threads) return false;
  plan->L = sh.L;
  plan->R = sh.R;
  plan->segs_per_row = static_cast<int>(segs_per_row);
  plan->rows_per_wg = static_cast<int>(rows);
  plan->threads = static_cast<int>(threads);
  plan->lds_bytes = static_cast<int>(rows * row_bytes);
  plan->nslots = static_cast<int>(2 * rows * slots_per_row);
  return true;
}

}  // namespace

bool rotq_plan(int64_t M, int64_t K, int log2b, int64_t gsz, int max_lds, RotqPlan* plan,
               int min_r) {
  if (M <= kWideRows) {
    for (const Shape& sh : kWideMenu)
      if (sh.R >= min_r && try_shape(sh, true, K, log2b, gsz, max_lds, plan)) return true;
  }
  for (const Shape& sh : kMenu)
    if (sh.R >= min_r && try_shape(sh, false, K, log2b, gsz, max_lds, plan)) return true;
  return false;
}

static ReadAhead read_ahead_of(const RotqExtras& ex) {
  ReadAhead r;
  r.pf = ex.pf;
  r.unit = ex.pf_unit;
  r.units = ex.pf_units;
  r.last = ex.pf_last;
  r.blocks = ex.pf_blocks / 8 * 8;
  r.magic = 0x9E3779B9u;
  return r;
}

hipError_t launch_rotq(const void* x, bool x_f16, int64_t M, int64_t K, int log2b, int mode,
                       int64_t gsz, bool scale_f16, float* xrot, uint8_t* q, void* scale,
                       const RotqPlan& plan, hipStream_t st, const RotqExtras* ex) {
  // Tiled 4-bit codes (FP6, or packed plain or offset-binary) of fp16 rows
  // with one float32 scale per row: the transform on the matrix instruction
  // (rotq_mfma.hip), for 128 <= b <= 4096.
  const bool plain_ex = !ex || (ex->qmax == 7 && !ex->asym_zero && ex->res_r == 0 && !ex->mx_scale &&
                                ex->lr_rank == 0 && !ex->pf);
  const bool tiled4 = mode == ROTQ_QUANT_F6 || mode == ROTQ_QUANT_TILED;
  // Decode launches with the low-rank or read-ahead roles (int4 codes of fp16
  // rows into FP6 or packed tiles, one float32 scale per row).
  const bool has_lr = ex && ex->lr_rank > 0 && x_f16 && M <= 16;
  const bool has_pf = ex && ex->pf && ex->pf_units > 0 && ex->pf_blocks >= 8;
  if (x_f16 && tiled4 && gsz == K && !scale_f16 && (has_lr || has_pf) && ex->qmax == 7 &&
      !ex->asym_zero && ex->res_r == 0 && !ex->mx_scale && !ex->ob_sum &&
      rotq_mfma_roles_ok(M, K, log2b))
    return launch_rotq_mfma_roles(static_cast<const _Float16*>(x), M, K, log2b, mode == ROTQ_QUANT_F6,
                                  q, static_cast<float*>(scale),
                                  has_lr ? static_cast<const _Float16*>(ex->lr_at) : nullptr,
                                  has_lr ? ex->lr_rank : 0, has_lr ? ex->lr_t : nullptr,
                                  has_pf ? read_ahead_of(*ex) : ReadAhead{}, st);
  if (x_f16 && tiled4 && gsz == K && !scale_f16 && plain_ex) {
    const _Float16* xh = static_cast<const _Float16*>(x);
    float* sf = static_cast<float*>(scale);
    int32_t* ob = ex ? ex->ob_sum : nullptr;
    if (rotq_mfma_ok(M, K, log2b))
      return launch_rotq_mfma(xh, M, K, log2b, mode == ROTQ_QUANT_F6 ? ROT_OUT_F6 : ROT_OUT_PACKED, 7,
                              q, sf, ob, nullptr, st);
  }
  // MXFP4 codes, or int8 tiles (qmax 7 or 127), same conditions otherwise.
  const bool bare_ex = !ex || (!ex->asym_zero && ex->res_r == 0 && ex->lr_rank == 0 && !ex->pf &&
                               !ex->ob_sum);
  const int qmax = ex ? ex->qmax : 7;
  if (x_f16 && mode == ROTQ_QUANT_TILED && gsz == K && bare_ex && ex && ex->mx_scale && qmax == 7 &&
      rotq_mfma_ok(M, K, log2b))
    return launch_rotq_mfma(static_cast<const _Float16*>(x), M, K, log2b, ROT_OUT_MX, 7, q, nullptr,
                            nullptr, ex->mx_scale, st);
  // Asymmetric codes per block of 128 (b = group = 128) into packed tiles.
  if (x_f16 && mode == ROTQ_QUANT_TILED && log2b == 7 && gsz == 128 && !scale_f16 && ex &&
      ex->asym_zero && qmax == 7 && ex->res_r == 0 && !ex->mx_scale && ex->lr_rank == 0 && !ex->pf &&
      !ex->ob_sum && rotq_mfma_ok(M, K, log2b))
    return launch_rotq_mfma(static_cast<const _Float16*>(x), M, K, log2b, ROT_OUT_ASYM, 7, q,
                            static_cast<float*>(scale), ex->asym_zero, nullptr, st);
  if (x_f16 && mode == ROTQ_QUANT_I8_TILED && gsz == K && !scale_f16 && bare_ex &&
      !(ex && ex->mx_scale) && rotq_mfma_ok(M, K, log2b))
    return launch_rotq_mfma(static_cast<const _Float16*>(x), M, K, log2b, ROT_OUT_I8, qmax, q,
                            static_cast<float*>(scale), nullptr, nullptr, st);
  RotqKArgs ka{};
  ka.x = x;
  ka.M = M;
  ka.K = static_cast<int>(K);
  ka.log2b = log2b;
  ka.rs = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(int64_t{1} << log2b)));
  ka.mode = mode;
  ka.gsz = static_cast<int>(gsz);
  ka.scale_f16 = scale_f16 ? 1 : 0;
  ka.fqmax = (ex && ex->qmax == 127) ? 127.0f : 7.0f;
  ka.asym = (ex && ex->asym_zero) ? 1 : 0;
  ka.zero = ex ? ex->asym_zero : nullptr;
  ka.mx = (ex && ex->mx_scale) ? 1 : 0;
  ka.mx_scale = ex ? ex->mx_scale : nullptr;
  ka.ob_sum = ex ? ex->ob_sum : nullptr;
  ka.res_r = ex ? ex->res_r : 0;
  ka.res_pad = (ka.res_r + 127) / 128 * 128;
  ka.tile_stride = K / 128 + ka.res_pad / 128;
  ka.xrot = xrot;
  ka.q = q;
  ka.scale = scale;
  ka.segs_per_row = plan.segs_per_row;
  ka.rows_per_wg = plan.rows_per_wg;
  ka.nslots = plan.nslots;
  ka.nrot_blocks = static_cast<int>((M + plan.rows_per_wg - 1) / plan.rows_per_wg);
  if (ex) {
    if (ex->lr_rank > 0 && x_f16 && M <= 16) {
      ka.lr_at = ex->lr_at;
      ka.lr_rank = ex->lr_rank;
      ka.lr_t = ex->lr_t;
    }
    if (ex->pf && ex->pf_units > 0 && ex->pf_blocks >= 8) ka.ra = read_ahead_of(*ex);
  }
  if (x_f16) return launch_typed<_Float16>(ka, plan, M, st);
  return launch_typed<float>(ka, plan, M, st);
}

}  // namespace w4a4
