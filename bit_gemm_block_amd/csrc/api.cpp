// api.cpp — the C ABI declared in include/w4a4.h: argument validation,
// kernel planning and stream-ordered launches.  No allocation happens here;
// every buffer belongs to the caller.
#include "w4a4.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "w4a4_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxK = 16384;
constexpr int64_t kMaxRank = 256;
constexpr int64_t kMaxHad = 4096;

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(int64_t v) {
  int r = 0;
  while ((int64_t{1} << r) < v) ++r;
  return r;
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int d) { return d == W4A4_F32 || d == W4A4_F16; }

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return W4A4_ERR_HIP;
}

// Per-device cache: 0 unknown, 1 gfx950, 2 other.  Also the LDS limit.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_kind[kMaxDevices];
std::atomic<int> g_dev_lds[kMaxDevices];

// Returns W4A4_OK and the usable LDS bytes per workgroup for the current
// device, or W4A4_ERR_UNSUPPORTED when there is no gfx950 device.
int device_check(int* max_lds) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return W4A4_ERR_UNSUPPORTED;
  }
  int kind = g_dev_kind[dev].load(std::memory_order_acquire);
  if (kind == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return W4A4_ERR_UNSUPPORTED;
    }
    kind = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    int lds = static_cast<int>(prop.sharedMemPerBlock);
    if (lds > 160 * 1024) lds = 160 * 1024;
    g_dev_lds[dev].store(lds, std::memory_order_relaxed);
    g_dev_kind[dev].store(kind, std::memory_order_release);
  }
  if (kind != 1) return W4A4_ERR_UNSUPPORTED;
  if (max_lds) *max_lds = g_dev_lds[dev].load(std::memory_order_relaxed);
  return W4A4_OK;
}

// Shared checks of K and the Hadamard block.  had_block 0/1 means none.
int check_k_had(int64_t K, int64_t had_block, bool need_rotation) {
  if (K <= 0 || had_block < 0) return W4A4_ERR_INVALID_ARG;
  if (K % 64 != 0 || K > kMaxK) return W4A4_ERR_UNSUPPORTED;
  if (need_rotation && had_block < 1) return W4A4_ERR_UNSUPPORTED;
  if (had_block > 1 && (!is_pow2(had_block) || had_block > kMaxHad || K % had_block != 0))
    return W4A4_ERR_UNSUPPORTED;
  return W4A4_OK;
}

int check_group(int64_t K, int64_t g, bool pow2_only) {
  if (g < 0) return W4A4_ERR_INVALID_ARG;
  if (g == 0) return W4A4_OK;
  if (g % 64 != 0 || K % g != 0) return W4A4_ERR_UNSUPPORTED;
  if (pow2_only && !is_pow2(g)) return W4A4_ERR_UNSUPPORTED;
  return W4A4_OK;
}

int plan_rotq(int64_t M, int64_t K, int64_t had_block, int64_t gsz, int max_lds,
              w4a4::RotqPlan* p, bool f6 = false) {
  const int log2b = had_block > 1 ? ilog2(had_block) : 0;
  // FP6 tiles pack 32 consecutive codes per instruction lane: at least 16
  // elements per lane, two lanes per chunk.
  return w4a4::rotq_plan(M, K, log2b, gsz, max_lds, p, f6 ? 16 : 8) ? W4A4_OK
                                                                    : W4A4_ERR_UNSUPPORTED;
}

constexpr size_t align256(size_t v) { return (v + 255) & ~size_t{255}; }

// With tiled weights, the layer keeps its activation codes packed (4 bits,
// the weights' tile layout): half the operand bytes the GEMM moves per step,
// at the price of widening both operands in registers.
constexpr bool kPackedTiledCodes = true;

// Weights at most this large are read ahead by decode-sized calls.
constexpr int64_t kMaxPrefetchBytes = int64_t{64} << 20;

// Decode-sized calls: the rotation launch also reads the tiled weights that
// the skinny GEMM's workgroups will stream (one 16-row block of row_bytes
// per workgroup), so that the GEMM finds them in cache.
void set_prefetch(w4a4::RotqExtras* ex, const uint8_t* wq, int64_t M, int64_t N,
                  int64_t row_bytes) {
  const int64_t units = (N + 15) / 16;
  const int64_t unit_bytes = 16 * row_bytes;
  if (M > 32 || units * unit_bytes > kMaxPrefetchBytes) return;
  ex->pf = wq;
  ex->pf_unit = unit_bytes;
  ex->pf_units = units;
  ex->pf_last = unit_bytes;
  ex->pf_blocks = static_cast<int>(8 * ((units + 15) / 16));
}

// Workspace of the layer: the activation codes (room for int8 codes of rows
// padded to a multiple of 16), the scales and X.A.
struct WsLayout {
  size_t xq, sx, t, total;
};
WsLayout ws_layout(int64_t M, int64_t K, int64_t rank) {
  WsLayout w;
  w.xq = 0;
  w.sx = align256(static_cast<size_t>((M + 15) / 16 * 16) * static_cast<size_t>(K));
  w.t = w.sx + align256(static_cast<size_t>(M) * 4);
  w.total = w.t + align256(static_cast<size_t>(M) * static_cast<size_t>(rank) * 4);
  return w;
}

bool layout_ok(int l) {
  return l == W4A4_CODES_PACKED || l == W4A4_CODES_I8 || l == W4A4_CODES_I8_TILED ||
         l == W4A4_CODES_PACKED_TILED;
}
bool codes_tiled(int l) { return l == W4A4_CODES_I8_TILED || l == W4A4_CODES_PACKED_TILED; }
bool codes_i8(int l) { return l == W4A4_CODES_I8 || l == W4A4_CODES_I8_TILED;
}
bool wlayout_ok(int l) { return l == W4A4_WEIGHTS_ROWMAJOR || l == W4A4_WEIGHTS_TILED; }
// Entry points that also take the offset-binary layouts check with these.
bool layout_ok_ob(int l) { return layout_ok(l) || l == W4A4_CODES_PACKED_TILED_OB; }
bool wlayout_ok_ob(int l) { return wlayout_ok(l) || l == W4A4_WEIGHTS_TILED_OB; }
// ... and these the FP6 tiled layouts as well.
bool layout_ok_f6(int l) { return layout_ok_ob(l) || l == W4A4_CODES_F6_TILED; }
bool wlayout_ok_f6(int l) { return wlayout_ok_ob(l) || l == W4A4_WEIGHTS_TILED_F6; }
// Offset-binary buffers: the row sums follow the ceil(rows/16)*16 tiled rows.
const int32_t* ob_sums(const uint8_t* q, int64_t rows, int64_t K) {
  return reinterpret_cast<const int32_t*>(q + (rows + 15) / 16 * 16 * (K / 2));
}

}  // namespace

extern "C" {

int w4a4_abi_version(void) { return W4A4_ABI_VERSION; }

const char* w4a4_status_string(int status) {
  switch (status) {
    case W4A4_OK: return "ok";
    case W4A4_ERR_INVALID_ARG: return "invalid argument";
    case W4A4_ERR_UNSUPPORTED: return "unsupported shape or device";
    case W4A4_ERR_MISALIGNED: return "pointer not aligned to 16 bytes";
    case W4A4_ERR_WORKSPACE: return "workspace too small";
    case W4A4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int w4a4_last_hip_error(void) { return g_last_hip_error; }

int w4a4_hadamard_rotate(const void* x, int x_dtype, float* x_rot, int64_t M, int64_t K,
                         int64_t had_block, void* stream) {
  if (!dtype_ok(x_dtype) || M < 0) return W4A4_ERR_INVALID_ARG;
  int s = check_k_had(K, had_block, true);
  if (s != W4A4_OK) return s;
  if (M == 0) return W4A4_OK;
  if (!x || !x_rot) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_rot)) return W4A4_ERR_MISALIGNED;
  int max_lds = 0;
  if ((s = device_check(&max_lds)) != W4A4_OK) return s;
  w4a4::RotqPlan plan;
  if ((s = plan_rotq(M, K, had_block, K, max_lds, &plan)) != W4A4_OK) return s;
  hipError_t e = w4a4::launch_rotq(x, x_dtype == W4A4_F16, M, K, ilog2(had_block), w4a4::ROTQ_ROTATE,
                                   K, false, x_rot, nullptr, nullptr, plan,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

namespace {

int quantize_act_impl(const void* x, int x_dtype, int64_t M, int64_t K, int64_t had_block,
                      uint8_t* xq, int codes_layout, float* x_scale, void* stream, int qmax) {
  if (!dtype_ok(x_dtype) || !layout_ok_f6(codes_layout) || M < 0) return W4A4_ERR_INVALID_ARG;
  if (qmax != 7 && !codes_i8(codes_layout)) return W4A4_ERR_INVALID_ARG;  // 8-bit codes
  int s = check_k_had(K, had_block, false);
  if (s != W4A4_OK) return s;
  const bool ob = codes_layout == W4A4_CODES_PACKED_TILED_OB;
  const bool f6 = codes_layout == W4A4_CODES_F6_TILED;
  if ((codes_tiled(codes_layout) || ob || f6) && K % 128 != 0) return W4A4_ERR_UNSUPPORTED;
  if (M == 0) return W4A4_OK;
  if (!x || !xq || !x_scale) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale)) return W4A4_ERR_MISALIGNED;
  int max_lds = 0;
  if ((s = device_check(&max_lds)) != W4A4_OK) return s;
  w4a4::RotqPlan plan;
  if ((s = plan_rotq(M, K, had_block, K, max_lds, &plan, f6)) != W4A4_OK) return s;
  const int log2b = had_block > 1 ? ilog2(had_block) : 0;
  const int mode = f6                                         ? w4a4::ROTQ_QUANT_F6
                   : codes_layout == W4A4_CODES_I8              ? w4a4::ROTQ_QUANT_I8
                   : codes_layout == W4A4_CODES_I8_TILED     ? w4a4::ROTQ_QUANT_I8_TILED
                   : codes_layout == W4A4_CODES_PACKED_TILED ? w4a4::ROTQ_QUANT_TILED
                   : ob                                      ? w4a4::ROTQ_QUANT_TILED
                                                             : w4a4::ROTQ_QUANT;
  w4a4::RotqExtras ex;
  ex.qmax = qmax;
  if (ob) ex.ob_sum = const_cast<int32_t*>(ob_sums(xq, M, K));
  hipError_t e = w4a4::launch_rotq(x, x_dtype == W4A4_F16, M, K, log2b, mode, K, false, nullptr, xq,
                                   x_scale, plan, static_cast<hipStream_t>(stream), &ex);
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

}  // namespace

int w4a4_quantize_act_int4(const void* x, int x_dtype, int64_t M, int64_t K, int64_t had_block,
                           uint8_t* xq, int codes_layout, float* x_scale, void* stream) {
  return quantize_act_impl(x, x_dtype, M, K, had_block, xq, codes_layout, x_scale, stream, 7);
}

int w4a4_quantize_act_int8(const void* x, int x_dtype, int64_t M, int64_t K, int64_t had_block,
                           uint8_t* xq, int codes_layout, float* x_scale, void* stream) {
  return quantize_act_impl(x, x_dtype, M, K, had_block, xq, codes_layout, x_scale, stream, 127);
}

int w4a4_quantize_weight_int4(const void* w, int w_dtype, int64_t N, int64_t K, int64_t had_block,
                              int64_t w_group, uint8_t* wq, int w_layout, void* w_scale,
                              int scale_dtype, void* stream) {
  const bool f6 = w_layout == W4A4_WEIGHTS_TILED_F6;
  if (!dtype_ok(w_dtype) || !dtype_ok(scale_dtype) || !(wlayout_ok(w_layout) || f6) || N < 0)
    return W4A4_ERR_INVALID_ARG;
  int s = check_k_had(K, had_block, false);
  if (s != W4A4_OK) return s;
  if ((w_layout == W4A4_WEIGHTS_TILED || f6) && K % 128 != 0) return W4A4_ERR_UNSUPPORTED;
  if ((s = check_group(K, w_group, true)) != W4A4_OK) return s;
  if (N == 0) return W4A4_OK;
  if (!w || !wq || !w_scale) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(wq) || !aligned16(w_scale)) return W4A4_ERR_MISALIGNED;
  int max_lds = 0;
  if ((s = device_check(&max_lds)) != W4A4_OK) return s;
  const int64_t gsz = w_group == 0 ? K : w_group;
  w4a4::RotqPlan plan;
  if ((s = plan_rotq(N, K, had_block, gsz, max_lds, &plan, f6)) != W4A4_OK) return s;
  const int log2b = had_block > 1 ? ilog2(had_block) : 0;
  const int mode = f6 ? w4a4::ROTQ_QUANT_F6
                   : w_layout == W4A4_WEIGHTS_TILED ? w4a4::ROTQ_QUANT_TILED : w4a4::ROTQ_QUANT;
  hipError_t e = w4a4::launch_rotq(w, w_dtype == W4A4_F16, N, K, log2b, mode, gsz,
                                   scale_dtype == W4A4_F16, nullptr, wq, w_scale, plan,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

int w4a4_lowrank_project(const void* x, int x_dtype, const void* At, int64_t M, int64_t K,
                         int64_t rank, float* t, void* stream) {
  if (!dtype_ok(x_dtype) || M < 0 || K <= 0 || rank < 1) return W4A4_ERR_INVALID_ARG;
  if (K % 64 != 0 || K > kMaxK || rank > kMaxRank) return W4A4_ERR_UNSUPPORTED;
  if (M == 0) return W4A4_OK;
  if (!x || !At || !t) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(At) || !aligned16(t)) return W4A4_ERR_MISALIGNED;
  int s = device_check(nullptr);
  if (s != W4A4_OK) return s;
  hipError_t e = w4a4::launch_lowrank_project(x, x_dtype == W4A4_F16, At, M, K,
                                              static_cast<int>(rank), t, false,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

int w4a4_qgemm_w4a4(const uint8_t* xq, int codes_layout, const float* x_scale, const uint8_t* wq,
                    int w_layout, const void* w_scale, int w_scale_dtype, int64_t w_group,
                    int64_t M, int64_t N, int64_t K, float* y, int32_t* acc, void* stream) {
  if (!dtype_ok(w_scale_dtype) || !layout_ok_f6(codes_layout) || !wlayout_ok_f6(w_layout) ||
      M < 0 || N < 0 || K <= 0)
    return W4A4_ERR_INVALID_ARG;
  if (K % 64 != 0 || K > kMaxK) return W4A4_ERR_UNSUPPORTED;
  int s = check_group(K, w_group, false);
  if (s != W4A4_OK) return s;
  // FP6 tiled codes go with FP6 tiled weights only
  const bool f6 = w_layout == W4A4_WEIGHTS_TILED_F6;
  if (f6 != (codes_layout == W4A4_CODES_F6_TILED)) return W4A4_ERR_INVALID_ARG;
  if (f6) {
    if (K % 128 != 0 || w_group % 128 != 0) return W4A4_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return W4A4_OK;
    if (!xq || !wq || (!y && !acc)) return W4A4_ERR_INVALID_ARG;
    if (y && (!x_scale || !w_scale)) return W4A4_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(wq) || (x_scale && !aligned16(x_scale)) ||
        (w_scale && !aligned16(w_scale)) || (y && !aligned16(y)) || (acc && !aligned16(acc)))
      return W4A4_ERR_MISALIGNED;
    if ((s = device_check(nullptr)) != W4A4_OK) return s;
    w4a4::GemmArgs g{};
    g.xq = xq; g.sx = x_scale; g.wq = wq; g.sw = w_scale;
    g.sw_f16 = w_scale_dtype == W4A4_F16;
    g.group = static_cast<int>(w_group);
    g.M = M; g.N = N; g.K = K;
    g.y = y; g.acc = acc;
    g.lr_mode = w4a4::LR_NONE;
    g.tiled = 1;
    g.f6 = 1;
    hipError_t e = w4a4::launch_qgemm(g, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A4_OK : hip_fail(e);
  }
  const bool w_ob = w_layout == W4A4_WEIGHTS_TILED_OB;
  const bool a_ob = codes_layout == W4A4_CODES_PACKED_TILED_OB;
  const bool tiled = w_layout != W4A4_WEIGHTS_ROWMAJOR;
  if (tiled != (codes_tiled(codes_layout) || a_ob)) return W4A4_ERR_INVALID_ARG;
  // offset-binary codes need offset-binary weights; the weights take them,
  // or packed tiled codes in the decode kernel, with per-channel scales
  if (a_ob && !w_ob) return W4A4_ERR_INVALID_ARG;
  if (w_ob && (w_group != 0 || (!a_ob && (codes_layout != W4A4_CODES_PACKED_TILED || M > 32))))
    return W4A4_ERR_UNSUPPORTED;
  if (tiled && (K % 128 != 0 || w_group % 128 != 0)) return W4A4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!xq || !wq || (!y && !acc)) return W4A4_ERR_INVALID_ARG;
  if (y && (!x_scale || !w_scale)) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(wq) || (x_scale && !aligned16(x_scale)) ||
      (w_scale && !aligned16(w_scale)) || (y && !aligned16(y)) || (acc && !aligned16(acc)))
    return W4A4_ERR_MISALIGNED;
  if ((s = device_check(nullptr)) != W4A4_OK) return s;
  w4a4::GemmArgs g{};
  g.xq = xq; g.sx = x_scale; g.wq = wq; g.sw = w_scale;
  g.sw_f16 = w_scale_dtype == W4A4_F16;
  g.group = static_cast<int>(w_group);
  g.M = M; g.N = N; g.K = K;
  g.y = y; g.acc = acc;
  g.t = nullptr; g.B = nullptr; g.lr_mode = w4a4::LR_NONE; g.rank = 0;
  g.a_i8 = codes_i8(codes_layout);
  g.tiled = tiled;
  g.w_ob = w_ob;
  if (a_ob) {
    g.ob_sa = ob_sums(xq, M, K);
    g.ob_sb = ob_sums(wq, N, K);
  }
  hipError_t e = w4a4::launch_qgemm(g, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

int w4a4_weights_tiled_to_ob(const uint8_t* wq, int64_t N, int64_t K, uint8_t* out,
                             void* stream) {
  if (N < 0 || K <= 0) return W4A4_ERR_INVALID_ARG;
  if (K % 128 != 0 || K > kMaxK) return W4A4_ERR_UNSUPPORTED;
  if (N == 0) return W4A4_OK;
  if (!wq || !out) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(wq) || !aligned16(out)) return W4A4_ERR_MISALIGNED;
  int s = device_check(nullptr);
  if (s != W4A4_OK) return s;
  hipError_t e = w4a4::launch_weights_to_ob(wq, (N + 15) / 16 * 16, K, out,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

size_t w4a4_qlinear_workspace_size(int64_t M, int64_t N, int64_t K, int64_t rank) {
  if (M <= 0 || N <= 0 || K <= 0 || rank < 0) return 0;
  return ws_layout(M, K, rank).total;
}

int w4a4_qlinear_workspace_layout(int64_t M, int64_t N, int64_t K, int64_t rank, int w_layout,
                                  int64_t w_group, int act_bits, size_t* codes_offset,
                                  int* codes_layout, size_t* scale_offset) {
  if (M <= 0 || N <= 0 || K <= 0 || rank < 0 || w_group < 0 || !wlayout_ok_f6(w_layout) ||
      (act_bits != 4 && act_bits != 8) || !codes_offset || !codes_layout || !scale_offset)
    return W4A4_ERR_INVALID_ARG;
  if (w_layout == W4A4_WEIGHTS_TILED_F6 && act_bits != 4) return W4A4_ERR_UNSUPPORTED;
  const WsLayout L = ws_layout(M, K, rank);
  const bool tiled = w_layout != W4A4_WEIGHTS_ROWMAJOR;
  const bool skinny = M <= 32 && (w_group == 0 || w_group % 128 == 0);
  int lay;
  if (w_layout == W4A4_WEIGHTS_TILED_F6)
    lay = W4A4_CODES_F6_TILED;
  else if (act_bits == 8)
    lay = tiled ? W4A4_CODES_I8_TILED : W4A4_CODES_I8;
  else if (!tiled)
    lay = W4A4_CODES_I8;
  else if (w_layout == W4A4_WEIGHTS_TILED_OB && !skinny)
    lay = W4A4_CODES_PACKED_TILED_OB;
  else
    lay = W4A4_CODES_PACKED_TILED;
  *codes_offset = L.xq;
  *codes_layout = lay;
  *scale_offset = L.sx;
  return W4A4_OK;
}

}  // extern "C"

namespace w4a4 {

int hip_status(hipError_t e) { return hip_fail(e); }

int qlinear_impl(const void* x, int x_dtype, const uint8_t* wq, int w_layout,
                         const void* w_scale, int w_scale_dtype, int64_t M, int64_t N, int64_t K,
                         int64_t had_block, int64_t w_group, const void* At, const void* Bt,
                         int64_t rank, float* y, void* workspace, size_t ws_bytes, void* stream,
                  int qmax) {
  if (!dtype_ok(x_dtype) || !dtype_ok(w_scale_dtype) || !wlayout_ok_f6(w_layout) || M < 0 ||
      N < 0 || rank < 0)
    return W4A4_ERR_INVALID_ARG;
  int s = check_k_had(K, had_block, false);
  if (s != W4A4_OK) return s;
  if ((s = check_group(K, w_group, false)) != W4A4_OK) return s;
  const bool w_f6 = w_layout == W4A4_WEIGHTS_TILED_F6;
  if (w_f6 && qmax != 7) return W4A4_ERR_UNSUPPORTED;  // FP6 tiles hold 4-bit codes
  const bool w_ob = w_layout == W4A4_WEIGHTS_TILED_OB;
  if (w_ob && (w_group != 0 || qmax != 7)) return W4A4_ERR_UNSUPPORTED;
  const bool tiled = w_layout != W4A4_WEIGHTS_ROWMAJOR;
  if (tiled && (K % 128 != 0 || w_group % 128 != 0)) return W4A4_ERR_UNSUPPORTED;
  if (rank > kMaxRank || (x_dtype == W4A4_F16 && rank % 8 != 0)) return W4A4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!x || !wq || !w_scale || !y || !workspace) return W4A4_ERR_INVALID_ARG;
  if (rank > 0 && (!At || !Bt)) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y) ||
      !aligned16(workspace) || (rank > 0 && (!aligned16(At) || !aligned16(Bt))))
    return W4A4_ERR_MISALIGNED;
  const WsLayout L = ws_layout(M, K, rank);
  if (ws_bytes < L.total) return W4A4_ERR_WORKSPACE;
  int max_lds = 0;
  if ((s = device_check(&max_lds)) != W4A4_OK) return s;
  w4a4::RotqPlan plan;
  if ((s = plan_rotq(M, K, had_block, K, max_lds, &plan, w_f6)) != W4A4_OK) return s;

  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* xq = ws + L.xq;
  float* sx = reinterpret_cast<float*>(ws + L.sx);
  void* t = ws + L.t;
  const bool f16 = x_dtype == W4A4_F16;

  const int log2b = had_block > 1 ? ilog2(had_block) : 0;
  // Decode-sized calls fold the low-rank projection and a read of the
  // weights (which the skinny GEMM then finds in cache) into the launch of
  // the rotation kernel, whose few rows leave most of the chip idle.
  w4a4::RotqExtras ex;
  ex.qmax = qmax;
  // 4-bit codes go packed into the tiled GEMM; 8-bit codes stay int8.
  const bool packed_codes = tiled && kPackedTiledCodes && qmax == 7;
  const bool fuse_lr = rank > 0 && f16 && M <= 16;
  if (fuse_lr) {
    ex.lr_at = At;
    ex.lr_rank = static_cast<int>(rank);
    ex.lr_t = t;
  }
  const bool skinny = !w_f6 && M <= 32 && (w_group == 0 || w_group % 128 == 0);
  // Offset-binary weights: offset-binary codes (and their row sums) for the
  // tiled GEMM; the decode kernel converts the weights and takes plain codes.
  const bool a_ob = w_ob && !skinny;
  if (a_ob) ex.ob_sum = const_cast<int32_t*>(ob_sums(xq, M, K));
  const int64_t units = (N + 15) / 16;
  const int64_t unit_bytes = 16 * (K / 2);
  if (skinny && units * unit_bytes <= kMaxPrefetchBytes) {
    ex.pf = wq;
    ex.pf_unit = unit_bytes;
    ex.pf_units = units;
    ex.pf_last = tiled ? unit_bytes : (N - 16 * (units - 1)) * (K / 2);
    ex.pf_blocks = static_cast<int>(8 * ((units + 15) / 16));
  }
  const int mode = w_f6 ? w4a4::ROTQ_QUANT_F6
                   : tiled ? (packed_codes ? w4a4::ROTQ_QUANT_TILED : w4a4::ROTQ_QUANT_I8_TILED)
                           : w4a4::ROTQ_QUANT_I8;
  hipError_t e = w4a4::launch_rotq(x, f16, M, K, log2b, mode, K, false, nullptr, xq, sx, plan, st,
                                   &ex);
  if (e != hipSuccess) return hip_fail(e);
  if (rank > 0 && !fuse_lr) {
    e = w4a4::launch_lowrank_project(x, f16, At, M, K, static_cast<int>(rank), t, f16, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  w4a4::GemmArgs g{};
  g.xq = xq; g.sx = sx; g.wq = wq; g.sw = w_scale;
  g.sw_f16 = w_scale_dtype == W4A4_F16;
  g.group = static_cast<int>(w_group);
  g.M = M; g.N = N; g.K = K;
  g.y = y; g.acc = nullptr;
  g.t = rank > 0 ? t : nullptr;
  g.B = rank > 0 ? Bt : nullptr;
  g.lr_mode = rank == 0 ? w4a4::LR_NONE : (f16 ? w4a4::LR_F16 : w4a4::LR_F32);
  g.rank = static_cast<int>(rank);
  g.a_i8 = !packed_codes;
  g.tiled = tiled;
  g.w_ob = w_ob;
  g.f6 = w_f6;
  if (a_ob) {
    g.ob_sa = ob_sums(xq, M, K);
    g.ob_sb = ob_sums(wq, N, K);
  }
  e = w4a4::launch_qgemm(g, st);
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

}  // namespace w4a4

extern "C" {

int w4a4_qlinear_forward(const void* x, int x_dtype, const uint8_t* wq, int w_layout,
                         const void* w_scale, int w_scale_dtype, int64_t M, int64_t N, int64_t K,
                         int64_t had_block, int64_t w_group, const void* At, const void* Bt,
                         int64_t rank, float* y, void* workspace, size_t ws_bytes, void* stream) {
  return w4a4::qlinear_impl(x, x_dtype, wq, w_layout, w_scale, w_scale_dtype, M, N, K, had_block,
                            w_group, At, Bt, rank, y, workspace, ws_bytes, stream, 7);
}

int w4a8_qlinear_forward(const void* x, int x_dtype, const uint8_t* wq, int w_layout,
                         const void* w_scale, int w_scale_dtype, int64_t M, int64_t N, int64_t K,
                         int64_t had_block, int64_t w_group, const void* At, const void* Bt,
                         int64_t rank, float* y, void* workspace, size_t ws_bytes, void* stream) {
  return w4a4::qlinear_impl(x, x_dtype, wq, w_layout, w_scale, w_scale_dtype, M, N, K, had_block,
                            w_group, At, Bt, rank, y, workspace, ws_bytes, stream, 127);
}

// ---- MXFP4 -----------------------------------------------------------------

int w4a4_quantize_mxfp4(const void* x, int x_dtype, int64_t M, int64_t K, int64_t had_block,
                        uint8_t* xq, int codes_layout, uint8_t* x_scale, void* stream) {
  if (!dtype_ok(x_dtype) || M < 0) return W4A4_ERR_INVALID_ARG;
  if (codes_layout != W4A4_CODES_PACKED && codes_layout != W4A4_CODES_PACKED_TILED)
    return W4A4_ERR_INVALID_ARG;
  int s = check_k_had(K, had_block, false);
  if (s != W4A4_OK) return s;
  if (codes_layout == W4A4_CODES_PACKED_TILED && K % 128 != 0) return W4A4_ERR_UNSUPPORTED;
  if (M == 0) return W4A4_OK;
  if (!x || !xq || !x_scale) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale)) return W4A4_ERR_MISALIGNED;
  int max_lds = 0;
  if ((s = device_check(&max_lds)) != W4A4_OK) return s;
  w4a4::RotqPlan plan;
  if ((s = plan_rotq(M, K, had_block, K, max_lds, &plan)) != W4A4_OK) return s;
  w4a4::RotqExtras ex;
  ex.mx_scale = x_scale;
  const int log2b = had_block > 1 ? ilog2(had_block) : 0;
  hipError_t e = w4a4::launch_rotq(
      x, x_dtype == W4A4_F16, M, K, log2b,
      codes_layout == W4A4_CODES_PACKED_TILED ? w4a4::ROTQ_QUANT_TILED : w4a4::ROTQ_QUANT, K, false,
      nullptr, xq, nullptr, plan, static_cast<hipStream_t>(stream), &ex);
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

int w4a4_qgemm_mxfp4(const uint8_t* xq, const uint8_t* x_scale, const uint8_t* wq,
                     const uint8_t* w_scale, int64_t M, int64_t N, int64_t K, float* y,
                     void* stream) {
  if (M < 0 || N < 0 || K <= 0) return W4A4_ERR_INVALID_ARG;
  if (K % 128 != 0 || K > kMaxK) return W4A4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!xq || !x_scale || !wq || !w_scale || !y) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(wq) || !aligned16(w_scale) ||
      !aligned16(y))
    return W4A4_ERR_MISALIGNED;
  int s = device_check(nullptr);
  if (s != W4A4_OK) return s;
  w4a4::GemmArgs g{};
  g.xq = xq; g.wq = wq;
  g.M = M; g.N = N; g.K = K;
  g.y = y;
  g.lr_mode = w4a4::LR_NONE;
  g.tiled = 1;
  g.mx_xs = x_scale;
  g.mx_ws = w_scale;
  hipError_t e = w4a4::launch_qgemm(g, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

int w4a4_qlinear_forward_mxfp4(const void* x, int x_dtype, const uint8_t* wq,
                               const uint8_t* w_scale, int64_t M, int64_t N, int64_t K,
                               int64_t had_block, const void* At, const void* Bt, int64_t rank,
                               float* y, void* workspace, size_t ws_bytes, void* stream) {
  if (!dtype_ok(x_dtype) || M < 0 || N < 0 || rank < 0) return W4A4_ERR_INVALID_ARG;
  int s = check_k_had(K, had_block, false);
  if (s != W4A4_OK) return s;
  if (K % 128 != 0) return W4A4_ERR_UNSUPPORTED;
  if (rank > kMaxRank || (x_dtype == W4A4_F16 && rank % 8 != 0)) return W4A4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!x || !wq || !w_scale || !y || !workspace) return W4A4_ERR_INVALID_ARG;
  if (rank > 0 && (!At || !Bt)) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y) ||
      !aligned16(workspace) || (rank > 0 && (!aligned16(At) || !aligned16(Bt))))
    return W4A4_ERR_MISALIGNED;
  const WsLayout L = ws_layout(M, K, rank);
  if (ws_bytes < L.total) return W4A4_ERR_WORKSPACE;
  // Codes take half of the int8 code area, their scale tiles 1/16 of it.
  const size_t rows = static_cast<size_t>((M + 15) / 16 * 16);
  const size_t xs_off = L.xq + align256(rows * static_cast<size_t>(K / 2));
  if (xs_off + rows * static_cast<size_t>(K / 32) > L.sx) return W4A4_ERR_UNSUPPORTED;
  int max_lds = 0;
  if ((s = device_check(&max_lds)) != W4A4_OK) return s;
  w4a4::RotqPlan plan;
  if ((s = plan_rotq(M, K, had_block, K, max_lds, &plan)) != W4A4_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* xq = ws + L.xq;
  uint8_t* xs = ws + xs_off;
  void* t = ws + L.t;
  const bool f16 = x_dtype == W4A4_F16;
  w4a4::RotqExtras ex;
  ex.mx_scale = xs;
  set_prefetch(&ex, wq, M, N, K / 2);
  const bool fuse_lr = rank > 0 && f16 && M <= 16;
  if (fuse_lr) {
    ex.lr_at = At;
    ex.lr_rank = static_cast<int>(rank);
    ex.lr_t = t;
  }
  const int log2b = had_block > 1 ? ilog2(had_block) : 0;
  hipError_t e = w4a4::launch_rotq(x, f16, M, K, log2b, w4a4::ROTQ_QUANT_TILED, K, false, nullptr,
                                   xq, nullptr, plan, st, &ex);
  if (e != hipSuccess) return hip_fail(e);
  if (rank > 0 && !fuse_lr) {
    e = w4a4::launch_lowrank_project(x, f16, At, M, K, static_cast<int>(rank), t, f16, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  w4a4::GemmArgs g{};
  g.xq = xq; g.wq = wq;
  g.M = M; g.N = N; g.K = K;
  g.y = y;
  g.t = rank > 0 ? t : nullptr;
  g.B = rank > 0 ? Bt : nullptr;
  g.lr_mode = rank == 0 ? w4a4::LR_NONE : (f16 ? w4a4::LR_F16 : w4a4::LR_F32);
  g.rank = static_cast<int>(rank);
  g.tiled = 1;
  g.mx_xs = xs;
  g.mx_ws = w_scale;
  e = w4a4::launch_qgemm(g, st);
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

// ---- in-GEMM residual of salient channels ---------------------------------

namespace {

// Residual rank r: 0 <= r <= K; the int32 accumulator holds
// 256 (8 sum_K + sum_r) of 4-bit products exactly while 8 K + r_pad < 2^17.
int check_res(int64_t K, int64_t r) {
  if (r < 0) return W4A4_ERR_INVALID_ARG;
  const int64_t rpad = (r + 127) / 128 * 128;
  if (r > K || 8 * K + rpad >= (int64_t{1} << 17)) return W4A4_ERR_UNSUPPORTED;
  return W4A4_OK;
}

w4a4::GemmArgs res_gemm_args(const uint8_t* xq, const float* x_scale, const uint8_t* wq,
                             const void* w_scale, int w_scale_dtype, int64_t r, int64_t M,
                             int64_t N, int64_t K, float* y, int32_t* acc) {
  w4a4::GemmArgs g{};
  g.xq = xq; g.sx = x_scale; g.wq = wq; g.sw = w_scale;
  g.sw_f16 = w_scale_dtype == W4A4_F16;
  g.group = 0;
  g.M = M; g.N = N; g.K = K;
  g.y = y; g.acc = acc;
  g.t = nullptr; g.B = nullptr; g.lr_mode = w4a4::LR_NONE; g.rank = 0;
  g.a_i8 = 0;
  g.tiled = 1;
  g.res = 1;
  g.res_iters = static_cast<int>((r + 127) / 128);
  return g;
}

}  // namespace

int w4a4_quantize_weight_residual_int4(const void* w, int w_dtype, int64_t N, int64_t K,
                                       int64_t had_block, int64_t res_rank, uint8_t* wq,
                                       void* w_scale, int scale_dtype, void* stream) {
  if (!dtype_ok(w_dtype) || !dtype_ok(scale_dtype) || N < 0) return W4A4_ERR_INVALID_ARG;
  int s = check_k_had(K, had_block, false);
  if (s != W4A4_OK) return s;
  if (K % 128 != 0) return W4A4_ERR_UNSUPPORTED;
  if ((s = check_res(K, res_rank)) != W4A4_OK) return s;
  if (N == 0) return W4A4_OK;
  if (!w || !wq || !w_scale) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(wq) || !aligned16(w_scale)) return W4A4_ERR_MISALIGNED;
  int max_lds = 0;
  if ((s = device_check(&max_lds)) != W4A4_OK) return s;
  w4a4::RotqPlan plan;
  if ((s = plan_rotq(N, K, had_block, K, max_lds, &plan)) != W4A4_OK) return s;
  w4a4::RotqExtras ex;
  ex.res_r = static_cast<int>(res_rank);
  const int log2b = had_block > 1 ? ilog2(had_block) : 0;
  hipError_t e = w4a4::launch_rotq(w, w_dtype == W4A4_F16, N, K, log2b, w4a4::ROTQ_QUANT_TILED, K,
                                   scale_dtype == W4A4_F16, nullptr, wq, w_scale, plan,
                                   static_cast<hipStream_t>(stream), &ex);
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

int w4a4_qgemm_residual(const uint8_t* xq, const float* x_scale, const uint8_t* wq,
                        const void* w_scale, int w_scale_dtype, int64_t res_rank, int64_t M,
                        int64_t N, int64_t K, float* y, int32_t* acc, void* stream) {
  if (!dtype_ok(w_scale_dtype) || M < 0 || N < 0 || K <= 0) return W4A4_ERR_INVALID_ARG;
  if (K % 128 != 0 || K > kMaxK) return W4A4_ERR_UNSUPPORTED;
  int s = check_res(K, res_rank);
  if (s != W4A4_OK) return s;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!xq || !wq || (!y && !acc)) return W4A4_ERR_INVALID_ARG;
  if (y && (!x_scale || !w_scale)) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(wq) || (x_scale && !aligned16(x_scale)) ||
      (w_scale && !aligned16(w_scale)) || (y && !aligned16(y)) || (acc && !aligned16(acc)))
    return W4A4_ERR_MISALIGNED;
  if ((s = device_check(nullptr)) != W4A4_OK) return s;
  const w4a4::GemmArgs g =
      res_gemm_args(xq, x_scale, wq, w_scale, w_scale_dtype, res_rank, M, N, K, y, acc);
  hipError_t e = w4a4::launch_qgemm(g, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

int w4a4_qlinear_forward_residual(const void* x, int x_dtype, const uint8_t* wq,
                                  const void* w_scale, int w_scale_dtype, int64_t res_rank,
                                  int64_t M, int64_t N, int64_t K, int64_t had_block, float* y,
                                  void* workspace, size_t ws_bytes, void* stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(w_scale_dtype) || M < 0 || N < 0)
    return W4A4_ERR_INVALID_ARG;
  int s = check_k_had(K, had_block, false);
  if (s != W4A4_OK) return s;
  if (K % 128 != 0) return W4A4_ERR_UNSUPPORTED;
  if ((s = check_res(K, res_rank)) != W4A4_OK) return s;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!x || !wq || !w_scale || !y || !workspace) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y) ||
      !aligned16(workspace))
    return W4A4_ERR_MISALIGNED;
  const WsLayout L = ws_layout(M, K, 0);
  if (ws_bytes < L.total) return W4A4_ERR_WORKSPACE;
  int max_lds = 0;
  if ((s = device_check(&max_lds)) != W4A4_OK) return s;
  w4a4::RotqPlan plan;
  if ((s = plan_rotq(M, K, had_block, K, max_lds, &plan)) != W4A4_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* xq = ws + L.xq;
  float* sx = reinterpret_cast<float*>(ws + L.sx);
  const int log2b = had_block > 1 ? ilog2(had_block) : 0;
  w4a4::RotqExtras ex;
  set_prefetch(&ex, wq, M, N, (K + (res_rank + 127) / 128 * 128) / 2);
  hipError_t e = w4a4::launch_rotq(x, x_dtype == W4A4_F16, M, K, log2b, w4a4::ROTQ_QUANT_TILED, K,
                                   false, nullptr, xq, sx, plan, st, &ex);
  if (e != hipSuccess) return hip_fail(e);
  const w4a4::GemmArgs g =
      res_gemm_args(xq, sx, wq, w_scale, w_scale_dtype, res_rank, M, N, K, y, nullptr);
  e = w4a4::launch_qgemm(g, st);
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

// ---- asymmetric group-wise activations ------------------------------------

namespace {

// Activation groups of the asymmetric path: a power of two in
// [128, kMaxHad] dividing K (the GEMM flushes per 128-code iteration).
int check_agroup(int64_t K, int64_t group) {
  if (group <= 0) return W4A4_ERR_INVALID_ARG;
  if (!is_pow2(group) || group < 128 || group > kMaxHad || K % group != 0)
    return W4A4_ERR_UNSUPPORTED;
  return W4A4_OK;
}

int launch_asym_quant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t had_block,
                      int64_t group, uint8_t* xq, bool tiled, float* x_scale, int32_t* x_zero,
                      int max_lds, hipStream_t st, w4a4::RotqExtras* ex) {
  w4a4::RotqPlan plan;
  int s = plan_rotq(M, K, had_block, group, max_lds, &plan);
  if (s != W4A4_OK) return s;
  ex->asym_zero = x_zero;
  const int log2b = had_block > 1 ? ilog2(had_block) : 0;
  hipError_t e = w4a4::launch_rotq(x, x_dtype == W4A4_F16, M, K, log2b,
                                   tiled ? w4a4::ROTQ_QUANT_TILED : w4a4::ROTQ_QUANT, group, false,
                                   nullptr, xq, x_scale, plan, st, ex);
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

w4a4::GemmArgs asym_gemm_args(const uint8_t* xq, const float* x_scale, const int32_t* x_zero,
                              int64_t group, const uint8_t* wq, const void* w_scale,
                              int w_scale_dtype, const int32_t* w_gsum, int64_t M, int64_t N,
                              int64_t K, float* y) {
  w4a4::GemmArgs g{};
  g.xq = xq; g.sx = x_scale; g.wq = wq; g.sw = w_scale;
  g.sw_f16 = w_scale_dtype == W4A4_F16;
  g.group = 0;
  g.M = M; g.N = N; g.K = K;
  g.y = y; g.acc = nullptr;
  g.t = nullptr; g.B = nullptr; g.lr_mode = w4a4::LR_NONE; g.rank = 0;
  g.a_i8 = 0;
  g.tiled = 1;
  g.zx = x_zero;
  g.wsum = w_gsum;
  g.agroup = static_cast<int>(group);
  return g;
}

}  // namespace

int w4a4_quantize_act_asym_int4(const void* x, int x_dtype, int64_t M, int64_t K,
                                int64_t had_block, int64_t group, uint8_t* xq, int codes_layout,
                                float* x_scale, int32_t* x_zero, void* stream) {
  if (!dtype_ok(x_dtype) || M < 0) return W4A4_ERR_INVALID_ARG;
  if (codes_layout != W4A4_CODES_PACKED && codes_layout != W4A4_CODES_PACKED_TILED)
    return W4A4_ERR_INVALID_ARG;
  int s = check_k_had(K, had_block, false);
  if (s != W4A4_OK) return s;
  if ((s = check_agroup(K, group)) != W4A4_OK) return s;
  if (had_block > 1 && had_block != group) return W4A4_ERR_UNSUPPORTED;
  if (M == 0) return W4A4_OK;
  if (!x || !xq || !x_scale || !x_zero) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale) || !aligned16(x_zero))
    return W4A4_ERR_MISALIGNED;
  int max_lds = 0;
  if ((s = device_check(&max_lds)) != W4A4_OK) return s;
  w4a4::RotqExtras ex;
  return launch_asym_quant(x, x_dtype, M, K, had_block, group, xq,
                           codes_layout == W4A4_CODES_PACKED_TILED, x_scale, x_zero, max_lds,
                           static_cast<hipStream_t>(stream), &ex);
}

int w4a4_weight_group_sums(const uint8_t* wq, int w_layout, int64_t N, int64_t K, int64_t group,
                           int32_t* w_gsum, void* stream) {
  if (!wlayout_ok(w_layout) || N < 0 || K <= 0 || group <= 0) return W4A4_ERR_INVALID_ARG;
  if (K % 64 != 0 || K > kMaxK) return W4A4_ERR_UNSUPPORTED;
  int s = check_group(K, group, false);
  if (s != W4A4_OK) return s;
  if (w_layout == W4A4_WEIGHTS_TILED && K % 128 != 0) return W4A4_ERR_UNSUPPORTED;
  if (N == 0) return W4A4_OK;
  if (!wq || !w_gsum) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(wq) || !aligned16(w_gsum)) return W4A4_ERR_MISALIGNED;
  if ((s = device_check(nullptr)) != W4A4_OK) return s;
  hipError_t e = w4a4::launch_weight_group_sums(wq, w_layout == W4A4_WEIGHTS_TILED, N, K,
                                                static_cast<int>(group), w_gsum,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

int w4a4_qgemm_asym(const uint8_t* xq, const float* x_scale, const int32_t* x_zero, int64_t group,
                    const uint8_t* wq, const void* w_scale, int w_scale_dtype,
                    const int32_t* w_gsum, int64_t M, int64_t N, int64_t K, float* y,
                    void* stream) {
  if (!dtype_ok(w_scale_dtype) || M < 0 || N < 0 || K <= 0) return W4A4_ERR_INVALID_ARG;
  if (K % 128 != 0 || K > kMaxK) return W4A4_ERR_UNSUPPORTED;
  int s = check_agroup(K, group);
  if (s != W4A4_OK) return s;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!xq || !x_scale || !x_zero || !wq || !w_scale || !w_gsum || !y) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(x_zero) || !aligned16(wq) ||
      !aligned16(w_scale) || !aligned16(w_gsum) || !aligned16(y))
    return W4A4_ERR_MISALIGNED;
  if ((s = device_check(nullptr)) != W4A4_OK) return s;
  const w4a4::GemmArgs g = asym_gemm_args(xq, x_scale, x_zero, group, wq, w_scale, w_scale_dtype,
                                          w_gsum, M, N, K, y);
  hipError_t e = w4a4::launch_qgemm(g, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

int w4a4_qlinear_forward_asym(const void* x, int x_dtype, const uint8_t* wq, const void* w_scale,
                              int w_scale_dtype, const int32_t* w_gsum, int64_t M, int64_t N,
                              int64_t K, int64_t had_block, const void* At, const void* Bt,
                              int64_t rank, float* y, void* workspace, size_t ws_bytes,
                              void* stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(w_scale_dtype) || M < 0 || N < 0 || rank < 0)
    return W4A4_ERR_INVALID_ARG;
  int s = check_k_had(K, had_block, false);
  if (s != W4A4_OK) return s;
  if ((s = check_agroup(K, had_block)) != W4A4_OK) return s;
  if (rank > kMaxRank || (x_dtype == W4A4_F16 && rank % 8 != 0)) return W4A4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!x || !wq || !w_scale || !w_gsum || !y || !workspace) return W4A4_ERR_INVALID_ARG;
  if (rank > 0 && (!At || !Bt)) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(w_gsum) ||
      !aligned16(y) || !aligned16(workspace) || (rank > 0 && (!aligned16(At) || !aligned16(Bt))))
    return W4A4_ERR_MISALIGNED;
  const WsLayout L = ws_layout(M, K, rank);
  if (ws_bytes < L.total) return W4A4_ERR_WORKSPACE;
  // The packed codes take half of the int8 code area; the group scales and
  // zero points (M * K / had_block words each) fit in the other half.
  const int64_t G = K / had_block;
  const size_t sx_off =
      L.xq + align256(static_cast<size_t>((M + 15) / 16 * 16) * static_cast<size_t>(K / 2));
  const size_t zx_off = sx_off + align256(static_cast<size_t>(M * G) * 4);
  if (zx_off + static_cast<size_t>(M * G) * 4 > L.sx) return W4A4_ERR_UNSUPPORTED;
  int max_lds = 0;
  if ((s = device_check(&max_lds)) != W4A4_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* xq = ws + L.xq;
  float* sx = reinterpret_cast<float*>(ws + sx_off);
  int32_t* zx = reinterpret_cast<int32_t*>(ws + zx_off);
  void* t = ws + L.t;
  const bool f16 = x_dtype == W4A4_F16;
  w4a4::RotqExtras ex;
  set_prefetch(&ex, wq, M, N, K / 2);
  const bool fuse_lr = rank > 0 && f16 && M <= 16;
  if (fuse_lr) {
    ex.lr_at = At;
    ex.lr_rank = static_cast<int>(rank);
    ex.lr_t = t;
  }
  if ((s = launch_asym_quant(x, x_dtype, M, K, had_block, had_block, xq, true, sx, zx, max_lds, st,
                             &ex)) != W4A4_OK)
    return s;
  hipError_t e;
  if (rank > 0 && !fuse_lr) {
    e = w4a4::launch_lowrank_project(x, f16, At, M, K, static_cast<int>(rank), t, f16, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  w4a4::GemmArgs g = asym_gemm_args(xq, sx, zx, had_block, wq, w_scale, w_scale_dtype, w_gsum, M,
                                    N, K, y);
  g.t = rank > 0 ? t : nullptr;
  g.B = rank > 0 ? Bt : nullptr;
  g.lr_mode = rank == 0 ? w4a4::LR_NONE : (f16 ? w4a4::LR_F16 : w4a4::LR_F32);
  g.rank = static_cast<int>(rank);
  e = w4a4::launch_qgemm(g, st);
  return e == hipSuccess ? W4A4_OK : hip_fail(e);
}

}  // extern "C"
