// noalloc.hip — w4a4_qlinear_forward_noalloc: the layer with its scratch (the
// activation codes, scales and X.A that w4a4_qlinear_forward keeps in the
// caller's workspace) in a fixed array of device memory inside the library,
// for callers that cannot allocate.
//
// The array is a file-scope device variable: every GPU the library runs on
// holds its own copy, from module load until the process ends.  Its device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and cached; host code passes that address to the kernels,
// never the variable itself (in host code its name stands for a host-side
// handle, not a device address).  Every call on a GPU uses that GPU's copy,
// so calls that overlap in time on one GPU race; nothing in it needs to start
// at zero (the layer's workspace contents on entry do not matter).
#include "w4a4.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "w4a4_internal.h"

namespace {

static_assert(W4A4_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[W4A4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// The device address of this device's copy of `scratch`, or null after a
// failed lookup (its HIP error in *err).
void* scratch_ptr(int dev, hipError_t* err) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  *err = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || !q) return nullptr;
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" int w4a4_qlinear_forward_noalloc(const void* x, int x_dtype, const uint8_t* wq,
                                            int w_layout, const void* w_scale, int w_scale_dtype,
                                            int64_t M, int64_t N, int64_t K, int64_t had_block,
                                            int64_t w_group, const void* At, const void* Bt,
                                            int64_t rank, float* y, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || rank < 0) return W4A4_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return W4A4_OK;
  const size_t need = w4a4_qlinear_workspace_size(M, N, K, rank);
  if (need > W4A4_NOALLOC_SCRATCH_BYTES) return W4A4_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return W4A4_ERR_UNSUPPORTED;
  }
  hipError_t e = hipSuccess;
  void* ws = scratch_ptr(dev, &e);
  if (!ws) {
    (void)hipGetLastError();
    return w4a4::hip_status(e == hipSuccess ? hipErrorInvalidSymbol : e);
  }
  return w4a4::qlinear_impl(x, x_dtype, wq, w_layout, w_scale, w_scale_dtype, M, N, K, had_block,
                            w_group, At, Bt, rank, y, ws, W4A4_NOALLOC_SCRATCH_BYTES, stream, 7);
}
