// decode_roles.h — the weight read-ahead role of a decode rotation launch: a
// few rows leave most of the chip idle, so workgroups after the rotation's
// read the weight slices that the skinny GEMM's workgroups will read next,
// which then find them in the last-level cache.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

// pf_units units of pf_unit bytes (the last one pf_last bytes) by pf_blocks
// workgroups of 256 threads; unit g is what the GEMM workgroup g will read.
struct ReadAhead {
  const uint8_t* pf = nullptr;
  int64_t unit = 0;
  int64_t units = 0;
  int64_t last = 0;
  int blocks = 0;
  uint32_t magic = 0;  // the loaded words are folded and compared with this
};

// Reads the units g = x + 8 (p / 8 + t * (blocks / 8)) of the prefetch area,
// where x is the XCD this block is assumed to run on (workgroups are placed
// on the eight XCDs round-robin by index): the GEMM workgroup g runs on XCD
// g mod 8, so its operand lands in that XCD's L2 and in the shared
// last-level cache.  The loaded words are folded into a value that is
// stored to LDS only if it equals a runtime constant, which keeps the loads.
__device__ __forceinline__ void read_ahead_role(const ReadAhead& a, int p, int64_t launch_index,
                                                uint32_t* sink) {
  const int x = static_cast<int>(launch_index & 7);
  const int per_xcd = a.blocks / 8;
  uint32_t fold = 0u;
  for (int64_t g = x + 8 * static_cast<int64_t>(p / 8); g < a.units; g += 8 * per_xcd) {
    const int64_t bytes = g == a.units - 1 ? a.last : a.unit;
    const uint8_t* base = a.pf + g * a.unit;
    for (int64_t off0 = 0; off0 < bytes; off0 += 4 * 4096) {
      uint4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t off = off0 + u * 4096 + 16 * threadIdx.x;
        w[u] = off + 16 <= bytes ? *reinterpret_cast<const uint4*>(base + off) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) fold ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
    }
  }
  if (fold == a.magic) sink[0] = fold;
}

}  // namespace w4a4
