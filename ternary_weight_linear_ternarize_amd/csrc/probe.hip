// Measurement probes: the floors the BitLinear kernels are compared against
// (declared in include/bitlinear_probe.h).
//
//  * bl_probe_read: a one-shot read of a buffer with the access pattern of the
//    decode GEMV -- every lane issues all of its 16-byte loads before it waits,
//    each wave covering contiguous 1 KiB pieces -- and nothing else, so its
//    duration is what reading those bytes costs on this chip at that size.
//  * bl_probe_empty: a kernel that does nothing (launch and completion cost).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitlinear_probe.h"

namespace bl {

typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));

// Block b reads the U KiB-wide rows b*W*U .. of the buffer (W waves of 64
// lanes x 16 bytes); loads past the end are skipped.  The XOR of what was read
// is stored only if it equals a value the caller passes (never, in practice),
// which keeps every load alive without writing.
template <int U>
__global__ __launch_bounds__(256) void probe_read_kernel(const probe_u32x4* __restrict__ p, int64_t n16,
                                                         uint32_t magic, uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
  probe_u32x4 v[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int64_t j = base + 256 * i;
    v[i] = j < n16 ? __builtin_nontemporal_load(p + j) : probe_u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t x = 0u;
#pragma unroll
  for (int i = 0; i < U; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  if (x == magic) sink[blockIdx.x & 1023] = x;
}

__global__ void probe_empty_kernel() {}

}  // namespace bl

extern "C" {

int bl_probe_read(const void* buf, size_t bytes, int per_lane, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0) return 1;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto* p = reinterpret_cast<const bl::probe_u32x4*>(buf);
  const uint32_t magic = 0x9e3779b9u;
#define BL_PROBE(U)                                                                            \
  hipLaunchKernelGGL(bl::probe_read_kernel<U>, dim3((unsigned)((n16 + 256 * U - 1) / (256 * U))), \
                     dim3(256), 0, s, p, n16, magic, sink)
  switch (per_lane) {
    case 1: BL_PROBE(1); break;
    case 2: BL_PROBE(2); break;
    case 4: BL_PROBE(4); break;
    case 8: BL_PROBE(8); break;
    default: return 1;
  }
#undef BL_PROBE
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int bl_probe_empty(void* stream) {
  hipLaunchKernelGGL(bl::probe_empty_kernel, dim3(1), dim3(64), 0,
                     reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
