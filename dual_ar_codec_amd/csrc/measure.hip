// A plain streaming read of device memory, used only to put the GEMV rates in context: the best
// rate a kernel that does nothing but read a buffer once reaches on this device (the nominal HBM
// peak is not reachable by any kernel).  Each thread keeps four 16-byte loads in flight per step
// of a grid-stride loop; the words are folded into one value that is stored only if it equals a
// constant, so that the loads cannot be dropped.
#include "kernels.h"

namespace s2k {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ p, size_t n16, uint32_t* sink) {
  constexpr int U = 4;
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x; i < n16; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + (size_t)u * 256;
      v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t s) {
  if (bytes % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read, dim3(4 * device_cus()), dim3(256), 0, s, static_cast<const u32x4*>(p), bytes / 16,
                     sink);
  return hipGetLastError();
}

}  // namespace s2k
