// Measurement probes for the benchmark's ceilings, not part of the product:
// a plain streaming read of a device buffer (the HBM read rate a kernel
// that only loads can reach on this GPU, at the same bytes per launch as a
// product) and an empty launch (the floor one dispatch costs back to back).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sherry.h"

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Every thread reads 16-byte chunks i, i + S, i + 2S, ... (S = threads in
// the grid), U of them in flight per loop trip, so each wave's loads cover
// whole 1 KB spans and the grid walks the buffer front to back.  The chunks
// are folded with XOR and the result is stored only if it equals a constant
// no buffer here produces, which keeps every load without writing memory.
template <int U>
__global__ __launch_bounds__(1024) void probe_read_kernel(const v4u* __restrict__ src, long long n16,
                                                          unsigned int* sink) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  v4u acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  const unsigned int r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == 0x9E3779B9u) sink[0] = r;
}

__global__ void probe_empty_kernel() {}

template <int U>
hipError_t launch_read(const void* src, size_t bytes, void* sink, int grid, int block, hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel<U>, dim3(grid), dim3(block), 0, s, static_cast<const v4u*>(src),
                     (long long)(bytes / 16), static_cast<unsigned int*>(sink));
  return hipGetLastError();
}

}  // namespace

extern "C" {

sherry_status sherry_probe_read(const void* src, size_t bytes, void* sink, int grid, int block,
                                int unroll, void* stream) {
  if (!src || !sink) return SHERRY_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0 || grid < 1 || grid > (1 << 20) || block < 64 || block > 1024 ||
      block % 64 != 0)
    return SHERRY_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return SHERRY_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (unroll) {
    case 1: e = launch_read<1>(src, bytes, sink, grid, block, s); break;
    case 2: e = launch_read<2>(src, bytes, sink, grid, block, s); break;
    case 4: e = launch_read<4>(src, bytes, sink, grid, block, s); break;
    case 8: e = launch_read<8>(src, bytes, sink, grid, block, s); break;
    default: return SHERRY_ERR_SHAPE;
  }
  return e == hipSuccess ? SHERRY_OK : SHERRY_ERR_HIP;
}

sherry_status sherry_probe_empty(void* stream) {
  hipLaunchKernelGGL(probe_empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? SHERRY_OK : SHERRY_ERR_HIP;
}

}  // extern "C"
