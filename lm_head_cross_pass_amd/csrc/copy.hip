// Plain streaming copy: the copy kernel of known size used to calibrate
// hardware byte counters and to measure the practical HBM ceiling.
#include "internal.h"

namespace lmx {

namespace {

// Four 16-byte chunks per thread in flight, all loads before the stores.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16) {
  constexpr int U = 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * U;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * U + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

__global__ void copy_tail_kernel(const uint8_t* src, uint8_t* dst, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace

int copy_enqueue(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 > 0) {
    // a large grid (up to 65536 workgroups) moves the most bytes on MI355X
    int64_t blocks = (n16 + 1023) / 1024;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    if (hipGetLastError() != hipSuccess) return LMX_ERR_HIP;
  }
  const int64_t tail = static_cast<int64_t>(bytes % 16);
  if (tail > 0) {
    hipLaunchKernelGGL(copy_tail_kernel, dim3(1), dim3(64), 0, stream,
                       static_cast<const uint8_t*>(src) + n16 * 16,
                       static_cast<uint8_t*>(dst) + n16 * 16, tail);
    if (hipGetLastError() != hipSuccess) return LMX_ERR_HIP;
  }
  return LMX_OK;
}

}  // namespace lmx
