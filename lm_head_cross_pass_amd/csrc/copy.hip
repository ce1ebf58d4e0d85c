// Plain streaming copy: the copy kernel of known size used to calibrate
// hardware byte counters and to measure the practical HBM ceiling.
#include "internal.h"

namespace lmx {

namespace {

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) {
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
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
    int64_t blocks = (n16 + 255) / 256;
    if (blocks > 256 * 16) blocks = 256 * 16;
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
