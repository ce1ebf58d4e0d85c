// Upstream-gradient scaling for the autograd wrappers of the reduced losses:
// the library computes d(loss)/d(x) for an upstream gradient of 1 in the
// forward call (greyhound functional API page, "cross_entropy": normal autograd
// behaviour over a one-pass loss-and-gradient kernel), and backward multiplies
// that gradient by the upstream scalar. The product is taken in fp32 and
// rounded once to the tensor's format, so an fp16 loss scale of 2^16 or more
// does not overflow on the way and a scale such as 1/3 is not rounded to a
// 16-bit value before it multiplies.
#include "internal.h"

namespace lmx {
namespace {

struct F32Fmt {
  static constexpr int kPerChunk = 4;
  __device__ static float load(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  __device__ static void store(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
  __device__ static u32x4 scale4(const u32x4& c, float s) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(__uint_as_float(c[e]) * s);
    return o;
  }
};

template <typename E>
struct Half16Fmt {
  static constexpr int kPerChunk = 8;
  __device__ static float load(const void* p, int64_t i) {
    return E::widen(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ static void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = E::narrow(v);
  }
  __device__ static u32x4 scale4(const u32x4& c, float s) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = E::pack2(E::widen(static_cast<uint16_t>(c[e] & 0xffffu)) * s,
                      E::widen(static_cast<uint16_t>(c[e] >> 16)) * s);
    }
    return o;
  }
};

// vec: src and dst both 16-byte aligned; then 16-byte chunks, else elements.
// src may equal dst: each element is read and written by the same thread.
template <typename F>
__global__ __launch_bounds__(256) void scale_kernel(const void* src,
                                                    void* dst, int64_t n,
                                                    const float* __restrict__ scale, int vec) {
  const float s = *scale;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t done = 0;
  if (vec) {
    const int64_t nc = n / F::kPerChunk;
    const u32x4* a = static_cast<const u32x4*>(src);
    u32x4* b = static_cast<u32x4*>(dst);
    for (int64_t i = tid; i < nc; i += stride) b[i] = F::scale4(a[i], s);
    done = nc * F::kPerChunk;
  }
  for (int64_t i = done + tid; i < n; i += stride) F::store(dst, i, F::load(src, i) * s);
}

}  // namespace

int scale_enqueue(const void* src, void* dst, int64_t n, int dtype, const float* scale,
                  hipStream_t stream) {
  if (n == 0) return LMX_OK;
  const int vec = (reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(dst) % 16 == 0) ? 1 : 0;
  const int epc = dtype == LMX_F32 ? 4 : 8;
  const int64_t work = vec ? (n + epc - 1) / epc : n;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  if (dtype == LMX_BF16) {
    hipLaunchKernelGGL(scale_kernel<Half16Fmt<Bf16>>, grid, block, 0, stream, src, dst, n, scale, vec);
  } else if (dtype == LMX_F16) {
    hipLaunchKernelGGL(scale_kernel<Half16Fmt<F16>>, grid, block, 0, stream, src, dst, n, scale, vec);
  } else {
    hipLaunchKernelGGL(scale_kernel<F32Fmt>, grid, block, 0, stream, src, dst, n, scale, vec);
  }
  return hipGetLastError() == hipSuccess ? LMX_OK : LMX_ERR_HIP;
}

}  // namespace lmx
