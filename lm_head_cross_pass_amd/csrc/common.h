// Device helpers shared by the cross-entropy and linear cross-entropy kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lmx.h"

namespace lmx {

// 16 bytes as a native vector, the unit of every 128-bit load and store.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_huge_valf();

// bf16 <-> fp32. A bf16 is the upper half of an fp32, so widening is a shift;
// narrowing uses the hardware round-to-nearest-even pack (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.f) & 0xffffu);
}

// IEEE binary16 <-> fp32: hardware converts (v_cvt_f32_f16, and the
// round-to-nearest-even v_cvt_f16_f32 behind the _Float16 cast).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(f16x2_t, w)[0]);
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(f16x2_t, w)[1]);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2_t v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// 16-bit element formats of the linear path, as tags for templates.
// pack2 narrows two values into one word (low half first); scaled_pack2(s,
// lo, hi) packs narrow(s * lo) and narrow(s * hi), each exactly as narrow(s * x)
// rounds (fp16: one rounding of the product, the compiler's mixed-precision
// fma; bf16: the fp32 product, then the pair conversion); lo / hi widen the
// halves of a word.
struct Bf16 {
  __device__ static float widen(uint16_t h) { return bf16_bits_to_f32(h); }
  __device__ static uint16_t narrow(float x) { return f32_to_bf16_bits(x); }
  __device__ static uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
  __device__ static uint32_t scaled_pack2(float s, float lo, float hi) {
    return pack_bf16x2(s * lo, s * hi);
  }
  __device__ static float lo(uint32_t w) { return bf16_lo(w); }
  __device__ static float hi(uint32_t w) { return bf16_hi(w); }
};
struct F16 {
  __device__ static float widen(uint16_t h) { return f16_bits_to_f32(h); }
  __device__ static uint16_t narrow(float x) { return f32_to_f16_bits(x); }
  __device__ static uint32_t pack2(float lo, float hi) { return pack_f16x2(lo, hi); }
  __device__ static uint32_t scaled_pack2(float s, float lo, float hi) {
    return static_cast<uint32_t>(narrow(s * lo)) | (static_cast<uint32_t>(narrow(s * hi)) << 16);
  }
  __device__ static float lo(uint32_t w) { return f16_lo(w); }
  __device__ static float hi(uint32_t w) { return f16_hi(w); }
};

// v_exp_f32 / v_log_f32 work in base 2.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Combine two (max, sum of exp(x - max)) pairs of an online log-sum-exp.
// A side whose max is -inf holds no mass and contributes nothing.
__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const float a = (m == -kInf) ? 0.f : s * exp2_fast((m - M) * kLog2e);
  const float b = (m2 == -kInf) ? 0.f : s2 * exp2_fast((m2 - M) * kLog2e);
  m = M;
  s = a + b;
}

__device__ __forceinline__ void wave_lse_combine(float& m, float& s) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float s2 = __shfl_xor(s, off, 64);
    lse_combine(m, s, m2, s2);
  }
}

}  // namespace lmx
