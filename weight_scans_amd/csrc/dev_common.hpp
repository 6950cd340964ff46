// dev_common.hpp -- small device helpers: bf16 <-> fp32 and typed element
// access for the io types (double, float, bf16 stored as uint16_t).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gls {

struct bf16 {
  uint16_t v;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ T load_as(const double* p, int64_t i) { return static_cast<T>(p[i]); }
template <typename T>
__device__ __forceinline__ T load_as(const float* p, int64_t i) { return static_cast<T>(p[i]); }
template <typename T>
__device__ __forceinline__ T load_as(const bf16* p, int64_t i) {
  return static_cast<T>(bf16_to_f32(p[i].v));
}

template <typename T>
__device__ __forceinline__ void store_from(double* p, int64_t i, T v) { p[i] = static_cast<double>(v); }
template <typename T>
__device__ __forceinline__ void store_from(float* p, int64_t i, T v) { p[i] = static_cast<float>(v); }
template <typename T>
__device__ __forceinline__ void store_from(bf16* p, int64_t i, T v) {
  p[i].v = f32_to_bf16(static_cast<float>(v));
}

}  // namespace gls
