// mfma.hpp -- CDNA4 (gfx950) matrix-core fragment helpers.
//
// v_mfma_f32_16x16x32_bf16, one wave64 (layout checked on the device):
//   A (16 x 32):  lane l supplies A[l % 16][8*(l/16) + q],  q = 0..7
//   B (32 x 16):  lane l supplies B[8*(l/16) + q][l % 16],  q = 0..7
//   D (16 x 16):  lane l holds    D[4*(l/16) + q][l % 16],  q = 0..3
// Fragments are read from LDS tiles stored "K-contiguous" (the 8 values a lane
// needs are adjacent), so each operand is a single 16-byte LDS read.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gls {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// Fragment of a K-contiguous tile: rows [row0, row0+16), K columns
// [k0, k0+32) of an LDS array with row stride `ld` (elements).
__device__ __forceinline__ bf16x8 frag(const __bf16* base, int ld, int row0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8*>(base + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

__device__ __forceinline__ float bf16_val(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

}  // namespace gls
