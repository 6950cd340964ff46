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

// LDS barrier that does not wait for outstanding global loads, so a prefetch
// of the next chunk stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-bit element q (0..7) of a 16-byte vector of bf16.
__device__ __forceinline__ uint32_t half_of(const uint4& u, int q) {
  const uint32_t w = (q >> 1) == 0 ? u.x : (q >> 1) == 1 ? u.y : (q >> 1) == 2 ? u.z : u.w;
  return (q & 1) ? (w >> 16) : (w & 0xffffu);
}

// Chunk gates, lane = token (one wave, 64 tokens).  Works in log2:
//   l_i = sum_{r <= i} log2 alpha_r (inclusive),  lq_i = l_{i-1} (l_{-1} = 0)
// Padding tokens must carry alpha = 1, eta = 0.
struct ChunkGates {
  float l, lq, llast;
};
__device__ __forceinline__ ChunkGates chunk_gates(float alpha, int lane) {
  float l = log2f(alpha);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float v = __shfl_up(l, off, 64);
    if (lane >= off) l += v;
  }
  float lp = __shfl_up(l, 1, 64);
  if (lane == 0) lp = 0.f;
  ChunkGates g;
  g.l = l;
  g.lq = lp;
  g.llast = __shfl(l, 63, 64);
  return g;
}

}  // namespace gls
