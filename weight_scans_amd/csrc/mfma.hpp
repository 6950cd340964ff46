// mfma.hpp -- CDNA4 (gfx950) matrix-core fragment helpers.
//
// v_mfma_f32_16x16x32_bf16, one wave64 (layout checked on the device):
//   A (16 x 32):  lane l supplies A[l % 16][8*(l/16) + q],  q = 0..7
//   B (32 x 16):  lane l supplies B[8*(l/16) + q][l % 16],  q = 0..7
//   D (16 x 16):  lane l holds    D[4*(l/16) + q][l % 16],  q = 0..3
// Fragments are read either from tiles stored "K-contiguous" (the 8 values a
// lane needs are adjacent: one 16-byte LDS read, frag) or, for products that
// contract over the rows of a row-major tile, with two transposing 8-byte
// reads (frag_t).
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Fragment whose K dimension runs down the rows of a row-major LDS tile T
// (row stride `ld` elements): lane l receives T[k0 + 8*(l/16) + q][c0 + l%16],
// q = 0..7 -- the A operand of a product contracting over T's rows (m = column
// of T) or, identically, the B operand (n = column of T).  Uses the gfx950
// transposing LDS read: each 16-lane group reads a 4 x 16 sub-tile (every lane
// 8 bytes of one row) and lane n receives column n.
__device__ __forceinline__ bf16x8 frag_t(const __bf16* base, int ld, int k0, int c0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const __bf16* p0 = base + (k0 + 8 * g + (s >> 2)) * ld + c0 + 4 * (s & 3);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * ld));
  const s16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// ---- swizzled LDS tiles ----
// A [rows][W] bf16 tile (W in {32, 64, 128}) is stored with its 16-byte
// column groups XOR-permuted per row (mask = swz(row), a linear function of
// the row's low four bits), so that the fragment reads below and the 8-byte
// result stores spread over the 64 four-byte LDS banks.  The masks were
// chosen by measuring SQ_LDS_BANK_CONFLICT on gfx950 for these exact access
// patterns: frag_s and frag_ts are conflict-free; put4 costs two passes
// (no row-linear mask does better for that pattern).
template <int W>
__device__ __forceinline__ int swz(int r) {
  if constexpr (W == 128)
    return (((r & 1) << 2) ^ (((r >> 1) & 1) << 1)) ^ (((r >> 3) & 1) * 9);
  else if constexpr (W == 64)
    return (r & 1) | (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2);
  else
    return ((r >> 3) & 1) << 1;
}
// Element offset of (row r, column c) in a swizzled [rows][W] tile.
template <int W>
__device__ __forceinline__ int sidx(int r, int c) {
  return r * W + ((((c >> 3) ^ swz<W>(r))) << 3) + (c & 7);
}
// Fragment reads of swizzled tiles.  The per-lane part of every read
// address is computed once (LaneOff); a read is then `base + const + (off ^
// const)`: the K or column block only XORs the 16-byte group bits (the row,
// group and byte fields of the offset are disjoint bit ranges).  Keeping the
// address in this short form also lets the compiler attribute every read to
// its LDS object, which it needs to see that the read does not depend on
// direct loads still in flight into other objects.
template <int W>
struct LaneOff {
  uint32_t b;       // frag_s: row lane%16, group lane/16
  uint32_t t0, t1;  // frag_ts: rows 8(g&1) + s/4 (+16(g>>1)), and 4 rows further
  uint32_t w;       // put4: row lane%16, columns 4*(lane/16)..+3
};
template <int W>
__device__ __forceinline__ LaneOff<W> lane_off(int lane) {
  static_assert(W == 32 || W == 64 || W == 128, "W");
  const int l = lane & 15, g = lane >> 4;
  LaneOff<W> o;
  o.b = static_cast<uint32_t>(l * W * 2 + ((g ^ swz<W>(l)) << 4));
  const int rl = 8 * (g & 1) + (l >> 2), rh = 16 * (g >> 1);
  const int hb = (l >> 1) & 1, e = 8 * (l & 1);
  o.t0 = static_cast<uint32_t>((rh + rl) * W * 2 + ((hb ^ swz<W>(rl)) << 4) + e);
  o.t1 = static_cast<uint32_t>((rh + rl + 4) * W * 2 + ((hb ^ swz<W>(rl + 4)) << 4) + e);
  o.w = static_cast<uint32_t>(l * W * 2 + ((((g >> 1)) ^ swz<W>(l)) << 4) + 8 * (g & 1));
  return o;
}
// frag on a swizzled [rows][W] tile: rows row0.. (multiple of 16), K columns
// k0.. (multiple of 32).
template <int W>
__device__ __forceinline__ bf16x8 frag_s(const __bf16* base, const LaneOff<W>& o, int row0, int k0) {
  const char* p = reinterpret_cast<const char*>(base) + row0 * W * 2 + (o.b ^ ((k0 >> 3) << 4));
  return *reinterpret_cast<const bf16x8*>(p);
}
// frag_t on a swizzled [rows][W] tile: K rows k0.. (multiple of 32), columns
// c0.. (multiple of 16).
template <int W>
__device__ __forceinline__ bf16x8 frag_ts(const __bf16* base, const LaneOff<W>& o, int k0, int c0) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const char* p = reinterpret_cast<const char*>(base) + k0 * W * 2;
  const uint32_t x = static_cast<uint32_t>((c0 >> 3) << 4);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + (o.t0 ^ x)));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + (o.t1 ^ x)));
  const s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// 8-byte store of the MFMA result layout into a swizzled tile: lane l writes
// row row0 + l%16, columns c0 + 4*(l/16) .. +3 (row0 multiple of 16, c0 of 16).
template <int W>
__device__ __forceinline__ void put4(__bf16* base, const LaneOff<W>& o, int row0, int c0,
                                     const uint2& v) {
  char* p = reinterpret_cast<char*>(base) + row0 * W * 2 + (o.w ^ ((c0 >> 3) << 4));
  *reinterpret_cast<uint2*>(p) = v;
}

// The 8 bytes at the put4 position (4 bf16 of row row0 + l%16, columns c0 + 4*(l/16)..).
template <int W>
__device__ __forceinline__ uint2 get4(const __bf16* base, const LaneOff<W>& o, int row0, int c0) {
  const char* p = reinterpret_cast<const char*>(base) + row0 * W * 2 + (o.w ^ ((c0 >> 3) << 4));
  return *reinterpret_cast<const uint2*>(p);
}

// ---- direct global -> LDS loads (no VGPR round trip) ----
// One wave instruction writes 64 consecutive LDS slots of `size` bytes
// starting at the wave-uniform `lds`, lane i into slot i, from byte offset
// `voff` (per lane) of a buffer.  Lanes whose offset is at or past the
// buffer's byte count write zeros.  Completion is tracked by vmcnt only.
// The per-lane offsets are loop invariants held in VGPRs (the buffer base
// moves per chunk), so no register that a load in flight reads is reused.
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kBufferFlags = 0x00020000;  // raw (untyped) buffer, dword3
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kBufferFlags);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds), 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds), 4, voff, 0, 0, 0);
}
// 8-byte buffer store (lanes whose offset is past the buffer's byte count
// store nothing).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, uint32_t voff, const uint2& v) {
  const u32x2_t d = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(d, r, voff, 0, 0);
}

// 16-byte buffer store (same dropping rule).
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t voff, const uint4& v) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t d = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(d, r, voff, 0, 0);
}

__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, voff, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_val(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Hardware base-2 exponential / logarithm (v_exp_f32 / v_log_f32).  Decay
// factors are always <= 1; results below the normal range flush to zero.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

// Causal lower-triangle block b (0..9) of the 4x4 grid of 16x16 blocks of a
// 64x64 score matrix, row-major over the triangle: (0,0),(1,0),(1,1),(2,0)...
// Computed from packed nibbles so that no memory load is involved.
__device__ __forceinline__ int tri_i(int b) {
  return static_cast<int>((0x3333222110ull >> (4 * b)) & 0xfull);
}
__device__ __forceinline__ int tri_j(int b) {
  return static_cast<int>((0x3210210100ull >> (4 * b)) & 0xfull);
}

// LDS barrier that does not wait for outstanding global loads, so a prefetch
// of the next chunk stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- wave64 scans on DPP (register-only cross-lane moves, GFX9 controls) ----
// dpp<CTRL, ROW_MASK>(old, v): v moved by the DPP pattern; lanes whose source
// is outside the pattern, or whose row is masked off, receive `old`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float old, float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                         CTRL, ROW_MASK, 0xf, false));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ float wave_scan_add(float x) {
  x += dpp<kRowShr1>(0.f, x);
  x += dpp<kRowShr2>(0.f, x);
  x += dpp<kRowShr4>(0.f, x);
  x += dpp<kRowShr8>(0.f, x);
  x += dpp<kRowBcast15, 0xa>(0.f, x);
  x += dpp<kRowBcast31, 0xc>(0.f, x);
  return x;
}

// Value of the previous lane (lane 0 receives `first`).
__device__ __forceinline__ float wave_shift_up(float x, float first) {
  return dpp<kWaveShr1>(first, x);
}

// Inclusive scan of affine pairs over the lanes: with (a_i, b_i) per lane the
// result is (prod_{j<=i} a_j, sum_{j<=i} (prod_{j<r<=i} a_r) b_j), i.e. the
// state after lane i of z <- a_i z + b_i started from z = 0 (the composition
// of the affine maps of lanes 0..i; identity (1, 0)).
template <int CTRL, int RM = 0xf>
__device__ __forceinline__ void affine_step(float& a, float& b) {
  const float as = dpp<CTRL, RM>(1.f, a), bs = dpp<CTRL, RM>(0.f, b);
  b = b + a * bs;
  a = a * as;
}
__device__ __forceinline__ void wave_scan_affine(float& a, float& b) {
  affine_step<kRowShr1>(a, b);
  affine_step<kRowShr2>(a, b);
  affine_step<kRowShr4>(a, b);
  affine_step<kRowShr8>(a, b);
  affine_step<kRowBcast15, 0xa>(a, b);
  affine_step<kRowBcast31, 0xc>(a, b);
}


__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// ---- cross-row moves (gfx950 v_permlane16_swap / v_permlane32_swap) ----
// Rows are the four groups of 16 lanes.  With rows a = [a0 a1 a2 a3] and
// b = [b0 b1 b2 b3], the 32-lane swap leaves a = [a0 a1 b0 b1],
// b = [a2 a3 b2 b3]; the 16-lane swap leaves a = [a0 b0 a2 b2],
// b = [a1 b1 a3 b3] (measured).  Written as VALU assembly with two wait
// states on either side, because the builtins' second result is not
// reliable in this compiler.
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// x summed over the four lanes that share lane & 15, in every lane.
__device__ __forceinline__ float sum_rows(float x) {
  float a = x, b = x;
  permlane16_swap(a, b);
  a += b;
  float c = a, d = a;
  permlane32_swap(c, d);
  return c + d;
}

constexpr int kRowMirror = 0x140;

// Lane order reversed (lane i <- lane 63 - i): each row mirrored by DPP,
// then the rows put in reverse order by the two swaps.
__device__ __forceinline__ float wave_reverse(float x, int lane) {
  const float y = dpp<kRowMirror>(0.f, x);
  float a = y, b = y;
  permlane32_swap(a, b);                 // a = [y0 y1 y0 y1], b = [y2 y3 y2 y3]
  const float h = lane < 32 ? b : a;     // [y2 y3 y0 y1]
  float c = h, d = h;
  permlane16_swap(c, d);                 // c = [h0 h0 h2 h2], d = [h1 h1 h3 h3]
  return (lane & 16) ? c : d;            // [h1 h0 h3 h2] = [y3 y2 y1 y0]
}

// Sum over the 64 lanes (every lane).
__device__ __forceinline__ float wave_sum(float x) {
  return readlane_f(wave_scan_add(x), 63);
}

// Chunk gates, lane = token (one wave, 64 tokens).  Works in log2:
//   l_i = sum_{r <= i} log2 alpha_r (inclusive),  lq_i = l_{i-1} (l_{-1} = 0)
// Padding tokens must carry alpha = 1, eta = 0.
struct ChunkGates {
  float l, lq, llast;
};
__device__ __forceinline__ ChunkGates chunk_gates(float alpha, int lane) {
  (void)lane;
  ChunkGates g;
  g.l = wave_scan_add(flog2(alpha));
  g.lq = wave_shift_up(g.l, 0.f);
  g.llast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g.l), 63));
  return g;
}

}  // namespace gls
