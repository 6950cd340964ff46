// bwd_fused.hpp -- pieces shared by the fused matrix-core reverse scans
// (k_mfma_bwd_f.hip for d = 64, k_mfma_bwd_f128.hip for d = 128).
//
// Per chunk of 64 tokens (chunk-local l = inclusive cumsum of log2 alpha,
// lq_i = l_{i-1}, e(.) = 2^(.), XX_ui = x_u . x_i; the exact adjoint of the
// forward scan, GradLev abstract, omanscience.com):
//   P_ui  = e(lq_u - l_i) XX_ui                         (u > i)
//   Be_ij = e(lq_i - l_j)(-eta_j)(dy_i . g_j)           (j < i),  M = Be + Be^T
// and the two Be dots of the dalpha identity, qq_i = sum_{j<i} Be_ij XX_ij and
// kk_j = sum_{u>j} Be_uj XX_uj: the row and column sums of Be o XX.
#pragma once

#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kFC = 64;     // tokens per chunk
constexpr int kMPad = 64;   // bf16 past each M tile: target of masked-off writes

struct alignas(16) RecF {  // gates of one chunk, lane = token
  float lq[kFC], li[kFC], nb[kFC], eq[kFC], e2[kFC], al[kFC];
  float gam, llast, pad[2];
};

struct alignas(16) QkF {  // per causal block: row sums (qq) and column sums (kk) of Be o XX
  float qq[10][16], kk[10][16];
};

// Gates of a chunk from this lane's token's eta and alpha (one wave, lane =
// token).  Padding tokens carry alpha = 1, eta = 0.
__device__ __forceinline__ void gates_v(float et, float al, RecF& r, int lane) {
  const ChunkGates gt = chunk_gates(al, lane);
  r.lq[lane] = gt.lq;
  r.li[lane] = gt.l;
  r.nb[lane] = -et;
  r.eq[lane] = fexp2(gt.lq);
  r.e2[lane] = fexp2(gt.llast - gt.l);
  r.al[lane] = al;
  if (lane == 0) {
    r.gam = fexp2(gt.llast);
    r.llast = gt.llast;
  }
}
// The same from the chunk's eta / alpha rows (cv valid tokens).
__device__ __forceinline__ void gates_f(const float* eta_row, const float* alpha_row, RecF& r,
                                        int cv, int lane) {
  gates_v(lane < cv ? eta_row[lane] : 0.f, lane < cv ? alpha_row[lane] : 1.f, r, lane);
}

__device__ __forceinline__ f32x4 unpack4f(const uint2& p) {
  f32x4 v;
  v[0] = bf16_val(p.x & 0xffffu);
  v[1] = bf16_val(p.x >> 16);
  v[2] = bf16_val(p.y & 0xffffu);
  v[3] = bf16_val(p.y >> 16);
  return v;
}

__device__ __forceinline__ float dot4f(const f32x4& a, const f32x4& b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

__device__ __forceinline__ uint2 pack4f(const f32x4& v) {
  uint2 pk;
  pk.x = pack2(v[0], v[1]);
  pk.y = pack2(v[2], v[3]);
  return pk;
}

// The 8 bf16 of a fragment, each times its own factor (e0: elements 0-3,
// e1: 4-7), rounded back to bf16.
__device__ __forceinline__ bf16x8 scale8(const bf16x8& f, const f32x4& e0, const f32x4& e1) {
  bf16x8 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r[q] = static_cast<__bf16>(static_cast<float>(f[q]) * e0[q]);
    r[q + 4] = static_cast<__bf16>(static_cast<float>(f[q + 4]) * e1[q]);
  }
  return r;
}

// Outputs dx, dg in bf16 (four per 8-byte store) or, for fp32 outputs, as
// the fp32 accumulators (four per 16-byte store at twice the offset).
template <bool F32>
using out4_t = typename std::conditional<F32, f32x4, uint2>::type;
template <bool F32>
__device__ __forceinline__ out4_t<F32> pack_out(const f32x4& v) {
  if constexpr (F32) return v;
  else return pack4f(v);
}
template <bool F32>
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t r, uint32_t off_bf16,
                                          const out4_t<F32>& v) {
  if constexpr (F32) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, 2 * off_bf16, 0, 0);
  } else {
    store8(r, off_bf16, v);
  }
}

// Sum over the 16 lanes of each row of 16; valid in lane 15 of the row.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kRowShr1>(0.f, x);
  x += dpp<kRowShr2>(0.f, x);
  x += dpp<kRowShr4>(0.f, x);
  x += dpp<kRowShr8>(0.f, x);
  return x;
}

// Causal block b (0..9) of a chunk whose x, g, dy tiles are [64][D] bf16
// (swizzled, lane offsets oD): rows a (block tri_i), columns b' (block tri_j).
// XX_ab' and dy_a . g_b' on the matrix cores, then
//   P^T[b'][a] = e(lq_a - l_b') XX_ab',  M[b'][a] = M[a][b'] = Be_ab'
// (zero unless b' < a; PT, M are [64][64] swizzled, lane offsets o64; M has
// kMPad elements of pad), and the row / column sums of Be o XX into qk.
template <int D>
__device__ __forceinline__ void causal_f(const __bf16* X, const __bf16* G, const __bf16* DY,
                                         const RecF& r, __bf16* PT, __bf16* M, QkF& qk,
                                         const LaneOff<D>& oD, const LaneOff<kFC>& o64, int b,
                                         int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const int rb = tri_i(b), cb = tri_j(b);
  f32x4 xx = zero4(), be = zero4();
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    xx = mfma16x16x32(frag_s<D>(X, oD, rb * 16, kk * 32), frag_s<D>(X, oD, cb * 16, kk * 32), xx);
    be = mfma16x16x32(frag_s<D>(DY, oD, rb * 16, kk * 32), frag_s<D>(G, oD, cb * 16, kk * 32), be);
  }
  const int col = cb * 16 + l16, r0 = rb * 16 + 4 * g4;
  const float lc = r.li[col], nbc = r.nb[col];
  const f32x4 lqr = *reinterpret_cast<const f32x4*>(&r.lq[r0]);
  f32x4 p, v, z;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float e = fexp2(lqr[q] - lc);
    const bool m = col < r0 + q;
    p[q] = m ? xx[q] * e : 0.f;
    v[q] = m ? be[q] * (e * nbc) : 0.f;
    z[q] = v[q] * xx[q];
  }
  put4<kFC>(PT, o64, cb * 16, rb * 16, pack4f(p));
  put4<kFC>(M, o64, cb * 16, rb * 16, pack4f(v));
  // the mirrored half of M, element by element, after the put4 above (on
  // the diagonal block both touch the same bytes, and one wave's LDS writes
  // land in order); lanes with nothing to write there write into the pad
  // past the tile instead, so that the store is unconditional
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = col < r0 + q ? sidx<kFC>(r0 + q, col) : kFC * kFC + lane;
    M[e] = static_cast<__bf16>(v[q]);
  }
  f32x4 zr;
#pragma unroll
  for (int q = 0; q < 4; ++q) zr[q] = row16_sum(z[q]);
  if (l16 == 15) *reinterpret_cast<f32x4*>(&qk.qq[b][4 * g4]) = zr;
  const float t = sum_rows(z[0] + z[1] + z[2] + z[3]);
  if (g4 == 0) qk.kk[b][l16] = t;
}

// qq and kk of token i from the per-block sums: causal block (R, C) is number
// R (R + 1) / 2 + C, so token i takes the row sums of blocks (i / 16, 0..i / 16)
// and the column sums of blocks (i / 16..3, i / 16) (fixed four terms, clamped
// indices, no branch).
__device__ __forceinline__ float qq_of(const QkF& q, int i) {
  const int R = i >> 4, b0 = R * (R + 1) / 2;
  float s = 0.f;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const float v = q.qq[cc <= R ? b0 + cc : b0][i & 15];
    s += cc <= R ? v : 0.f;
  }
  return s;
}
__device__ __forceinline__ float kk_of(const QkF& q, int i) {
  const int Cc = i >> 4;
  float s = 0.f;
#pragma unroll
  for (int R = 0; R < 4; ++R) {
    const float v = q.kk[R >= Cc ? R * (R + 1) / 2 + Cc : 0][i & 15];
    s += R >= Cc ? v : 0.f;
  }
  return s;
}

// dalpha of one chunk (one wave, lane = token i), from its gates and dots:
//   dalpha_i = e(l_last - l_i + lq_i) c0 + e(l_last - l_i) sum_{j<i} e(lq_i - l_j)(-eta_j) pp_j
//              + e(lq_i) sum_{u>i} e(lq_u - l_i) rr_u
//              + (sum_{u>i} qq_u - sum_{j>=i} kk_j) / alpha_i
// with c0 = <Lam_out, D_in> (affine-pair and plain scans over the lanes; the
// suffix sums run on the reversed lane order: rr_r, z_r = qq - kk and the
// gates at lane 63 - i).
__device__ __forceinline__ float dalpha_f(const RecF& rp, const QkF& qr, float pp, float rr_r,
                                          float c0, int lane) {
  const int ir = kFC - 1 - lane;
  const float kk = kk_of(qr, lane);
  const float z_r = qq_of(qr, ir) - kk_of(qr, ir);
  const float al = rp.al[lane], al_r = rp.al[ir];
  const float li = rp.li[lane], lqi = rp.lq[lane], lq_r = rp.lq[ir], llast = rp.llast;
  float a2 = al, b2 = rp.nb[lane] * pp;
  wave_scan_affine(a2, b2);
  const float s2 = wave_shift_up(b2, 0.f);
  float a3 = al_r, b3 = rr_r;
  wave_scan_affine(a3, b3);
  const float s3_r = wave_shift_up(b3, 0.f);
  const float zs_r = wave_shift_up(wave_scan_add(z_r), 0.f);
  const float t34 = wave_reverse(fexp2(lq_r) * s3_r + zs_r * __builtin_amdgcn_rcpf(al_r), lane);
  return fexp2(llast - li + lqi) * c0 + fexp2(llast - li) * s2 + t34 -
         kk * __builtin_amdgcn_rcpf(al);
}

}  // namespace
}  // namespace gls
