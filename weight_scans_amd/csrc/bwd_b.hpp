// bwd_b.hpp -- matrix-core reverse scan, column tiles of the adjoint
// (bf16 io, d_in = d_out = D in {64, 128}; gfx950, v_mfma_f32_16x16x32_bf16).
//
// Same reverse walk as k_mfma_bwd_a.hip (exact adjoint of the forward scan,
// GradLev abstract, omanscience.com); this kernel owns a tile K of kT = 32
// columns of Lam and of the saved forward state D_in, so it produces dx and
// dalpha (per-token quantities that reduce over rows).  With
// Be_ij = e(lq_i - l_j)(-eta_j)(dy_i . g_j) for j < i:
//   dx_i = W0^T dy_i + e(lq_i) D_in^T dy_i + (Be X)_i + (Be^T X)_i
//          - eta_i e(l_last - l_i) Lam_out^T g_i
//   dalpha_i = <Lam_i, D_i> = e(l_last - l_i + lq_i) <Lam_out, D_in>
//              + e(l_last - l_i) sum_{j<i} Mf_ij (-eta_j) x_j.(Lam_out^T g_j)
//              + e(lq_i) sum_{u>i} Mf_ui x_u.(D_in^T dy_u)
//              + (sum_{u>i} x_u.(Be X)_u - sum_{j>=i} x_j.(Be^T X)_j) / alpha_i
// (Mf_ij = e(lq_i - l_j)) and the column tile of Lam carried as
//   Lam_in[:, K] = e(l_last) Lam_out[:, K] + sum_u e(lq_u) dy_u x_u[K]^T.
//
// Pipeline: two chunk slots filled by direct buffer loads (the chunk's full
// dy and g tiles make a deeper ring too large for LDS at D = 128), two
// barriers per chunk.  A slot holds the tiles of one chunk and the gate
// inputs (eta, alpha) of the chunk visited after it, so the gates of the next
// chunk are derived one visit early.  Phase 1: e(lq) x, Be, the
// <Lam_out, D_in> partials; one wave stores dalpha of the chunk visited two
// visits earlier.  Phase 2: wave w owns the 16 x 16 block (token block w/2,
// column block w%2) of dx and its per-token dots, and D/64 16 x 16 blocks of
// the Lam update; meanwhile one wave derives the gates of the next chunk and
// two waves run the forward and the reversed scans of dalpha of the previous
// chunk.
#pragma once

#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kC = 64;         // tokens per chunk
constexpr int kT = 32;         // columns per work-group
constexpr int kNW = 8;         // waves per work-group
constexpr int kNT = 64 * kNW;  // threads
constexpr int kDaWave = 7;     // stores dalpha
constexpr int kGateWave = 0;   // derives the gates of the next chunk
constexpr int kFwdWave = 2;    // forward scan of dalpha
constexpr int kRevWave = 3;    // reversed scans of dalpha

template <int D>
struct alignas(16) SlotB {
  __bf16 Dy[kC * D];     // dy of the chunk, swizzled [token][D]
  __bf16 G[kC * D];      // g of the chunk, swizzled [token][D]
  __bf16 Xk[kC * kT];    // x of the column tile, swizzled [token][kT]
  __bf16 Sn[D * kT];     // D_in[:, K], swizzled [row][kT]
  float q[2][kC];        // eta, alpha of the chunk visited next
};

// Gates of one chunk (lane = token) and the two parts of its dalpha.
struct alignas(16) GatesB {
  float lq[kC], li[kC], nb[kC], eq[kC], e2[kC], al[kC];
  float fpart[kC], rpart[kC];
  float gam[4];  // gam[0] = e(l_last), gam[1] = l_last
};

// Per-lane byte offsets of the chunk loads (loop invariant).
template <int D>
struct DmaOffB {
  uint32_t dg[D / 64];  // dy / g rows: instructions w + 8 s
  uint32_t sn;          // D_in column tile
  uint32_t xk;          // x column tile
  uint32_t q;           // gate row
};
template <int D>
__device__ __forceinline__ DmaOffB<D> dma_off_b(int wave, int lane) {
  constexpr int U = D / 8;
  DmaOffB<D> o;
#pragma unroll
  for (int s = 0; s < D / 64; ++s) {
    const int p = (wave + 8 * s) * 64 + lane;
    const int row = p / U, kl = (p % U) ^ swz<D>(row);
    o.dg[s] = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  }
  // D = 128: wave w loads D_in instruction w (of 8) and x quarter w & 3;
  // D = 64: waves 0-3 load D_in quarter w, waves 4-7 x quarter w & 3
  {
    const int p = (D == 128 ? wave : (wave & 3)) * 64 + lane;
    const int row = p >> 2, kl = (p & 3) ^ swz<kT>(row);
    o.sn = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  }
  {
    const int p = (wave & 3) * 64 + lane;
    const int row = p >> 2, kl = (p & 3) ^ swz<kT>(row);
    o.xk = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  }
  o.q = static_cast<uint32_t>(lane * 4);
  return o;
}

// Gate row (eta for even waves, alpha for odd ones; four waves write the
// same bytes) of chunk k into q, one dword per lane.  k < 0: zero fill.
__device__ __forceinline__ void issue_gate_row(float (*q)[kC], uint32_t voff, const float* eta,
                                               const float* alpha, int64_t T, int k, int wave) {
  const bool in = k >= 0;
  const int64_t t0 = in ? static_cast<int64_t>(k) * kC : 0;
  const int cv = in ? static_cast<int>(std::min<int64_t>(kC, T - t0)) : 0;
  const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(((wave & 1) == 0 ? eta : alpha) + t0, cv * 4);
  dma4(rq, voff, q[wave & 1]);
}

// Tiles of chunk k and the gate rows of chunk kq into `sl` (negative: zero fill).
template <int D>
__device__ __forceinline__ void issue_chunk_b(SlotB<D>& sl, const DmaOffB<D>& o,
                                              const uint16_t* dy, const uint16_t* g,
                                              const uint16_t* x, const uint16_t* st,
                                              const float* eta, const float* alpha, int64_t T,
                                              int k, int kq, int k0, int wave) {
  const bool in = k >= 0;
  const int64_t t0 = in ? static_cast<int64_t>(k) * kC : 0;
  const int cv = in ? static_cast<int>(std::min<int64_t>(kC, T - t0)) : 0;
  const __amdgpu_buffer_rsrc_t rdy = buffer_rsrc(dy + t0 * D, cv * D * 2);
  const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g + t0 * D, cv * D * 2);
#pragma unroll
  for (int s = 0; s < D / 64; ++s) {
    dma16(rdy, o.dg[s], sl.Dy + (wave + 8 * s) * 512);
    dma16(rg, o.dg[s], sl.G + (wave + 8 * s) * 512);
  }
  const __amdgpu_buffer_rsrc_t rs =
      buffer_rsrc(st + (in ? static_cast<int64_t>(k) : 0) * D * D + k0, in ? (D * D - k0) * 2 : 0);
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + t0 * D + k0, cv > 0 ? (cv * D - k0) * 2 : 0);
  if constexpr (D == 128) {
    dma16(rs, o.sn, sl.Sn + wave * 512);
    dma16(rx, o.xk, sl.Xk + (wave & 3) * 512);  // waves 4-7 repeat 0-3: same bytes
  } else {
    // the same instruction in every wave: scalar-selected source / destination
    const bool sw = wave < 4;
    const int off = sw ? static_cast<int>(offsetof(SlotB<D>, Sn)) + wave * 1024
                       : static_cast<int>(offsetof(SlotB<D>, Xk)) + (wave & 3) * 1024;
    dma16(sw ? rs : rx, sw ? o.sn : o.xk, reinterpret_cast<char*>(&sl) + off);
  }
  issue_gate_row(sl.q, o.q, eta, alpha, T, kq, wave);
}
template <int D>
constexpr int kLoadOpsB = D == 128 ? 7 : 4;

// Gates of a chunk from its gate rows (one wave, lane = token).  Padding
// tokens carry alpha = 1, eta = 0.
__device__ __forceinline__ void gates_b(const float (*q)[kC], GatesB& gs, int cv, int lane) {
  const float et = lane < cv ? q[0][lane] : 0.f;
  const float al = lane < cv ? q[1][lane] : 1.f;
  const ChunkGates gt = chunk_gates(al, lane);
  gs.lq[lane] = gt.lq;
  gs.li[lane] = gt.l;
  gs.nb[lane] = -et;
  gs.eq[lane] = fexp2(gt.lq);
  gs.e2[lane] = fexp2(gt.llast - gt.l);
  gs.al[lane] = al;
  if (lane == 0) {
    gs.gam[0] = fexp2(gt.llast);
    gs.gam[1] = gt.llast;
  }
}
// Block b of Be, written transposed: BeT[j][i] = Be_ij (j < i).
template <int D>
__device__ __forceinline__ void be_block(const SlotB<D>& sl, const GatesB& gs, __bf16* BeT,
                                         const LaneOff<D>& oD, const LaneOff<kC>& oA, int b,
                                         int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const int ib = tri_i(b), jb = tri_j(b);
  f32x4 d = zero4();
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
    d = mfma16x16x32(frag_s<D>(sl.Dy, oD, ib * 16, kb * 32), frag_s<D>(sl.G, oD, jb * 16, kb * 32),
                     d);
  const int j = jb * 16 + l16, i0 = ib * 16 + 4 * g4;
  const float lj = gs.li[j], nj = gs.nb[j];
  const f32x4 lqi = *reinterpret_cast<const f32x4*>(&gs.lq[i0]);
  f32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float e = d[q] * fexp2(lqi[q] - lj) * nj;
    v[q] = (j < i0 + q) ? e : 0.f;
  }
  uint2 pk;
  pk.x = pack2(v[0], v[1]);
  pk.y = pack2(v[2], v[3]);
  put4<kC>(BeT, oA, jb * 16, ib * 16, pk);
}

__device__ __forceinline__ f32x4 unpack4(const uint2& p) {
  f32x4 v;
  v[0] = bf16_val(p.x & 0xffffu);
  v[1] = bf16_val(p.x >> 16);
  v[2] = bf16_val(p.y & 0xffffu);
  v[3] = bf16_val(p.y >> 16);
  return v;
}

// LDS objects of the column-tile pass.  Each of them must be a separate LDS
// variable in the calling kernel (so the compiler can tell the slot being
// read from the one being filled by direct loads).
template <int D>
struct SmemB {
  SlotB<D>& ring0;
  SlotB<D>& ring1;
  __bf16* BeT;        // [kC * kC]      BeT[j][i] = Be_ij, swizzled
  __bf16* L0;         // [D * kT]       Lam_out[:, K] (bf16) [row][col], even visits
  __bf16* L1;         // [D * kT]       odd visits
  __bf16* XS;         // [kC * kT]      e(lq_u) x_u[K]
  GatesB* gs;         // [3]            gates of the chunk of visit v in gs[v % 3]
  float* dots;        // [2][2][4][kC]  per-token dots by parity, column block, kind
  float* c0;          // [2][kNW]       <Lam_out, D_in> partials by parity, wave
};

// The column-tile pass for sequence-head bh, column tile `tile`, segment
// `seg` (its chunks visited from the last; Lam entering from the right is
// seg_lam, or zero).
template <int D>
__device__ __forceinline__ void role_b_body(const BwdArgs& a, int64_t bh, int tile, int seg,
                                            const SmemB<D>& m) {
  static_assert(D == 64 || D == 128, "D");
  constexpr int NS = D / 64;  // 16x16 Lam blocks per wave
  constexpr int S = 2;        // stores per wave per chunk: dalpha (or a dropped one), dx
  SlotB<D>* const rs[2] = {&m.ring0, &m.ring1};
  __bf16* const BeT_s = m.BeT;
  __bf16* const L_s[2] = {m.L0, m.L1};
  __bf16* const XS_s = m.XS;
  float (*dots_s)[2][4][kC] = reinterpret_cast<float (*)[2][4][kC]>(m.dots);
  float (*c0_s)[kNW] = reinterpret_cast<float (*)[kNW]>(m.c0);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int tb = wave >> 1, cbw = wave & 1;
  const int k0 = tile * kT;
  const int h = static_cast<int>(bh % a.H);
  const int64_t T = a.T, BHT = a.B * a.H * T;
  const int n = a.n_chunks;
  const int c_beg = seg * a.seg_chunks;
  const int c_end = std::min(n, c_beg + a.seg_chunks);
  const int nloc = c_end - c_beg;
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * D;
  const uint16_t* g = static_cast<const uint16_t*>(a.g) + bh * T * D;
  const uint16_t* dy = static_cast<const uint16_t*>(a.dy) + bh * T * D;
  const float* eta = static_cast<const float*>(a.eta) + bh * T;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * D * D;
  const uint16_t* st = static_cast<const uint16_t*>(a.states) + bh * static_cast<int64_t>(n) * D * D;
  uint16_t* dx = static_cast<uint16_t*>(a.dx) + bh * T * D;
  float* pa = static_cast<float*>(a.part_alpha) + tile * BHT + bh * T;

  const LaneOff<D> oD = lane_off<D>(lane);
  const LaneOff<kT> oT = lane_off<kT>(lane);
  const LaneOff<kC> oA = lane_off<kC>(lane);

  // W0[:, K] as MFMA A fragments of W0[:,K]^T dy^T, staged through L_s[1]
  for (int idx = tid; idx < D * kT / 8; idx += kNT) {
    const int r = idx >> 2, cc = 8 * (idx & 3);
    *reinterpret_cast<uint4*>(&L_s[1][sidx<kT>(r, cc)]) =
        *reinterpret_cast<const uint4*>(W0 + static_cast<int64_t>(r) * D + k0 + cc);
  }
  for (int idx = tid; idx < kC * kC / 8; idx += kNT)
    reinterpret_cast<uint4*>(&BeT_s[0])[idx] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  bf16x8 w0f[D / 32];
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) w0f[kb] = frag_ts<kT>(L_s[1], oT, kb * 32, cbw * 16);
  __syncthreads();

  // Lam columns of the tile entering from the right (fp32 accumulators, and
  // the bf16 copy read by the first visit)
  f32x4 lam[NS];
  if (a.seg_lam) {
    const float* sl = a.seg_lam + (bh * a.n_seg + seg) * D * D;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      lam[s] = *reinterpret_cast<const f32x4*>(sl + ((tb + 4 * s) * 16 + l16) * D + k0 +
                                               cbw * 16 + 4 * g4);
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) lam[s] = zero4();
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    uint2 pk;
    pk.x = pack2(lam[s][0], lam[s][1]);
    pk.y = pack2(lam[s][2], lam[s][3]);
    put4<kT>(L_s[0], oT, (tb + 4 * s) * 16, cbw * 16, pk);
  }
  wait_vm<0>();

  // valid tokens of chunk c (none outside this segment)
  const auto cv_of = [&](int c) {
    return (c < c_beg || c >= c_end)
               ? 0
               : static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };
  const auto in_seg = [&](int c) { return c >= c_beg ? c : -1; };
  const DmaOffB<D> od = dma_off_b<D>(wave, lane);
  const uint32_t odx = static_cast<uint32_t>(((tb * 16 + l16) * D + k0 + cbw * 16 + 4 * g4) * 2);
  const uint32_t opa = static_cast<uint32_t>(lane * 4);
  const __amdgpu_buffer_rsrc_t r_none = buffer_rsrc(a.x, 0);
  const int xs_row = tid >> 3;
  const uint32_t xs_off = static_cast<uint32_t>(sidx<kT>(xs_row, 4 * (tid & 7)) * 2);

  // The last chunk (its tiles and the gate rows of the chunk before it) into
  // slot 0; its own gate rows into slot 1, which the first visit's loads
  // overwrite only after the gates are derived; then S dropped stores
  // (stream shape as in the loop).
  issue_chunk_b<D>(*rs[0], od, dy, g, x, st, eta, alpha, T, c_end - 1, in_seg(c_end - 2), k0,
                   wave);
  issue_gate_row(rs[1]->q, od.q, eta, alpha, T, c_end - 1, wave);
  store4(r_none, opa, 0.f);
  store8(r_none, odx, make_uint2(0, 0));
  wait_vm<S>();
  lds_barrier();
  if (wave == kGateWave) gates_b(rs[1]->q, m.gs[0], cv_of(c_end - 1), lane);

  // The two parts of dalpha of a chunk (lane = token), written into its gate
  // record; the store adds them.  Forward part: the <Lam_out, D_in> term,
  // the forward affine scan sum_{j<i} e(l_{i-1} - l_j)(-eta_j) pp_j, and
  // -kk_i / alpha_i.  Reversed part: sum_{u>i} e(l_{u-1} - l_i) rr_u and
  // sum_{u>i} (qq_u - kk_u), run on the reversed lane order with inputs read
  // from LDS reversed and the result written back reversed.
  const auto dalpha_fwd = [&](int par, GatesB& gt) {
    const float* dt = &dots_s[par][0][0][0];
    const int i = lane;
    const float pp = dt[0 * kC + i] + dt[4 * kC + 0 * kC + i];
    const float kk = dt[3 * kC + i] + dt[4 * kC + 3 * kC + i];
    float c0 = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) c0 += c0_s[par][w];
    const float al = gt.al[i], l = gt.li[i], lq = gt.lq[i], llast = gt.gam[1];
    float a2 = al, b2 = gt.nb[i] * pp;
    wave_scan_affine(a2, b2);
    const float s2 = wave_shift_up(b2, 0.f);
    gt.fpart[i] = fexp2(llast - l + lq) * c0 + fexp2(llast - l) * s2 -
                  kk * __builtin_amdgcn_rcpf(al);
  };
  const auto dalpha_rev = [&](int par, GatesB& gt) {
    const float* dt = &dots_s[par][0][0][0];
    const int ir = kC - 1 - lane;
    const auto both = [&](int kind) { return dt[kind * kC + ir] + dt[4 * kC + kind * kC + ir]; };
    const float rr_r = both(1), z_r = both(2) - both(3);
    const float al_r = gt.al[ir], lq_r = gt.lq[ir];
    float a3 = al_r, b3 = rr_r;
    wave_scan_affine(a3, b3);
    const float s3_r = wave_shift_up(b3, 0.f);
    const float zs_r = wave_shift_up(wave_scan_add(z_r), 0.f);
    gt.rpart[ir] = fexp2(lq_r) * s3_r + zs_r * __builtin_amdgcn_rcpf(al_r);
  };

  const auto step = [&](auto KC, int vis) {
    constexpr int K = decltype(KC)::value;
    SlotB<D>& cur = *rs[K];
    SlotB<D>& dst = *rs[K ^ 1];
    const int c = c_end - 1 - vis;
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = cv_of(c);
    GatesB& gc = m.gs[vis % 3];        // chunk c
    GatesB& gn = m.gs[(vis + 1) % 3];  // chunk c + 2, then (phase 2) chunk c - 1
    GatesB& gp = m.gs[(vis + 2) % 3];  // chunk c + 1
    wait_vm<S>();   // chunk c loaded: after it only the previous visit's stores
    lds_barrier();  // and the previous visit's reads of the other slot are done
    issue_chunk_b<D>(dst, od, dy, g, x, st, eta, alpha, T, in_seg(c - 1), in_seg(c - 2), k0, wave);

    // ---- phase 1
    {
      // this thread's 4 elements of e(lq_u) x_u[K]
      const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(cur.Xk) + xs_off);
      const float s = gc.eq[xs_row];
      uint2 r;
      r.x = pack2(bf16_val(v.x & 0xffffu) * s, bf16_val(v.x >> 16) * s);
      r.y = pack2(bf16_val(v.y & 0xffffu) * s, bf16_val(v.y >> 16) * s);
      *reinterpret_cast<uint2*>(reinterpret_cast<char*>(XS_s) + xs_off) = r;
    }
    be_block<D>(cur, gc, BeT_s, oD, oA, wave, lane);
    if (wave < 2) be_block<D>(cur, gc, BeT_s, oD, oA, wave + 8, lane);
    {
      // <Lam_out, D_in> over this wave's blocks
      float p = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const f32x4 sv = unpack4(get4<kT>(cur.Sn, oT, (tb + 4 * s) * 16, cbw * 16));
        p += lam[s][0] * sv[0] + lam[s][1] * sv[1] + lam[s][2] * sv[2] + lam[s][3] * sv[3];
      }
      p = wave_sum(p);
      if (lane == 0) c0_s[vis & 1][wave] = p;
    }
    {
      // dalpha of chunk c + 2 (its parts were formed in the previous visit);
      // the store stays outside the branch (one VMEM stream shape for all waves)
      const bool fin = wave == kDaWave && vis >= 2;
      const __amdgpu_buffer_rsrc_t r_pa =
          fin ? buffer_rsrc(pa + static_cast<int64_t>(c + 2) * kC, cv_of(c + 2) * 4) : r_none;
      float v = 0.f;
      if (wave == kDaWave) v = gn.fpart[lane] + gn.rpart[lane];
      store4(r_pa, opa, v);
    }
    lds_barrier();  // Be, e(lq) x visible; the gate record of chunk c + 2 is free

    // ---- phase 2: dx^T[c][i] of this wave's block, stored straight from the accumulators
    {
      const __bf16* L_in = L_s[vis & 1];
      f32x4 aws = zero4(), as_ = zero4(), al = zero4(), aq = zero4(), ak = zero4();
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8 df = frag_s<D>(cur.Dy, oD, tb * 16, kb * 32);
        aws = mfma16x16x32(w0f[kb], df, aws);
        as_ = mfma16x16x32(frag_ts<kT>(cur.Sn, oT, kb * 32, cbw * 16), df, as_);
        al = mfma16x16x32(frag_ts<kT>(L_in, oT, kb * 32, cbw * 16),
                          frag_s<D>(cur.G, oD, tb * 16, kb * 32), al);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 xf = frag_ts<kT>(cur.Xk, oT, kb * 32, cbw * 16);
        aq = mfma16x16x32(xf, frag_ts<kC>(BeT_s, oA, kb * 32, tb * 16), aq);
        ak = mfma16x16x32(xf, frag_s<kC>(BeT_s, oA, tb * 16, kb * 32), ak);
      }
      const int i = tb * 16 + l16;
      const float eqi = gc.eq[i], fl = gc.nb[i] * gc.e2[i];
      const f32x4 v = aws + as_ * eqi + aq + ak + al * fl;
      uint2 pk;
      pk.x = pack2(v[0], v[1]);
      pk.y = pack2(v[2], v[3]);
      store8(buffer_rsrc(dx + t0 * D, cv * D * 2), odx, pk);
      const f32x4 xv = unpack4(get4<kT>(cur.Xk, oT, tb * 16, cbw * 16));
      float pp = 0.f, rr = 0.f, qq = 0.f, kk = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pp += xv[q] * al[q];
        rr += xv[q] * as_[q];
        qq += xv[q] * aq[q];
        kk += xv[q] * ak[q];
      }
      pp = sum_rows(pp);
      rr = sum_rows(rr);
      qq = sum_rows(qq);
      kk = sum_rows(kk);
      if (g4 == 0) {
        float* dt = &dots_s[vis & 1][cbw][0][0];
        dt[0 * kC + i] = pp;
        dt[1 * kC + i] = rr;
        dt[2 * kC + i] = qq;
        dt[3 * kC + i] = kk;
      }
    }
    // Lam^T[c][r] = Gamma Lam^T + sum_u e(lq_u) x_u[c] dy_u[r]   (c in K)
    {
      bf16x8 xsf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) xsf[kb] = frag_ts<kT>(XS_s, oT, kb * 32, cbw * 16);
      const float gam = gc.gam[0];
      __bf16* L_out = L_s[(vis + 1) & 1];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int rb = tb + 4 * s;
        lam[s] = lam[s] * gam;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          lam[s] = mfma16x16x32(xsf[kb], frag_ts<D>(cur.Dy, oD, kb * 32, rb * 16), lam[s]);
        uint2 pk;
        pk.x = pack2(lam[s][0], lam[s][1]);
        pk.y = pack2(lam[s][2], lam[s][3]);
        put4<kT>(L_out, oT, rb * 16, cbw * 16, pk);
      }
    }
    // the gates of chunk c - 1 (its gate rows came with this chunk's tiles),
    // and the two parts of dalpha of chunk c + 1 (dots and partials of the
    // previous visit)
    if (wave == kGateWave) gates_b(cur.q, gn, cv_of(c - 1), lane);
    if (wave == kFwdWave && vis >= 1) dalpha_fwd((vis + 1) & 1, gp);
    if (wave == kRevWave && vis >= 1) dalpha_rev((vis + 1) & 1, gp);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  for (int vis = 0; vis < nloc; vis += 2) {
    step(I0{}, vis);
    if (vis + 1 >= nloc) break;
    step(I1{}, vis + 1);
  }
  // dalpha of the last two chunks: chunk c_beg + 1 has its parts, chunk
  // c_beg needs both
  wait_vm<0>();
  lds_barrier();
  const int vl = nloc - 1;
  GatesB& gl = m.gs[vl % 3];
  if (wave == kFwdWave) dalpha_fwd(vl & 1, gl);
  if (wave == kRevWave) dalpha_rev(vl & 1, gl);
  lds_barrier();
  if (wave == kDaWave) {
    if (nloc >= 2) {
      GatesB& g1 = m.gs[(vl + 2) % 3];
      store4(buffer_rsrc(pa + static_cast<int64_t>(c_beg + 1) * kC, cv_of(c_beg + 1) * 4), opa,
             g1.fpart[lane] + g1.rpart[lane]);
    }
    store4(buffer_rsrc(pa + static_cast<int64_t>(c_beg) * kC, cv_of(c_beg) * 4), opa,
           gl.fpart[lane] + gl.rpart[lane]);
  }
}

}  // namespace
}  // namespace gls
