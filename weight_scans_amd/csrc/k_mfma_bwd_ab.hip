// k_mfma_bwd_ab.hip -- both passes of the matrix-core reverse scan in one
// launch, for D = 64 (bf16 io).  The row-tile pass (dg, deta, dW0) and the
// column-tile pass (dx, dalpha; bwd_b.hpp) each fit in under half of a CU's
// LDS here, so a CU holds two work-groups -- typically one of each kind --
// and the two serial chains of a sequence-head run side by side instead of
// one after the other.
//
// Row-tile pass (mathematics as in k_mfma_bwd_a.hip; exact adjoint of the
// forward scan, GradLev abstract, omanscience.com), two chunk slots and two
// barriers per chunk:
//   phase 1: gates (every wave, same values), e(lq) dy of the row tile, P,
//            and the deta of the previous chunk (one wave);
//   phase 2: u, dg and the deta partials; the Lam and dW0 update.
#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "bwd_b.hpp"

namespace gls {
namespace {

constexpr int kFinWaveA = 7;

template <int D>
struct alignas(16) SlotA2 {
  __bf16 X[kC * D];    // x of the chunk, swizzled [token][D]
  __bf16 Dr[kC * kT];  // dy of the row tile, swizzled [token][kT]
  __bf16 Gr[kC * kT];  // g of the row tile, swizzled [token][kT]
  float q[2][4 * kC];  // eta = q[0][0..63], alpha = q[1][0..63]
};

struct alignas(16) GatesA2 {
  float lq[kC], li[kC], nb[kC], eq[kC], e2[kC];
  float gam[4];
};

template <int D>
struct DmaOffA2 {
  uint32_t x[D / 64];
  uint32_t t;
  uint32_t q;
};
template <int D>
__device__ __forceinline__ DmaOffA2<D> dma_off_a2(int wave, int lane) {
  constexpr int U = D / 8;
  DmaOffA2<D> o;
#pragma unroll
  for (int s = 0; s < D / 64; ++s) {
    const int p = (wave + 8 * s) * 64 + lane;
    const int row = p / U, kl = (p % U) ^ swz<D>(row);
    o.x[s] = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  }
  const int p = (wave & 3) * 64 + lane;
  const int row = p >> 2, kl = (p & 3) ^ swz<kT>(row);
  o.t = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  o.q = static_cast<uint32_t>(lane * 16);
  return o;
}

template <int D>
__device__ __forceinline__ void issue_chunk_a2(SlotA2<D>& sl, const DmaOffA2<D>& o,
                                               const uint16_t* x, const uint16_t* dy,
                                               const uint16_t* g, const float* eta,
                                               const float* alpha, int64_t T, int k, int r0,
                                               int wave) {
  const bool in = k >= 0;
  const int64_t t0 = in ? static_cast<int64_t>(k) * kC : 0;
  const int cv = in ? static_cast<int>(std::min<int64_t>(kC, T - t0)) : 0;
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + t0 * D, cv * D * 2);
#pragma unroll
  for (int s = 0; s < D / 64; ++s) dma16(rx, o.x[s], sl.X + (wave + 8 * s) * 512);
  const __amdgpu_buffer_rsrc_t rt =
      buffer_rsrc((wave < 4 ? dy : g) + t0 * D + r0, cv > 0 ? (cv * D - r0) * 2 : 0);
  const int t_off = (wave < 4 ? static_cast<int>(offsetof(SlotA2<D>, Dr))
                              : static_cast<int>(offsetof(SlotA2<D>, Gr))) + (wave & 3) * 1024;
  dma16(rt, o.t, reinterpret_cast<char*>(&sl) + t_off);
  const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(((wave & 1) == 0 ? eta : alpha) + t0, cv * 4);
  dma16(rq, o.q, reinterpret_cast<char*>(&sl) + static_cast<int>(offsetof(SlotA2<D>, q)) +
                     (wave & 1) * 1024);
}

// LDS objects of the row-tile pass (separate LDS variables in the caller;
// the adjoint-only instance never touches PT, L0, L1 and red).
template <int D>
struct SmemA2 {
  SlotA2<D>& ring0;
  SlotA2<D>& ring1;
  __bf16* PT;   // [kC * kC]  PT[i][u] = P_ui, swizzled
  __bf16* L0;   // [kT * D]   Lam_out rows of the tile (bf16), even visits
  __bf16* L1;   // [kT * D]   odd visits
  __bf16* DS;   // [kC * kT]  e(lq_u) dy_u of the row tile
  GatesA2& gs;
  float* red;   // [2][2][kC] deta partial by parity, row block
};

// The row-tile pass for sequence-head bh, row tile `tile`, segment `seg`
// (chunks seg * seg_chunks .. , visited from the last; Lam entering from the
// right is seg_lam, or zero).  LAM_ONLY: the adjoint-only pass of the
// segmented scan -- no P, u, dg, deta or dW0; it reports the tile's rows of
// Lam at the segment's left end (zero start) and the summed log2 alpha.
template <int D, bool LAM_ONLY>
__device__ __forceinline__ void role_a2_body(const BwdArgs& a, int64_t bh, int tile, int seg,
                                             const SmemA2<D>& m) {
  static_assert(D == 64 || D == 128, "D");
  constexpr int NS = D / 64;
  // stores per wave per chunk: deta (or a dropped one), then dg -- or, in
  // the adjoint-only pass, the NS blocks of Lam_out (dropped unless stored)
  constexpr int S = LAM_ONLY ? 1 + NS : 2;
  SlotA2<D>* const rs[2] = {&m.ring0, &m.ring1};
  __bf16* const L_s[2] = {m.L0, m.L1};
  GatesA2& gs = m.gs;
  float (*red_s)[2][kC] = reinterpret_cast<float (*)[2][kC]>(m.red);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int tb = wave >> 1, rbw = wave & 1;
  const int r0 = tile * kT;
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
  uint16_t* dg = static_cast<uint16_t*>(a.dg) + bh * T * D;
  float* pe = static_cast<float*>(a.part_eta) + tile * BHT + bh * T;

  if constexpr (!LAM_ONLY)
    for (int idx = tid; idx < kC * kC / 8; idx += kNT)
      reinterpret_cast<uint4*>(m.PT)[idx] = make_uint4(0, 0, 0, 0);

  // valid tokens of chunk c (none outside this segment)
  const auto cv_of = [&](int c) {
    return (c < c_beg || c >= c_end)
               ? 0
               : static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };
  const LaneOff<D> oX = lane_off<D>(lane);
  const LaneOff<kT> oT = lane_off<kT>(lane);
  const LaneOff<kC> oA = lane_off<kC>(lane);
  const DmaOffA2<D> od = dma_off_a2<D>(wave, lane);
  const uint32_t odg = static_cast<uint32_t>(((tb * 16 + l16) * D + r0 + rbw * 16 + 4 * g4) * 2);
  const uint32_t ope = static_cast<uint32_t>(lane * 4);
  const __amdgpu_buffer_rsrc_t r_none = buffer_rsrc(a.x, 0);
  const int ds_row = tid >> 3;
  const uint32_t ds_off = static_cast<uint32_t>(sidx<kT>(ds_row, 4 * (tid & 7)) * 2);

  // Lam rows of the tile entering from the right (fp32 accumulators, and the
  // bf16 copy read by the first visit)
  f32x4 lam[NS], dw[NS];
  if (a.seg_lam) {
    const float* sl = a.seg_lam + (bh * a.n_seg + seg) * D * D;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      lam[s] = *reinterpret_cast<const f32x4*>(sl + (r0 + rbw * 16 + l16) * D + (tb + 4 * s) * 16 +
                                               4 * g4);
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) lam[s] = zero4();
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    dw[s] = zero4();
    if constexpr (!LAM_ONLY) {
      uint2 pk;
      pk.x = pack2(lam[s][0], lam[s][1]);
      pk.y = pack2(lam[s][2], lam[s][3]);
      put4<D>(L_s[0], oX, rbw * 16, (tb + 4 * s) * 16, pk);
    }
  }
  wait_vm<0>();

  issue_chunk_a2<D>(*rs[0], od, x, dy, g, eta, alpha, T, c_end - 1, r0, wave);
#pragma unroll
  for (int k = 0; k < S - 1; ++k) store8(r_none, odg + 64 * k, make_uint2(0, 0));  // not merged
  store4(r_none, ope, 0.f);
  // Lam_out stores of the adjoint-only pass: rows of this wave's blocks
  uint16_t* lo = a.lam_out ? static_cast<uint16_t*>(a.lam_out) + bh * static_cast<int64_t>(n) * D * D
                           : nullptr;
  uint32_t olo[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    olo[s] = static_cast<uint32_t>(((r0 + rbw * 16 + l16) * D + (tb + 4 * s) * 16 + 4 * g4) * 2);
  float lsum = 0.f;  // sum of l_last over the segment (adjoint-only pass)

  const auto step = [&](auto KC, int vis) {
    constexpr int K = decltype(KC)::value;
    SlotA2<D>& cur = *rs[K];
    SlotA2<D>& dst = *rs[K ^ 1];
    const int c = c_end - 1 - vis;
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = cv_of(c);
    wait_vm<S>();
    lds_barrier();
    issue_chunk_a2<D>(dst, od, x, dy, g, eta, alpha, T, c - 1 >= c_beg ? c - 1 : -1, r0, wave);

    // ---- phase 1: gates (same values from every wave), e(lq) dy, P
    {
      const float et = lane < cv ? cur.q[0][lane] : 0.f;
      const ChunkGates gt = chunk_gates(lane < cv ? cur.q[1][lane] : 1.f, lane);
      gs.lq[lane] = gt.lq;
      gs.li[lane] = gt.l;
      gs.nb[lane] = -et;
      gs.eq[lane] = fexp2(gt.lq);
      gs.e2[lane] = fexp2(gt.llast - gt.l);
      if (lane == 0) gs.gam[0] = fexp2(gt.llast);
      lsum += gt.llast;
    }
    {
      const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(cur.Dr) + ds_off);
      const float s = gs.eq[ds_row];
      uint2 r;
      r.x = pack2(bf16_val(v.x & 0xffffu) * s, bf16_val(v.x >> 16) * s);
      r.y = pack2(bf16_val(v.y & 0xffffu) * s, bf16_val(v.y >> 16) * s);
      *reinterpret_cast<uint2*>(reinterpret_cast<char*>(m.DS) + ds_off) = r;
    }
    const auto p_block = [&](int b) {
      const int ub = tri_i(b), ib = tri_j(b);
      f32x4 xx = zero4();
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
        xx = mfma16x16x32(frag_s<D>(cur.X, oX, ub * 16, kb * 32),
                          frag_s<D>(cur.X, oX, ib * 16, kb * 32), xx);
      const int i = ib * 16 + l16, u0 = ub * 16 + 4 * g4;
      const float li = gs.li[i];
      const f32x4 lqu = *reinterpret_cast<const f32x4*>(&gs.lq[u0]);
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float e = xx[q] * fexp2(lqu[q] - li);
        v[q] = (i < u0 + q) ? e : 0.f;
      }
      uint2 pk;
      pk.x = pack2(v[0], v[1]);
      pk.y = pack2(v[2], v[3]);
      put4<kC>(m.PT, oA, ib * 16, ub * 16, pk);
    };
    if constexpr (!LAM_ONLY) {
      p_block(wave);
      if (wave < 2) p_block(wave + 8);
    }
    {
      // deta of chunk c + 1: sum of the two row-block partials
      const int cn = c + 1;
      const bool fin = !LAM_ONLY && wave == kFinWaveA && vis > 0;
      const __amdgpu_buffer_rsrc_t r_pe =
          fin ? buffer_rsrc(pe + static_cast<int64_t>(cn) * kC, cv_of(cn) * 4) : r_none;
      float val = 0.f;
      if constexpr (!LAM_ONLY) {
        const float* rd = &red_s[(vis + 1) & 1][0][0];
        val = -(rd[lane] + rd[kC + lane]);
      }
      store4(r_pe, ope, val);
    }
    lds_barrier();  // gates, e(lq) dy, P visible

    // ---- phase 2: u, dg, deta partials
    if constexpr (LAM_ONLY) {
      // Lam_out of chunk c (the adjoint entering it from the right), bf16
      const __amdgpu_buffer_rsrc_t r_lo =
          lo ? buffer_rsrc(lo + static_cast<int64_t>(c) * D * D, D * D * 2) : r_none;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        uint2 pk;
        pk.x = pack2(lam[s][0], lam[s][1]);
        pk.y = pack2(lam[s][2], lam[s][3]);
        store8(r_lo, olo[s], pk);
      }
    } else {
      const __bf16* L_in = L_s[vis & 1];
      f32x4 ain = zero4(), apd = zero4();
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
        ain = mfma16x16x32(frag_s<D>(L_in, oX, rbw * 16, kb * 32),
                           frag_s<D>(cur.X, oX, tb * 16, kb * 32), ain);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        apd = mfma16x16x32(frag_ts<kT>(cur.Dr, oT, kb * 32, rbw * 16),
                           frag_s<kC>(m.PT, oA, tb * 16, kb * 32), apd);
      const int i = tb * 16 + l16;
      const float e2 = gs.e2[i], ne = gs.nb[i];
      const f32x4 u = ain * e2 + apd;
      uint2 pk;
      pk.x = pack2(u[0] * ne, u[1] * ne);
      pk.y = pack2(u[2] * ne, u[3] * ne);
      store8(buffer_rsrc(dg + t0 * D, cv * D * 2), odg, pk);
      const uint2 gv = get4<kT>(cur.Gr, oT, tb * 16, rbw * 16);
      float p = bf16_val(gv.x & 0xffffu) * u[0] + bf16_val(gv.x >> 16) * u[1] +
                bf16_val(gv.y & 0xffffu) * u[2] + bf16_val(gv.y >> 16) * u[3];
      p = sum_rows(p);
      if (g4 == 0) red_s[vis & 1][rbw][i] = p;
    }
    // Lam^T[c][r] = Gamma Lam^T + sum_u x_u[c] e(lq_u) dy_u[r];  dW0^T += sum_u x_u[c] dy_u[r]
    {
      bf16x8 dsf[2], drf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dsf[kb] = frag_ts<kT>(m.DS, oT, kb * 32, rbw * 16);
        drf[kb] = frag_ts<kT>(cur.Dr, oT, kb * 32, rbw * 16);
      }
      const float gam = gs.gam[0];
      __bf16* L_out = L_s[(vis + 1) & 1];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int cb = tb + 4 * s;
        lam[s] = lam[s] * gam;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 xa = frag_ts<D>(cur.X, oX, kb * 32, cb * 16);
          lam[s] = mfma16x16x32(xa, dsf[kb], lam[s]);
          if constexpr (!LAM_ONLY) dw[s] = mfma16x16x32(xa, drf[kb], dw[s]);
        }
        if constexpr (!LAM_ONLY) {
          uint2 pk;
          pk.x = pack2(lam[s][0], lam[s][1]);
          pk.y = pack2(lam[s][2], lam[s][3]);
          put4<D>(L_out, oX, rbw * 16, cb * 16, pk);
        }
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  for (int vis = 0; vis < nloc; vis += 2) {
    step(I0{}, vis);
    if (vis + 1 >= nloc) break;
    step(I1{}, vis + 1);
  }
  wait_vm<0>();
  lds_barrier();
  if constexpr (LAM_ONLY) {
    if (a.seg_out) {
      float* so = a.seg_out + (bh * a.n_seg + seg) * D * D;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int cb = tb + 4 * s;
        *reinterpret_cast<f32x4*>(so + (r0 + rbw * 16 + l16) * D + cb * 16 + 4 * g4) = lam[s];
      }
      if (tile == 0 && wave == 0 && lane == 0) a.seg_lg[bh * a.n_seg + seg] = lsum;
    }
  } else {
    if (wave == kFinWaveA) {
      const float* rd = &red_s[(nloc - 1) & 1][0][0];
      store4(buffer_rsrc(pe + static_cast<int64_t>(c_beg) * kC, cv_of(c_beg) * 4), ope,
             -(rd[lane] + rd[kC + lane]));
    }
    float* pw = static_cast<float*>(a.part_dW0) + (seg * a.B * a.H + bh) * D * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int cb = tb + 4 * s;
      *reinterpret_cast<f32x4*>(pw + (r0 + rbw * 16 + l16) * D + cb * 16 + 4 * g4) = dw[s];
    }
  }
}

// One launch, both passes.  Per group of 8 sequence-heads the work-groups are
// (row tile 0, col tile 0, row tile 1, col tile 1, ...) x 8 heads, so row and
// column work-groups alternate in dispatch order; all of a head's
// work-groups land on one XCD.  The LDS objects are shared by the two kinds
// (each kind uses them with its own layout).
constexpr int kD = 64;
constexpr size_t kRingBytes =
    sizeof(SlotB<kD>) > sizeof(SlotA2<kD>) ? sizeof(SlotB<kD>) : sizeof(SlotA2<kD>);
constexpr size_t kGateBytes =
    3 * sizeof(GatesB) > sizeof(GatesA2) ? 3 * sizeof(GatesB) : sizeof(GatesA2);

__global__ __launch_bounds__(kNT, 4) void bwd_ab64(BwdArgs a) {
  __shared__ alignas(16) char ring0[kRingBytes], ring1[kRingBytes];
  __shared__ alignas(16) __bf16 tt_s[kC * kC];    // P^T | Be^T
  __shared__ alignas(16) __bf16 L0_s[kD * kT], L1_s[kD * kT];
  __shared__ alignas(16) __bf16 sc_s[kC * kT];    // e(lq) dy rows | e(lq) x cols
  __shared__ alignas(16) char gs_s[kGateBytes];
  __shared__ alignas(16) float red_s[2 * 2 * 4 * kC + 2 * kNW];
  constexpr int NTILE = kD / kT;
  // (segment is the slowest index, so the XCD of a head does not change)
  const int per_seg = static_cast<int>((a.B * a.H + 7) / 8) * 16 * NTILE;
  const int seg = blockIdx.x / per_seg, bid = blockIdx.x % per_seg;
  const int grp = bid / (16 * NTILE), within = bid % (16 * NTILE);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  if (bh >= a.B * a.H) return;
  const int sub = within >> 3, tile = sub >> 1;
  if ((sub & 1) == 0) {
    const SmemA2<kD> m{*reinterpret_cast<SlotA2<kD>*>(ring0), *reinterpret_cast<SlotA2<kD>*>(ring1),
                       tt_s, L0_s, L1_s, sc_s, *reinterpret_cast<GatesA2*>(gs_s), red_s};
    role_a2_body<kD, false>(a, bh, tile, seg, m);
  } else {
    const SmemB<kD> m{*reinterpret_cast<SlotB<kD>*>(ring0), *reinterpret_cast<SlotB<kD>*>(ring1),
                      tt_s, L0_s, L1_s, sc_s, reinterpret_cast<GatesB*>(gs_s), red_s,
                      red_s + 2 * 2 * 4 * kC};
    role_b_body<kD>(a, bh, tile, seg, m);
  }
}

// Adjoint-only pass of the segmented reverse scan: one work-group per
// (segment, head, row tile).
template <int D>
__global__ __launch_bounds__(kNT) void bwd_lam(BwdArgs a) {
  __shared__ SlotA2<D> ring0, ring1;
  __shared__ __bf16 DS_s[kC * kT];
  __shared__ GatesA2 gs;
  constexpr int NTILE = D / kT;
  const int per_seg = static_cast<int>((a.B * a.H + 7) / 8) * 8 * NTILE;
  // segment 0's own adjoint is never used (nothing lies to its left): the
  // pass covers segments 1 .. n_seg - 1
  const int seg = 1 + static_cast<int>(blockIdx.x / per_seg), bid = blockIdx.x % per_seg;
  const int grp = bid / (8 * NTILE), within = bid % (8 * NTILE);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  if (bh >= a.B * a.H) return;
  const SmemA2<D> m{ring0, ring1, nullptr, nullptr, nullptr, DS_s, gs, nullptr};
  role_a2_body<D, true>(a, bh, within >> 3, seg, m);
}

template <int D>
hipError_t launch_lam(const BwdArgs& a, hipStream_t s) {
  const int64_t groups = (a.B * a.H + 7) / 8;
  if (a.n_seg <= 1) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (D / kT) * (a.n_seg - 1)));
  hipLaunchKernelGGL(bwd_lam<D>, grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_bwd_ab64(const BwdArgs& a, hipStream_t s) {
  const int64_t groups = (a.B * a.H + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 16 * (kD / kT) * a.n_seg));
  hipLaunchKernelGGL(bwd_ab64, grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mfma_bwd_lam(const BwdArgs& a, hipStream_t s) {
  return a.d_in == 128 ? launch_lam<128>(a, s) : launch_lam<64>(a, s);
}

}  // namespace gls
