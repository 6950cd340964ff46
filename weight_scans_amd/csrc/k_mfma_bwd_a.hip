// k_mfma_bwd_a.hip -- matrix-core reverse scan, row tiles of the adjoint
// (bf16 io, d_in = d_out = D in {64, 128}; gfx950, v_mfma_f32_16x16x32_bf16).
//
// The exact adjoint of the forward scan for L = sum_t <dy_t, y_t> (the
// gradients propagate "in reverse" with exact parallel scans: GradLev
// abstract, omanscience.com).  Walking the chunks backwards (chunk-local
// l = inclusive cumsum of log2 alpha, lq_i = l_{i-1}, e(.) = 2^(.)), the
// adjoint Lam = dL/dD after a token is carried as
//   Lam_in = e(l_last) Lam_out + sum_u e(lq_u) dy_u x_u^T
// and, with P_ui = e(lq_u - l_i) (x_u . x_i) for u > i:
//   u_i = e(l_last - l_i) Lam_out x_i + sum_{u>i} P_ui dy_u
//   dg_i = -eta_i u_i,   deta_i = -g_i . u_i,   dW0 += sum_u dy_u x_u^T.
// One work-group owns one sequence-head and one tile of kT = 32 rows of Lam
// (rows are independent chains: u reduces over columns), so it produces dg
// for its rows, its rows' share of deta (summed over the tiles later, in a
// fixed order) and its rows of the dW0 partial.
//
// Pipeline (one work-group barrier per chunk; as in the forward kernel):
// chunk tiles stream HBM -> LDS by direct buffer loads into a ring of R
// slots; while chunk c is finished (u, dg, the Lam update), P and the scaled
// dy tile of chunk c - 1 are formed and one wave derives the gates of chunk
// c - 2.  Eight waves: wave w owns the 16 x 16 block (token block w/2, row
// block w%2) of u and D/64 16 x 16 blocks of Lam and dW0.
#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kC = 64;         // tokens per chunk
constexpr int kT = 32;         // rows of Lam per work-group
constexpr int kNW = 8;         // waves per work-group
constexpr int kNT = 64 * kNW;  // threads
constexpr int kPrepWave = 2;   // derives the gates
constexpr int kFinWave = 7;    // sums and stores the deta partials

template <int D>
constexpr int kRingA = D == 64 ? 5 : 4;  // chunk slots (LDS bound at D = 128)

// Gate rows of a chunk: eta / alpha as loaded, then (same bytes, after the
// gate pass; i = token, b = its 16-token block, m_b = l_{16 b - 1}, m_0 = 0)
//   R_i = e(lq_i - m_b),  C_{b', i} = e(m_b' - l_i)  (b' = 1..3),
//   e2_i = e(l_last - l_i),  eq_i = e(lq_i)
// so that e(lq_u - l_i) = R_u C_{b', i} when u is in block b' > block of i.
struct GateRowsA {
  float eta[kC], R[kC], C1[kC], C2[kC];
  float alpha[kC], C3[kC], e2[kC], eq[kC];
};

template <int D>
struct alignas(16) SlotA {
  __bf16 X[kC * D];     // x of the chunk, swizzled [token][D]
  __bf16 Dr[kC * kT];   // dy of the row tile, swizzled [token][kT]
  __bf16 Gr[kC * kT];   // g of the row tile, swizzled [token][kT]
  union {
    float q[2][4 * kC];  // loaded: eta = q[0][0..63], alpha = q[1][0..63]
    GateRowsA f;
  };
  float lq[kC], li[kC], nb[kC], pad_[kC];  // l_{i-1}, l_i, -eta_i
  float gam[4];                            // gam[0] = e(l_last)
};

// Per-lane byte offsets of the chunk loads.  Wave w loads x units of
// instructions w + 8 s, a quarter of the dy (w < 4) or g (w >= 4) row tile,
// and a gate row (w even: eta, odd: alpha; four waves write the same bytes).
template <int D>
struct DmaOffA {
  uint32_t x[D / 64];
  uint32_t t;  // dy / g tile
  uint32_t q;  // gate row
};
template <int D>
__device__ __forceinline__ DmaOffA<D> dma_off_a(int wave, int lane) {
  constexpr int U = D / 8;
  DmaOffA<D> o;
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
constexpr int kLoadOpsA = D / 64 + 2;

template <int D>
__device__ __forceinline__ void issue_chunk_a(SlotA<D>& sl, const DmaOffA<D>& o, const uint16_t* x,
                                              const uint16_t* dy, const uint16_t* g,
                                              const float* eta, const float* alpha, int64_t T,
                                              int k, int r0, int wave) {
  const bool in = k >= 0;
  const int64_t t0 = in ? static_cast<int64_t>(k) * kC : 0;
  const int cv = in ? static_cast<int>(std::min<int64_t>(kC, T - t0)) : 0;
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + t0 * D, cv * D * 2);
#pragma unroll
  for (int s = 0; s < D / 64; ++s) dma16(rx, o.x[s], sl.X + (wave + 8 * s) * 512);
  // the same instructions in every wave: scalar-selected sources / destinations
  const __amdgpu_buffer_rsrc_t rt =
      buffer_rsrc((wave < 4 ? dy : g) + t0 * D + r0, cv > 0 ? (cv * D - r0) * 2 : 0);
  const int t_off = (wave < 4 ? static_cast<int>(offsetof(SlotA<D>, Dr))
                              : static_cast<int>(offsetof(SlotA<D>, Gr))) + (wave & 3) * 1024;
  dma16(rt, o.t, reinterpret_cast<char*>(&sl) + t_off);
  const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(((wave & 1) == 0 ? eta : alpha) + t0, cv * 4);
  dma16(rq, o.q, reinterpret_cast<char*>(&sl) + static_cast<int>(offsetof(SlotA<D>, q)) +
                     (wave & 1) * 1024);
}

// Gates of a chunk, lane = token (one wave).
template <int D>
__device__ __forceinline__ void prep_gates_a(SlotA<D>& sl, int cv, int lane) {
  const float et = lane < cv ? sl.f.eta[lane] : 0.f;
  const ChunkGates gt = chunk_gates(lane < cv ? sl.f.alpha[lane] : 1.f, lane);
  const float m1 = readlane_f(gt.l, 15), m2 = readlane_f(gt.l, 31), m3 = readlane_f(gt.l, 47);
  const int b = lane >> 4;
  const float mb = b == 0 ? 0.f : b == 1 ? m1 : b == 2 ? m2 : m3;
  sl.lq[lane] = gt.lq;
  sl.li[lane] = gt.l;
  sl.nb[lane] = -et;
  sl.f.e2[lane] = fexp2(gt.llast - gt.l);
  sl.f.eq[lane] = fexp2(gt.lq);
  sl.f.R[lane] = fexp2(gt.lq - mb);
  sl.f.C1[lane] = fexp2(fminf(m1 - gt.l, 0.f));
  sl.f.C2[lane] = fexp2(fminf(m2 - gt.l, 0.f));
  sl.f.C3[lane] = fexp2(fminf(m3 - gt.l, 0.f));
  if (lane == 0) sl.gam[0] = fexp2(gt.llast);
}

// Block b (0..9) of P^T for a chunk: PT[i][u] = P_ui for u > i (u block
// tri_i(b) >= i block tri_j(b)); blocks below the diagonal stay zero.
template <int D>
__device__ __forceinline__ void p_block(const SlotA<D>& sl, __bf16* PT, const LaneOff<D>& oX,
                                        const LaneOff<kC>& oA, int b, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const int ub = tri_i(b), ib = tri_j(b);
  f32x4 xx = zero4();
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
    xx = mfma16x16x32(frag_s<D>(sl.X, oX, ub * 16, kb * 32), frag_s<D>(sl.X, oX, ib * 16, kb * 32),
                      xx);
  const int i = ib * 16 + l16, u0 = ub * 16 + 4 * g4;
  f32x4 v;
  if (ub == ib) {
    const float li = sl.li[i];
    const f32x4 lqu = *reinterpret_cast<const f32x4*>(&sl.lq[u0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float e = xx[q] * fexp2(lqu[q] - li);
      v[q] = (i < u0 + q) ? e : 0.f;
    }
  } else {
    const float ci = (ub == 1 ? sl.f.C1 : ub == 2 ? sl.f.C2 : sl.f.C3)[i];
    const f32x4 ru = *reinterpret_cast<const f32x4*>(&sl.f.R[u0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = xx[q] * (ru[q] * ci);
  }
  uint2 pk;
  pk.x = pack2(v[0], v[1]);
  pk.y = pack2(v[2], v[3]);
  put4<kC>(PT, oA, ib * 16, ub * 16, pk);
}

// One thread's 4 elements of the scaled dy tile: DS[u][r] = bf16(e(lq_u) dy_u[r]).
template <int D>
__device__ __forceinline__ void scale_dy(const SlotA<D>& sl, __bf16* DS, uint32_t off, int row) {
  const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(sl.Dr) + off);
  const float s = sl.f.eq[row];
  uint2 r;
  r.x = pack2(bf16_val(v.x & 0xffffu) * s, bf16_val(v.x >> 16) * s);
  r.y = pack2(bf16_val(v.y & 0xffffu) * s, bf16_val(v.y >> 16) * s);
  *reinterpret_cast<uint2*>(reinterpret_cast<char*>(DS) + off) = r;
}

template <int D>
__global__ __launch_bounds__(kNT) void bwd_a(BwdArgs a) {
  static_assert(D == 64 || D == 128, "D");
  constexpr int R = kRingA<D>;
  constexpr int NTILE = D / kT;
  constexpr int NS = D / 64;  // 16x16 Lam / dW0 blocks per wave
  constexpr int P = kLoadOpsA<D>;
  constexpr int S = 2;        // stores per wave per chunk: dg, deta (or a dropped one)
  __shared__ SlotA<D> ring0, ring1, ring2, ring3, ring4;
  __shared__ __bf16 PT_s[2][kC * kC];   // P^T by chunk parity, swizzled
  __shared__ __bf16 L_s[2][kT * D];     // Lam_out rows of the tile (bf16), by parity
  __shared__ __bf16 DS_s[2][kC * kT];   // e(lq) dy of the row tile, by parity
  __shared__ float red_s[2][2][kC];     // deta partial per row block, by parity
  SlotA<D>* const rs[5] = {&ring0, &ring1, &ring2, &ring3, R == 5 ? &ring4 : &ring0};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int tb = wave >> 1, rbw = wave & 1;
  // (segment is the slowest index, so the XCD of a head does not change)
  const int per_seg = static_cast<int>((a.B * a.H + 7) / 8) * 8 * NTILE;
  const int seg = blockIdx.x / per_seg, bid = blockIdx.x % per_seg;
  const int grp = bid / (8 * NTILE), within = bid % (8 * NTILE);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  const int tile = within >> 3;
  if (bh >= a.B * a.H) return;
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

  for (int idx = tid; idx < 2 * kC * kC / 8; idx += kNT)
    reinterpret_cast<uint4*>(&PT_s[0][0])[idx] = make_uint4(0, 0, 0, 0);

  // valid tokens of chunk c (none outside this segment)
  const auto cv_of = [&](int c) {
    return (c < c_beg || c >= c_end)
               ? 0
               : static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };
  // chunk index to load for visit v (-1: nothing, a zero fill)
  const auto chunk_at = [&](int v) { return c_end - 1 - v >= c_beg ? c_end - 1 - v : -1; };
  const LaneOff<D> oX = lane_off<D>(lane);
  const LaneOff<kT> oT = lane_off<kT>(lane);
  const LaneOff<kC> oA = lane_off<kC>(lane);
  const DmaOffA<D> od = dma_off_a<D>(wave, lane);
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
    uint2 pk;
    pk.x = pack2(lam[s][0], lam[s][1]);
    pk.y = pack2(lam[s][2], lam[s][3]);
    put4<D>(L_s[0], oX, rbw * 16, (tb + 4 * s) * 16, pk);
  }
  wait_vm<0>();

  // Chunks are visited from the last to the first; visit v handles chunk
  // n - 1 - v, which lives in ring slot v % R.
  // Initial loads, each followed by S dropped stores (stream shape as in the loop).
#pragma unroll
  for (int v = 0; v < R - 1; ++v) {
    issue_chunk_a<D>(*rs[v], od, x, dy, g, eta, alpha, T, chunk_at(v), r0, wave);
    store8(r_none, odg + v, make_uint2(0, 0));
    store4(r_none, ope + v, 0.f);
  }
  // chunks n-1 and n-2 loaded: after the latter come S + (R - 3) (P + S) instructions
  wait_vm<S + (R - 3) * (P + S)>();
  lds_barrier();
  if (wave == kPrepWave) {
    prep_gates_a<D>(*rs[0], cv_of(c_end - 1), lane);
    prep_gates_a<D>(*rs[1], cv_of(c_end - 2), lane);
  }
  lds_barrier();
  scale_dy<D>(*rs[0], DS_s[0], ds_off, ds_row);
  p_block<D>(*rs[0], PT_s[0], oX, oA, wave, lane);
  if (wave < 2) p_block<D>(*rs[0], PT_s[0], oX, oA, wave + 8, lane);

  const auto step = [&](auto KC, int v) {
    constexpr int K = decltype(KC)::value;
    SlotA<D>& cur = *rs[K];
    SlotA<D>& nx1 = *rs[(K + 1) % R];
    SlotA<D>& nx2 = *rs[(K + 2) % R];
    SlotA<D>& dst = *rs[(K + R - 1) % R];
    const int c = c_end - 1 - v;
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = cv_of(c);
    // chunk c - 2 loaded (past the first chunk: a zero fill)
    wait_vm<S + (R - 4) * (P + S)>();
    lds_barrier();  // P, scaled dy, gates of c - 1; Lam_out and deta partials of c + 1 visible
    issue_chunk_a<D>(dst, od, x, dy, g, eta, alpha, T, chunk_at(v + R - 1), r0, wave);

    // deta of chunk c + 1: sum of the two row-block partials
    {
      const int cn = c + 1;
      const bool fin = wave == kFinWave && cn < c_end;
      const __amdgpu_buffer_rsrc_t r_pe =
          fin ? buffer_rsrc(pe + static_cast<int64_t>(cn) * kC, cv_of(cn) * 4) : r_none;
      const float* rd = &red_s[(v + 1) & 1][0][0];
      store4(r_pe, ope, -(rd[lane] + rd[kC + lane]));
    }
    if (wave == kPrepWave) prep_gates_a<D>(nx2, cv_of(c - 2), lane);
    scale_dy<D>(nx1, DS_s[(v + 1) & 1], ds_off, ds_row);
    p_block<D>(nx1, PT_s[(v + 1) & 1], oX, oA, wave, lane);
    if (wave < 2) p_block<D>(nx1, PT_s[(v + 1) & 1], oX, oA, wave + 8, lane);

    {
      // u^T[r][i] for this wave's block; dg stored straight from the
      // accumulators (4 rows of one token per lane); deta partial to LDS
      const __bf16* L_in = L_s[v & 1];
      const __bf16* PT = PT_s[v & 1];
      f32x4 ain = zero4(), apd = zero4();
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
        ain = mfma16x16x32(frag_s<D>(L_in, oX, rbw * 16, kb * 32),
                           frag_s<D>(cur.X, oX, tb * 16, kb * 32), ain);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        apd = mfma16x16x32(frag_ts<kT>(cur.Dr, oT, kb * 32, rbw * 16),
                           frag_s<kC>(PT, oA, tb * 16, kb * 32), apd);
      const int i = tb * 16 + l16;
      const float e2 = cur.f.e2[i], ne = cur.nb[i];
      const f32x4 u = ain * e2 + apd;
      uint2 pk;
      pk.x = pack2(u[0] * ne, u[1] * ne);
      pk.y = pack2(u[2] * ne, u[3] * ne);
      store8(buffer_rsrc(dg + t0 * D, cv * D * 2), odg, pk);
      const uint2 gv = get4<kT>(cur.Gr, oT, tb * 16, rbw * 16);
      float p = bf16_val(gv.x & 0xffffu) * u[0] + bf16_val(gv.x >> 16) * u[1] +
                bf16_val(gv.y & 0xffffu) * u[2] + bf16_val(gv.y >> 16) * u[3];
      p = sum_rows(p);
      if (g4 == 0) red_s[v & 1][rbw][i] = p;
    }

    // Lam^T[c][r] = Gamma Lam^T + sum_u x_u[c] e(lq_u) dy_u[r];  dW0^T += sum_u x_u[c] dy_u[r]
    // (into the other Lam buffer: the current one may still be read)
    {
      const __bf16* DS = DS_s[v & 1];
      bf16x8 dsf[2], drf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dsf[kb] = frag_ts<kT>(DS, oT, kb * 32, rbw * 16);
        drf[kb] = frag_ts<kT>(cur.Dr, oT, kb * 32, rbw * 16);
      }
      const float gam = cur.gam[0];
      __bf16* L_out = L_s[(v + 1) & 1];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int cb = tb + 4 * s;
        lam[s] = lam[s] * gam;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 xa = frag_ts<D>(cur.X, oX, kb * 32, cb * 16);
          lam[s] = mfma16x16x32(xa, dsf[kb], lam[s]);
          dw[s] = mfma16x16x32(xa, drf[kb], dw[s]);
        }
        uint2 pk;
        pk.x = pack2(lam[s][0], lam[s][1]);
        pk.y = pack2(lam[s][2], lam[s][3]);
        put4<D>(L_out, oX, rbw * 16, cb * 16, pk);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  for (int v = 0; v < nloc; v += R) {
    step(I0{}, v);
    if (v + 1 >= nloc) break;
    step(I1{}, v + 1);
    if (v + 2 >= nloc) break;
    step(I2{}, v + 2);
    if (v + 3 >= nloc) break;
    step(I3{}, v + 3);
    if constexpr (R == 5) {
      if (v + 4 >= nloc) break;
      step(I4{}, v + 4);
    }
  }
  wait_vm<0>();
  lds_barrier();
  if (wave == kFinWave) {
    // deta of the segment's first chunk
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

template <int D>
hipError_t launch_a(const BwdArgs& a, hipStream_t s) {
  const int64_t groups = (a.B * a.H + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (D / kT) * a.n_seg));
  hipLaunchKernelGGL(bwd_a<D>, grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_bwd_a(const BwdArgs& a, hipStream_t s) {
  return a.d_in == 128 ? launch_a<128>(a, s) : launch_a<64>(a, s);
}

}  // namespace gls
