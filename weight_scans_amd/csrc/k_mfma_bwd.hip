// k_mfma_bwd.hip -- matrix-core reverse scan for bf16 io, d_in = d_out = D in
// {64, 128} (gfx950, v_mfma_f32_16x16x32_bf16), the exact adjoint of the
// forward scan for L = sum_t <dy_t, y_t> ("exact parallel scans for both
// forward evaluation and reverse backpropagation", GradLev abstract,
// omanscience.com).
//
// Chunk-local notation as in the forward (l = inclusive cumsum of log2 alpha,
// lq_i = l_{i-1}, e(.) = 2^(.), Mf_ij = e(lq_i - l_j) for j < i).  Walking the
// chunks backwards, the adjoint Lam (dL/dD after a token) is carried as
//   Lam_in = e(l_last) Lam_out + sum_u e(lq_u) dy_u x_u^T
// and, with P_ui = Mf_ui (x_u . x_i) and Be_ij = Mf_ij (dy_i . g_j)(-eta_j):
//   u_i      = e(l_last - l_i) Lam_out x_i + sum_{u>i} P_ui dy_u
//   dg_i     = -eta_i u_i,            deta_i = -g_i . u_i
//   dx_i     = W0^T dy_i + e(lq_i) D_in^T dy_i + (Be X)_i + (Be^T X)_i
//              - eta_i e(l_last - l_i) Lam_out^T g_i
//   dalpha_i = <Lam_i, D_i> = e(l_last - l_i + lq_i) <Lam_out, D_in>
//              + e(l_last - l_i) sum_{j<i} Mf_ij (-eta_j) x_j.(Lam_out^T g_j)
//              + e(lq_i) sum_{u>i} Mf_ui x_u.(D_in^T dy_u)
//              + (sum_{u>i} x_u.(Be X)_u - sum_{j>=i} x_j.(Be^T X)_j) / alpha_i
//   dW0     += sum_u dy_u x_u^T
// D_in (the adaptation at the chunk start) comes from the forward's saved
// states (bf16, natural [row][col] layout).  LDS tiles are token-major; products
// that contract over tokens or rows use transposing LDS reads, and outputs are
// produced transposed so that every write is 8 or 16 bytes wide.
// The backward needs the adjoint both by rows (u reduces over columns) and by
// columns (dx reduces over rows), so every (b, h) gets two kinds of
// work-group in one launch:
//   role A, row tile R (32 rows): Lam[R, :] -> dg[:, R], deta partial, dW0[R, :]
//   role B, col tile K (32 cols): Lam[:, K], D_in[:, K] -> dx[:, K], dalpha partial
// Per-token partials are summed over the tiles by the finalize kernel in a
// fixed order, so results are bit-reproducible.
#include <algorithm>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kC = 64;    // tokens per chunk
constexpr int kT = 32;    // rows / columns per tile
constexpr int kNT = 256;  // threads (4 waves)
constexpr int NP = kT + 8, CP = kC + 8;

template <int D>
struct alignas(16) SmA {
  static constexpr int XP = D + 8;
  __bf16 X[kC][XP];    // x                          [token][feature]
  __bf16 Dr[kC][NP];   // dy of the row tile         [token][row]
  __bf16 Drs[kC][NP];  // e(lq_u) dy of the row tile [token][row]
  __bf16 Gr[kC][NP];   // g of the row tile          [token][row]
  __bf16 PT[kC][CP];   // PT[i][u] = P_ui (u > i)
  __bf16 L[2][kT][XP]; // Lam_out[R, :] (bf16)       [row][col], double-buffered
};

template <int D>
struct alignas(16) SmB {
  static constexpr int XP = D + 8;
  __bf16 Dy[kC][XP];   // dy                         [token][feature]
  __bf16 G[kC][XP];    // g                          [token][feature]
  __bf16 Xk[kC][NP];   // x of the column tile       [token][col]
  __bf16 Xks[kC][NP];  // e(lq_u) x of the col tile  [token][col]
  __bf16 BeT[kC][CP];  // BeT[j][i] = Be_ij (j < i)
  __bf16 Sn[D][NP];    // D_in[:, K] (bf16)          [row][col]
  __bf16 L[D][NP];     // Lam_out[:, K] (bf16)       [row][col]
};

template <int D>
union alignas(16) BwdSmem {
  SmA<D> a;
  SmB<D> b;
};

struct alignas(16) GateSmem {
  float lq[kC], li[kC], e2[kC], eq[kC], neta[kC], al[kC];
  float sp[kC], sr[kC], sq[kC], sk[kC];
  float red[4];
  float gam, llast, pad_[2];
};

__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

__device__ __forceinline__ float sum_groups(float v) {  // over the 4 lane groups of 16
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ uint4 scale_bf16x8(const uint4& v, float s) {
  uint4 r;
  r.x = pack2(bf16_val(v.x & 0xffffu) * s, bf16_val(v.x >> 16) * s);
  r.y = pack2(bf16_val(v.y & 0xffffu) * s, bf16_val(v.y >> 16) * s);
  r.z = pack2(bf16_val(v.z & 0xffffu) * s, bf16_val(v.z >> 16) * s);
  r.w = pack2(bf16_val(v.w & 0xffffu) * s, bf16_val(v.w >> 16) * s);
  return r;
}

__device__ __forceinline__ uint2 pack4(const f32x4& v) {
  uint2 p;
  p.x = pack2(v[0], v[1]);
  p.y = pack2(v[2], v[3]);
  return p;
}

__device__ __forceinline__ f32x4 unpack4(const uint2& p) {
  f32x4 v;
  v[0] = bf16_val(p.x & 0xffffu);
  v[1] = bf16_val(p.x >> 16);
  v[2] = bf16_val(p.y & 0xffffu);
  v[3] = bf16_val(p.y >> 16);
  return v;
}

// Gates of the staged chunk, every wave (lane = token); wave 0 publishes them.
struct LaneGates {
  float lq, l, llast, eq, e2, neta, al;
};
__device__ __forceinline__ LaneGates lane_gates(float eta, float alpha, int lane, int cv) {
  LaneGates r;
  const float et = lane < cv ? eta : 0.f;
  r.al = lane < cv ? alpha : 1.f;
  const ChunkGates g = chunk_gates(r.al, lane);
  r.lq = g.lq;
  r.l = g.l;
  r.llast = g.llast;
  r.eq = fexp2(g.lq);
  r.e2 = fexp2(g.llast - g.l);
  r.neta = -et;
  return r;
}
__device__ __forceinline__ void publish_gates(GateSmem& gs, const LaneGates& g, int lane) {
  gs.lq[lane] = g.lq;
  gs.li[lane] = g.l;
  gs.e2[lane] = g.e2;
  gs.eq[lane] = g.eq;
  gs.neta[lane] = g.neta;
  gs.al[lane] = g.al;
  if (lane == 0) {
    gs.gam = fexp2(g.llast);
    gs.llast = g.llast;
  }
}

// ----------------------------------------------------------------- role A
template <int D>
__device__ __forceinline__ void role_a(const BwdArgs& a, SmA<D>& sm, GateSmem& gs, int64_t bh,
                                       int tile) {
  constexpr int XP = SmA<D>::XP;
  constexpr int RPT = kC * D / (8 * kNT);
  constexpr int CG = D / 8;
  constexpr int NS = (2 * (D / 16)) / 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int r0 = tile * kT;
  const int64_t T = a.T, BHT = a.B * a.H * T;
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * D;
  const uint16_t* g = static_cast<const uint16_t*>(a.g) + bh * T * D;
  const uint16_t* dy = static_cast<const uint16_t*>(a.dy) + bh * T * D;
  const float* eta = static_cast<const float*>(a.eta) + bh * T;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;
  uint16_t* dg = static_cast<uint16_t*>(a.dg) + bh * T * D;
  float* pe = static_cast<float*>(a.part_eta) + tile * BHT + bh * T;

  for (int idx = tid; idx < kC * CP; idx += kNT) (&sm.PT[0][0])[idx] = static_cast<__bf16>(0.f);
  for (int idx = tid; idx < 2 * kT * XP; idx += kNT) (&sm.L[0][0][0])[idx] = static_cast<__bf16>(0.f);
  f32x4 lam[NS], dw[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    lam[s] = zero4();
    dw[s] = zero4();
  }

  struct {
    uint4 x[RPT];
    uint4 dy, g;
    float eta, alpha;
  } pf;
  const int cg = tid % CG, rg = tid / CG, jg = tid >> 2, c8 = 8 * (tid & 3);
  auto load = [&](int c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = static_cast<int>(std::min<int64_t>(kC, T - t0));
#pragma unroll
    for (int s = 0; s < RPT; ++s) pf.x[s] = load_row16(x + t0 * D + 8 * cg, D, rg * RPT + s, cv);
    pf.dy = load_row16(dy + t0 * D + r0 + c8, D, jg, cv);
    pf.g = load_row16(g + t0 * D + r0 + c8, D, jg, cv);
    const int jt = tid & (kC - 1), jc = jt < cv ? jt : cv - 1;
    pf.eta = eta[t0 + jc];
    pf.alpha = alpha[t0 + jc];
  };

  // Stage the loaded chunk (cv valid tokens) and publish its gates.
  const auto stage = [&](int cv) {
    const LaneGates lg = lane_gates(pf.eta, pf.alpha, lane, cv);
    if (wave == 0) publish_gates(gs, lg, lane);
#pragma unroll
    for (int s = 0; s < RPT; ++s)
      *reinterpret_cast<uint4*>(&sm.X[rg * RPT + s][8 * cg]) = keep_row(pf.x[s], rg * RPT + s, cv);
    const uint4 dv = keep_row(pf.dy, jg, cv);
    *reinterpret_cast<uint4*>(&sm.Dr[jg][c8]) = dv;
    *reinterpret_cast<uint4*>(&sm.Drs[jg][c8]) = scale_bf16x8(dv, __shfl(lg.eq, jg, 64));
    *reinterpret_cast<uint4*>(&sm.Gr[jg][c8]) = keep_row(pf.g, jg, cv);
  };
  const auto cv_of = [&](int c) {
    return static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };

  load(a.n_chunks - 1);
  stage(cv_of(a.n_chunks - 1));
  lds_barrier();
  for (int c = a.n_chunks - 1; c >= 0; --c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = cv_of(c);
    // loads of the previous chunk: issued now, staged at the end of this iteration
    if (c > 0) load(c - 1);

    // P^T[i][u] = e(lq_u - l_i) (x_u . x_i) for u > i
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int b = wave + 4 * s;
      if (b < 10) {
        const int ub = tri_i(b), ib = tri_j(b);
        f32x4 xx = zero4();
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb)
          xx = mfma16x16x32(frag(&sm.X[0][0], XP, ub * 16, kb * 32, lane),
                            frag(&sm.X[0][0], XP, ib * 16, kb * 32, lane), xx);
        const int i = ib * 16 + l16, u0 = ub * 16 + 4 * g4;
        const float li = gs.li[i];
        const f32x4 lqu = *reinterpret_cast<const f32x4*>(&gs.lq[u0]);
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float e = xx[q] * fexp2(lqu[q] - li);
          v[q] = (i < u0 + q) ? e : 0.f;
        }
        *reinterpret_cast<uint2*>(&sm.PT[i][u0]) = pack4(v);
      }
    }
    lds_barrier();  // P visible

    {
      // u^T[r][i] = e(l_last - l_i) (Lam_out x_i)[r] + sum_{u>i} P_ui dy_u[r];
      // dg stored straight from the accumulators (4 rows of one token per lane)
      const int w = wave, i = w * 16 + l16;
      f32x4 ain[2] = {zero4(), zero4()}, apd[2] = {zero4(), zero4()};
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8 xf = frag(&sm.X[0][0], XP, w * 16, kb * 32, lane);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          ain[rb] = mfma16x16x32(frag(&sm.L[c & 1][0][0], XP, rb * 16, kb * 32, lane), xf, ain[rb]);
      }
      for (int kb = w / 2; kb < 2; ++kb) {
        const bf16x8 pf_ = frag(&sm.PT[0][0], CP, w * 16, kb * 32, lane);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          apd[rb] = mfma16x16x32(frag_t(&sm.Dr[0][0], NP, kb * 32, rb * 16, lane), pf_, apd[rb]);
      }
      const float e2 = gs.e2[i], ne = gs.neta[i];
      float dpart = 0.f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const f32x4 u = ain[rb] * e2 + apd[rb];
        if (i < cv) *reinterpret_cast<uint2*>(dg + (t0 + i) * D + r0 + rb * 16 + 4 * g4) = pack4(u * ne);
        const f32x4 gv = unpack4(*reinterpret_cast<const uint2*>(&sm.Gr[i][rb * 16 + 4 * g4]));
        dpart += gv[0] * u[0] + gv[1] * u[1] + gv[2] * u[2] + gv[3] * u[3];
      }
      dpart = sum_groups(dpart);
      if (g4 == 0 && i < cv) pe[t0 + i] = -dpart;
    }

    // Lam^T[c][r] = Gamma Lam^T + sum_u x_u[c] e(lq_u) dy_u[r];  dW0^T += sum_u x_u[c] dy_u[r]
    // (written to the other Lam buffer: the current one may still be read)
    const float gam = gs.gam;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int b = wave + 4 * s, cb = b >> 1, rb = b & 1;
      lam[s] = lam[s] * gam;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 xa = frag_t(&sm.X[0][0], XP, kb * 32, cb * 16, lane);
        lam[s] = mfma16x16x32(xa, frag_t(&sm.Drs[0][0], NP, kb * 32, rb * 16, lane), lam[s]);
        dw[s] = mfma16x16x32(xa, frag_t(&sm.Dr[0][0], NP, kb * 32, rb * 16, lane), dw[s]);
      }
      *reinterpret_cast<uint2*>(&sm.L[(c & 1) ^ 1][rb * 16 + l16][cb * 16 + 4 * g4]) = pack4(lam[s]);
    }
    lds_barrier();  // every read of this chunk's tiles is done
    if (c > 0) {
      stage(cv_of(c - 1));
      lds_barrier();
    }
  }

  float* pw = static_cast<float*>(a.part_dW0) + bh * D * D;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int b = wave + 4 * s, cb = b >> 1, rb = b & 1;
    *reinterpret_cast<f32x4*>(pw + (r0 + rb * 16 + l16) * D + cb * 16 + 4 * g4) = dw[s];
  }
}

// ----------------------------------------------------------------- role B
template <int D>
__device__ __forceinline__ void role_b(const BwdArgs& a, SmB<D>& sm, GateSmem& gs, int64_t bh,
                                       int tile) {
  constexpr int XP = SmB<D>::XP;
  constexpr int RPT = kC * D / (8 * kNT);
  constexpr int CG = D / 8;
  constexpr int SPT = D * kT / (8 * kNT);  // 16-byte state pieces per thread
  constexpr int NS = (2 * (D / 16)) / 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int k0 = tile * kT;
  const int h = static_cast<int>(bh % a.H);
  const int64_t T = a.T, BHT = a.B * a.H * T;
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * D;
  const uint16_t* g = static_cast<const uint16_t*>(a.g) + bh * T * D;
  const uint16_t* dy = static_cast<const uint16_t*>(a.dy) + bh * T * D;
  const float* eta = static_cast<const float*>(a.eta) + bh * T;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * D * D;
  const uint16_t* st = static_cast<const uint16_t*>(a.states) + bh * a.n_chunks * D * D;
  uint16_t* dx = static_cast<uint16_t*>(a.dx) + bh * T * D;
  float* pa = static_cast<float*>(a.part_alpha) + tile * BHT + bh * T;

  // W0[:, K] fragments as the A operand of W0[:,K]^T dy^T (constant): via Sn
#pragma unroll
  for (int s = 0; s < SPT; ++s) {
    const int idx = tid + kNT * s, r = idx >> 2, cc = 8 * (idx & 3);
    *reinterpret_cast<uint4*>(&sm.Sn[r][cc]) =
        *reinterpret_cast<const uint4*>(W0 + static_cast<int64_t>(r) * D + k0 + cc);
  }
  for (int idx = tid; idx < kC * CP; idx += kNT) (&sm.BeT[0][0])[idx] = static_cast<__bf16>(0.f);
  for (int idx = tid; idx < D * NP; idx += kNT) (&sm.L[0][0])[idx] = static_cast<__bf16>(0.f);
  lds_barrier();
  bf16x8 w0f[D / 32][2];
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) w0f[kb][cb] = frag_t(&sm.Sn[0][0], NP, kb * 32, cb * 16, lane);
  lds_barrier();

  f32x4 lam[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) lam[s] = zero4();

  struct {
    uint4 dy[RPT], g[RPT];
    uint4 x;
    uint4 sn[SPT];
    float eta, alpha;
  } pf;
  const int cg = tid % CG, rg = tid / CG, jg = tid >> 2, c8 = 8 * (tid & 3);
  auto load = [&](int c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = static_cast<int>(std::min<int64_t>(kC, T - t0));
#pragma unroll
    for (int s = 0; s < RPT; ++s) {
      pf.dy[s] = load_row16(dy + t0 * D + 8 * cg, D, rg * RPT + s, cv);
      pf.g[s] = load_row16(g + t0 * D + 8 * cg, D, rg * RPT + s, cv);
    }
    pf.x = load_row16(x + t0 * D + k0 + c8, D, jg, cv);
    const uint16_t* sc = st + static_cast<int64_t>(c) * D * D + k0;
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int idx = tid + kNT * s;
      pf.sn[s] = *reinterpret_cast<const uint4*>(sc + (idx >> 2) * D + 8 * (idx & 3));
    }
    const int jt = tid & (kC - 1), jc = jt < cv ? jt : cv - 1;
    pf.eta = eta[t0 + jc];
    pf.alpha = alpha[t0 + jc];
  };

  // Stage the loaded chunk and publish its gates; returns the lane gates
  // (lane = token) of the staged chunk.
  const auto stage = [&](int cv) {
    const LaneGates lg = lane_gates(pf.eta, pf.alpha, lane, cv);
    if (wave == 0) publish_gates(gs, lg, lane);
#pragma unroll
    for (int s = 0; s < RPT; ++s) {
      *reinterpret_cast<uint4*>(&sm.Dy[rg * RPT + s][8 * cg]) = keep_row(pf.dy[s], rg * RPT + s, cv);
      *reinterpret_cast<uint4*>(&sm.G[rg * RPT + s][8 * cg]) = keep_row(pf.g[s], rg * RPT + s, cv);
    }
    const uint4 xv = keep_row(pf.x, jg, cv);
    *reinterpret_cast<uint4*>(&sm.Xk[jg][c8]) = xv;
    *reinterpret_cast<uint4*>(&sm.Xks[jg][c8]) = scale_bf16x8(xv, __shfl(lg.eq, jg, 64));
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int idx = tid + kNT * s;
      *reinterpret_cast<uint4*>(&sm.Sn[idx >> 2][8 * (idx & 3)]) = pf.sn[s];
    }
    return lg;
  };
  const auto cv_of = [&](int c) {
    return static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };

  load(a.n_chunks - 1);
  LaneGates lg = stage(cv_of(a.n_chunks - 1));
  lds_barrier();
  for (int c = a.n_chunks - 1; c >= 0; --c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = cv_of(c);
    // loads of the previous chunk: issued now, staged at the end of this iteration
    if (c > 0) load(c - 1);

    // Be_ij = e(lq_i - l_j)(-eta_j)(dy_i . g_j), j < i, stored as BeT[j][i]
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int b = wave + 4 * s;
      if (b < 10) {
        const int ib = tri_i(b), jb = tri_j(b);
        f32x4 d = zero4();
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb)
          d = mfma16x16x32(frag(&sm.Dy[0][0], XP, ib * 16, kb * 32, lane),
                           frag(&sm.G[0][0], XP, jb * 16, kb * 32, lane), d);
        const int j = jb * 16 + l16, i0 = ib * 16 + 4 * g4;
        const float lj = gs.li[j], nj = gs.neta[j];
        const f32x4 lqi = *reinterpret_cast<const f32x4*>(&gs.lq[i0]);
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float e = d[q] * fexp2(lqi[q] - lj) * nj;
          v[q] = (j < i0 + q) ? e : 0.f;
        }
        *reinterpret_cast<uint2*>(&sm.BeT[j][i0]) = pack4(v);
      }
    }
    {
      // <Lam_out, D_in> over this tile's columns
      float p = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int b = wave + 4 * s, cb = b & 1, rb = b >> 1;
        const f32x4 sv = unpack4(*reinterpret_cast<const uint2*>(&sm.Sn[rb * 16 + l16][cb * 16 + 4 * g4]));
        p += lam[s][0] * sv[0] + lam[s][1] * sv[1] + lam[s][2] * sv[2] + lam[s][3] * sv[3];
      }
      p = sum_groups(sum16(p));
      if (lane == 0) gs.red[wave] = p;
    }
    lds_barrier();  // Be visible

    {
      // dx^T[c][i] for this wave's token block, both column blocks; stored
      // straight from the accumulators (4 columns of one token per lane)
      const int w = wave, i = w * 16 + l16;
      f32x4 aws[2] = {zero4(), zero4()}, as_[2] = {zero4(), zero4()}, al[2] = {zero4(), zero4()};
      f32x4 aq[2] = {zero4(), zero4()}, ak[2] = {zero4(), zero4()};
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8 df = frag(&sm.Dy[0][0], XP, w * 16, kb * 32, lane);
        const bf16x8 gf = frag(&sm.G[0][0], XP, w * 16, kb * 32, lane);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          aws[cb] = mfma16x16x32(w0f[kb][cb], df, aws[cb]);
          as_[cb] = mfma16x16x32(frag_t(&sm.Sn[0][0], NP, kb * 32, cb * 16, lane), df, as_[cb]);
          al[cb] = mfma16x16x32(frag_t(&sm.L[0][0], NP, kb * 32, cb * 16, lane), gf, al[cb]);
        }
      }
      for (int kb = 0; kb < (w + 2) / 2; ++kb) {
        const bf16x8 bf = frag_t(&sm.BeT[0][0], CP, kb * 32, w * 16, lane);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          aq[cb] = mfma16x16x32(frag_t(&sm.Xk[0][0], NP, kb * 32, cb * 16, lane), bf, aq[cb]);
      }
      for (int kb = w / 2; kb < 2; ++kb) {
        const bf16x8 bt = frag(&sm.BeT[0][0], CP, w * 16, kb * 32, lane);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          ak[cb] = mfma16x16x32(frag_t(&sm.Xk[0][0], NP, kb * 32, cb * 16, lane), bt, ak[cb]);
      }
      const float eqi = gs.eq[i], fl = gs.neta[i] * gs.e2[i];
      float pp = 0.f, rr = 0.f, qq = 0.f, kk = 0.f;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const f32x4 v = aws[cb] + as_[cb] * eqi + aq[cb] + ak[cb] + al[cb] * fl;
        if (i < cv)
          *reinterpret_cast<uint2*>(dx + (t0 + i) * D + k0 + cb * 16 + 4 * g4) = pack4(v);
        const f32x4 xv = unpack4(*reinterpret_cast<const uint2*>(&sm.Xk[i][cb * 16 + 4 * g4]));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          pp += xv[q] * al[cb][q];
          rr += xv[q] * as_[cb][q];
          qq += xv[q] * aq[cb][q];
          kk += xv[q] * ak[cb][q];
        }
      }
      pp = sum_groups(pp);
      rr = sum_groups(rr);
      qq = sum_groups(qq);
      kk = sum_groups(kk);
      if (g4 == 0) {
        gs.sp[i] = pp;
        gs.sr[i] = rr;
        gs.sq[i] = qq;
        gs.sk[i] = kk;
      }
    }
    lds_barrier();  // per-token dots visible; reads of L, Sn, BeT done

    if (wave == 0) {
      // dalpha partial, lane = token i.  With the decay Mf_ij = prod_{j<r<i} alpha_r:
      //   s2_i = sum_{j<i} Mf_ij (-eta_j) p_j      forward affine scan
      //   s3_i = sum_{u>i} Mf_ui r_u               same scan over reversed lanes
      //   s4_i = sum_{u>i} q_u - sum_{j>=i} k_j    suffix sums
      const int i = lane;
      float a2 = lg.al, b2 = lg.neta * gs.sp[i];
      wave_scan_affine(a2, b2);
      const float s2 = wave_shift_up(b2, 0.f);
      float a3 = wave_reverse(lg.al, lane), b3 = wave_reverse(gs.sr[i], lane);
      wave_scan_affine(a3, b3);
      const float s3 = wave_reverse(wave_shift_up(b3, 0.f), lane);
      const float qsuf = wave_reverse(wave_shift_up(wave_scan_add(wave_reverse(gs.sq[i], lane)), 0.f), lane);
      const float ksuf = wave_reverse(wave_scan_add(wave_reverse(gs.sk[i], lane)), lane);
      const float c0 = gs.red[0] + gs.red[1] + gs.red[2] + gs.red[3];
      const float ll = lg.llast, lii = lg.l, lqi = lg.lq;
      if (i < cv)
        pa[t0 + i] = fexp2(ll - lii + lqi) * c0 + fexp2(ll - lii) * s2 + fexp2(lqi) * s3 +
                     (qsuf - ksuf) / lg.al;
    }
    // Lam^T[c][r] = Gamma Lam^T + sum_u e(lq_u) x_u[c] dy_u[r]   (c in K)
    const float gam = gs.gam;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int b = wave + 4 * s, cb = b & 1, rb = b >> 1;
      lam[s] = lam[s] * gam;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        lam[s] = mfma16x16x32(frag_t(&sm.Xks[0][0], NP, kb * 32, cb * 16, lane),
                              frag_t(&sm.Dy[0][0], XP, kb * 32, rb * 16, lane), lam[s]);
      *reinterpret_cast<uint2*>(&sm.L[rb * 16 + l16][cb * 16 + 4 * g4]) = pack4(lam[s]);
    }
    lds_barrier();  // every read of this chunk's tiles is done
    if (c > 0) {
      lg = stage(cv_of(c - 1));
      lds_barrier();
    }
  }
}

template <int D>
__global__ __launch_bounds__(kNT) void bwd_mfma(BwdArgs a) {
  static_assert(D == 64 || D == 128, "D");
  constexpr int NT = D / kT;
  __shared__ BwdSmem<D> sm;
  __shared__ GateSmem gs;
  const int grp = blockIdx.x / (16 * NT), within = blockIdx.x % (16 * NT);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  const int sub = within >> 3;
  if (bh >= a.B * a.H) return;
  if (sub < NT)
    role_a<D>(a, sm.a, gs, bh, sub);
  else
    role_b<D>(a, sm.b, gs, bh, sub - NT);
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t s) {
  const int64_t groups = (a.B * a.H + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 16 * (D / kT)));
  hipLaunchKernelGGL(bwd_mfma<D>, grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int mfma_bwd_tiles(int d) { return d / kT; }

hipError_t launch_mfma_bwd(const BwdArgs& a, hipStream_t s) {
  return a.d_in == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace gls
