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
// states.  The backward needs the adjoint both by rows (u reduces over
// columns) and by columns (dx reduces over rows), so every (b, h) gets two
// kinds of work-group in one launch:
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

template <int D>
struct SmA {
  static constexpr int XP = D + 8, TP = kC + 8, RP = kT + 8;
  __bf16 X[kC][XP];   // x                       [token][feature]
  __bf16 Xt[D][TP];   // x^T                     [feature][token]
  __bf16 Dt[kT][TP];  // dy of the row tile, ^T  [row][token]
  __bf16 PT[kC][TP];  // PT[i][u] = P_ui (u > i)
  __bf16 L[kT][XP];   // Lam_out[R, :] (bf16)    [row][col]
  __bf16 Gr[kC][RP];  // g of the row tile       [token][row]
  __bf16 DGs[kC][RP]; // dg staging              [token][row]
};

template <int D>
struct SmB {
  static constexpr int XP = D + 8, TP = kC + 8;
  __bf16 Dy[kC][XP];  // dy                      [token][feature]
  __bf16 G[kC][XP];   // g                       [token][feature]
  __bf16 Xt[kT][TP];  // x of the col tile, ^T   [col][token]
  __bf16 Be[kC][TP];  // Be[i][j]
  __bf16 BeT[kC][TP]; // BeT[j][i] = Be[i][j]
  __bf16 Sn[kT][XP];  // D_in[:, K]^T (bf16)     [col][row]
  __bf16 L[kT][XP];   // Lam_out[:, K]^T (bf16)  [col][row]
};

template <int D>
union BwdSmem {
  SmA<D> a;
  SmB<D> b;
};

struct GateSmem {
  float lq[kC], li[kC], eq[kC], e2[kC], neta[kC], al[kC];
  float eta_raw[kC], alpha_raw[kC];
  float sp[kC], sr[kC], sq[kC], sk[kC];
  float red[4];
  float gam, llast;
};

__constant__ int kBlkI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kBlkJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

__device__ __forceinline__ void gates_to_smem(GateSmem& gs, int lane) {
  const float et = gs.eta_raw[lane], al = gs.alpha_raw[lane];
  const ChunkGates cg = chunk_gates(al, lane);
  gs.lq[lane] = cg.lq;
  gs.li[lane] = cg.l;
  gs.eq[lane] = exp2f(cg.lq);
  gs.e2[lane] = exp2f(cg.llast - cg.l);
  gs.neta[lane] = -et;
  gs.al[lane] = al;
  if (lane == 0) {
    gs.gam = exp2f(cg.llast);
    gs.llast = cg.llast;
  }
}

__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

// ----------------------------------------------------------------- role A
template <int D>
__device__ __forceinline__ void role_a(const BwdArgs& a, SmA<D>& sm, GateSmem& gs, int64_t bh,
                                       int tile) {
  constexpr int XP = SmA<D>::XP, TP = SmA<D>::TP;
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

  for (int idx = tid; idx < kC * TP; idx += kNT) (&sm.PT[0][0])[idx] = static_cast<__bf16>(0.f);
  for (int idx = tid; idx < kT * XP; idx += kNT) (&sm.L[0][0])[idx] = static_cast<__bf16>(0.f);
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
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < RPT; ++s) {
      const int j = rg * RPT + s;
      pf.x[s] = (j < cv) ? *reinterpret_cast<const uint4*>(x + (t0 + j) * D + 8 * cg) : z;
    }
    pf.dy = (jg < cv) ? *reinterpret_cast<const uint4*>(dy + (t0 + jg) * D + r0 + c8) : z;
    pf.g = (jg < cv) ? *reinterpret_cast<const uint4*>(g + (t0 + jg) * D + r0 + c8) : z;
    if (tid < kC) {
      pf.eta = (tid < cv) ? eta[t0 + tid] : 0.f;
      pf.alpha = (tid < cv) ? alpha[t0 + tid] : 1.f;
    }
  };

  load(a.n_chunks - 1);
  for (int c = a.n_chunks - 1; c >= 0; --c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = static_cast<int>(std::min<int64_t>(kC, T - t0));
    // ---- stage the chunk
#pragma unroll
    for (int s = 0; s < RPT; ++s) *reinterpret_cast<uint4*>(&sm.X[rg * RPT + s][8 * cg]) = pf.x[s];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(&sm.Xt[8 * cg + q][rg * RPT]);
      if constexpr (RPT == 4) {
        uint2 v;
        v.x = half_of(pf.x[0], q) | (half_of(pf.x[1], q) << 16);
        v.y = half_of(pf.x[2], q) | (half_of(pf.x[3], q) << 16);
        *reinterpret_cast<uint2*>(dst) = v;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = half_of(pf.x[0], q) | (half_of(pf.x[1], q) << 16);
      }
      reinterpret_cast<uint16_t*>(&sm.Dt[c8 + q][0])[jg] = static_cast<uint16_t>(half_of(pf.dy, q));
    }
    *reinterpret_cast<uint4*>(&sm.Gr[jg][c8]) = pf.g;
    if (tid < kC) {
      gs.eta_raw[tid] = pf.eta;
      gs.alpha_raw[tid] = pf.alpha;
    }
    lds_barrier();  // S1
    if (c > 0) load(c - 1);
    if (wave == 0) gates_to_smem(gs, lane);

    // x_u . x_i for u-block >= i-block
    f32x4 xx[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int b = wave + 4 * s;
      xx[s] = zero4();
      if (b < 10) {
        const int ub = kBlkI[b], ib = kBlkJ[b];
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb)
          xx[s] = mfma16x16x32(frag(&sm.X[0][0], XP, ub * 16, kb * 32, lane),
                               frag(&sm.X[0][0], XP, ib * 16, kb * 32, lane), xx[s]);
      }
    }
    lds_barrier();  // S2: gates visible

#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int b = wave + 4 * s;
      if (b < 10) {
        const int ub = kBlkI[b], ib = kBlkJ[b];
        const int i = ib * 16 + l16, u0 = ub * 16 + 4 * g4;
        const float li = gs.li[i];
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (i < u0 + q) ? xx[s][q] * exp2f(gs.lq[u0 + q] - li) : 0.f;
        uint2 pk;
        pk.x = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
        pk.y = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
        *reinterpret_cast<uint2*>(&sm.PT[i][u0]) = pk;
      }
    }
    lds_barrier();  // S3: P visible

    {
      const int ib = wave;
      f32x4 ain[2] = {zero4(), zero4()}, apd[2] = {zero4(), zero4()};
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8 xf = frag(&sm.X[0][0], XP, ib * 16, kb * 32, lane);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          ain[nb] = mfma16x16x32(xf, frag(&sm.L[0][0], XP, nb * 16, kb * 32, lane), ain[nb]);
      }
      for (int kb = ib / 2; kb < 2; ++kb) {
        const bf16x8 pf_ = frag(&sm.PT[0][0], TP, ib * 16, kb * 32, lane);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          apd[nb] = mfma16x16x32(pf_, frag(&sm.Dt[0][0], TP, nb * 16, kb * 32, lane), apd[nb]);
      }
      float dpart[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = ib * 16 + 4 * g4 + q, r = nb * 16 + l16;
          const float u = gs.e2[i] * ain[nb][q] + apd[nb][q];
          sm.DGs[i][r] = static_cast<__bf16>(gs.neta[i] * u);
          dpart[q] += static_cast<float>(sm.Gr[i][r]) * u;
        }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s = sum16(dpart[q]);
        const int i = ib * 16 + 4 * g4 + q;
        if (l16 == 0 && i < cv) pe[t0 + i] = -s;
      }
    }
    lds_barrier();  // S4: dg staged; reads of L done

    {
      const int i = tid >> 2, cc = 8 * (tid & 3);
      if (i < cv)
        *reinterpret_cast<uint4*>(dg + (t0 + i) * D + r0 + cc) =
            *reinterpret_cast<const uint4*>(&sm.DGs[i][cc]);
    }
    const float gam = gs.gam;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int b = wave + 4 * s, rb = b / (D / 16), cb = b % (D / 16);
      lam[s] = lam[s] * gam;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 dr = frag(&sm.Dt[0][0], TP, rb * 16, kb * 32, lane);
        bf16x8 ds;
        const int u0 = kb * 32 + 8 * g4;
#pragma unroll
        for (int e = 0; e < 8; ++e) ds[e] = static_cast<__bf16>(static_cast<float>(dr[e]) * gs.eq[u0 + e]);
        const bf16x8 xb = frag(&sm.Xt[0][0], TP, cb * 16, kb * 32, lane);
        lam[s] = mfma16x16x32(ds, xb, lam[s]);
        dw[s] = mfma16x16x32(dr, xb, dw[s]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sm.L[rb * 16 + 4 * g4 + q][cb * 16 + l16] = static_cast<__bf16>(lam[s][q]);
    }
    lds_barrier();  // S5
  }

  float* pw = static_cast<float*>(a.part_dW0) + bh * D * D;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int b = wave + 4 * s, rb = b / (D / 16), cb = b % (D / 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) pw[(r0 + rb * 16 + 4 * g4 + q) * D + cb * 16 + l16] = dw[s][q];
  }
}

// ----------------------------------------------------------------- role B
template <int D>
__device__ __forceinline__ void role_b(const BwdArgs& a, SmB<D>& sm, GateSmem& gs, int64_t bh,
                                       int tile) {
  constexpr int XP = SmB<D>::XP, TP = SmB<D>::TP;
  constexpr int RPT = kC * D / (8 * kNT);
  constexpr int CG = D / 8;
  constexpr int SPT = kT * D / (8 * kNT);  // state rows per thread (16-byte units)
  constexpr int NS = ((D / 16) * 2) / 4;
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

  // W0[:, K]^T fragments (constant): stage through Sn once
  for (int idx = tid; idx < D * 4; idx += kNT) {
    const int r = idx >> 2, cc = 8 * (idx & 3);
    const uint4 v = *reinterpret_cast<const uint4*>(W0 + static_cast<int64_t>(r) * D + k0 + cc);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      reinterpret_cast<uint16_t*>(&sm.Sn[cc + q][0])[r] = static_cast<uint16_t>(half_of(v, q));
  }
  for (int idx = tid; idx < kC * TP; idx += kNT) {
    (&sm.Be[0][0])[idx] = static_cast<__bf16>(0.f);
    (&sm.BeT[0][0])[idx] = static_cast<__bf16>(0.f);
  }
  for (int idx = tid; idx < kT * XP; idx += kNT) (&sm.L[0][0])[idx] = static_cast<__bf16>(0.f);
  lds_barrier();
  bf16x8 w0f[D / 32][2];
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) w0f[kb][nb] = frag(&sm.Sn[0][0], XP, nb * 16, kb * 32, lane);
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
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < RPT; ++s) {
      const int j = rg * RPT + s;
      pf.dy[s] = (j < cv) ? *reinterpret_cast<const uint4*>(dy + (t0 + j) * D + 8 * cg) : z;
      pf.g[s] = (j < cv) ? *reinterpret_cast<const uint4*>(g + (t0 + j) * D + 8 * cg) : z;
    }
    pf.x = (jg < cv) ? *reinterpret_cast<const uint4*>(x + (t0 + jg) * D + k0 + c8) : z;
    const uint16_t* sc = st + (static_cast<int64_t>(c) * D + k0) * D;
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int idx = tid + kNT * s;
      pf.sn[s] = *reinterpret_cast<const uint4*>(sc + (idx / CG) * D + 8 * (idx % CG));
    }
    if (tid < kC) {
      pf.eta = (tid < cv) ? eta[t0 + tid] : 0.f;
      pf.alpha = (tid < cv) ? alpha[t0 + tid] : 1.f;
    }
  };

  load(a.n_chunks - 1);
  for (int c = a.n_chunks - 1; c >= 0; --c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = static_cast<int>(std::min<int64_t>(kC, T - t0));
    // ---- stage the chunk
#pragma unroll
    for (int s = 0; s < RPT; ++s) {
      *reinterpret_cast<uint4*>(&sm.Dy[rg * RPT + s][8 * cg]) = pf.dy[s];
      *reinterpret_cast<uint4*>(&sm.G[rg * RPT + s][8 * cg]) = pf.g[s];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      reinterpret_cast<uint16_t*>(&sm.Xt[c8 + q][0])[jg] = static_cast<uint16_t>(half_of(pf.x, q));
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int idx = tid + kNT * s;
      *reinterpret_cast<uint4*>(&sm.Sn[idx / CG][8 * (idx % CG)]) = pf.sn[s];
    }
    if (tid < kC) {
      gs.eta_raw[tid] = pf.eta;
      gs.alpha_raw[tid] = pf.alpha;
    }
    lds_barrier();  // S1
    if (c > 0) load(c - 1);
    if (wave == 0) gates_to_smem(gs, lane);

    // dy_i . g_j for i-block >= j-block
    f32x4 dgx[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int b = wave + 4 * s;
      dgx[s] = zero4();
      if (b < 10) {
        const int ib = kBlkI[b], jb = kBlkJ[b];
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb)
          dgx[s] = mfma16x16x32(frag(&sm.Dy[0][0], XP, ib * 16, kb * 32, lane),
                                frag(&sm.G[0][0], XP, jb * 16, kb * 32, lane), dgx[s]);
      }
    }
    // <Lam_out, D_in> over this tile's columns
    {
      float p = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int b = wave + 4 * s, rb = b >> 1, cb = b & 1;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          p += lam[s][q] * static_cast<float>(sm.Sn[cb * 16 + l16][rb * 16 + 4 * g4 + q]);
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) p += __shfl_xor(p, off, 64);
      if (lane == 0) gs.red[wave] = p;
    }
    lds_barrier();  // S2: gates visible

#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int b = wave + 4 * s;
      if (b < 10) {
        const int ib = kBlkI[b], jb = kBlkJ[b];
        const int j = jb * 16 + l16, i0 = ib * 16 + 4 * g4;
        const float lj = gs.li[j], nj = gs.neta[j];
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = (j < i0 + q) ? dgx[s][q] * exp2f(gs.lq[i0 + q] - lj) * nj : 0.f;
          sm.Be[i0 + q][j] = static_cast<__bf16>(v[q]);
        }
        uint2 pk;
        pk.x = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
        pk.y = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
        *reinterpret_cast<uint2*>(&sm.BeT[j][i0]) = pk;
      }
    }
    lds_barrier();  // S3: Be visible

    {
      const int w = wave;
      f32x4 aws[2] = {zero4(), zero4()}, as_[2] = {zero4(), zero4()}, al[2] = {zero4(), zero4()};
      f32x4 aq[2] = {zero4(), zero4()}, ak[2] = {zero4(), zero4()};
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8 df = frag(&sm.Dy[0][0], XP, w * 16, kb * 32, lane);
        const bf16x8 gf = frag(&sm.G[0][0], XP, w * 16, kb * 32, lane);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          aws[nb] = mfma16x16x32(df, w0f[kb][nb], aws[nb]);
          as_[nb] = mfma16x16x32(df, frag(&sm.Sn[0][0], XP, nb * 16, kb * 32, lane), as_[nb]);
          al[nb] = mfma16x16x32(gf, frag(&sm.L[0][0], XP, nb * 16, kb * 32, lane), al[nb]);
        }
      }
      for (int kb = 0; kb < (w + 2) / 2; ++kb) {
        const bf16x8 bf = frag(&sm.Be[0][0], TP, w * 16, kb * 32, lane);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          aq[nb] = mfma16x16x32(bf, frag(&sm.Xt[0][0], TP, nb * 16, kb * 32, lane), aq[nb]);
      }
      for (int kb = w / 2; kb < 2; ++kb) {
        const bf16x8 bt = frag(&sm.BeT[0][0], TP, w * 16, kb * 32, lane);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          ak[nb] = mfma16x16x32(bt, frag(&sm.Xt[0][0], TP, nb * 16, kb * 32, lane), ak[nb]);
      }
      float pp[4] = {0.f, 0.f, 0.f, 0.f}, rr[4] = {0.f, 0.f, 0.f, 0.f};
      float qq[4] = {0.f, 0.f, 0.f, 0.f}, kk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int cc = nb * 16 + l16;
        const uint2 xr = *reinterpret_cast<const uint2*>(&sm.Xt[cc][w * 16 + 4 * g4]);
        const float xv[4] = {bf16_val(xr.x & 0xffffu), bf16_val(xr.x >> 16),
                             bf16_val(xr.y & 0xffffu), bf16_val(xr.y >> 16)};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = w * 16 + 4 * g4 + q;
          const float v = aws[nb][q] + gs.eq[i] * as_[nb][q] + aq[nb][q] + ak[nb][q] +
                          gs.neta[i] * gs.e2[i] * al[nb][q];
          if (i < cv) dx[(t0 + i) * D + k0 + cc] = static_cast<uint16_t>(bf16_bits(v));
          pp[q] += xv[q] * al[nb][q];
          rr[q] += xv[q] * as_[nb][q];
          qq[q] += xv[q] * aq[nb][q];
          kk[q] += xv[q] * ak[nb][q];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float p = sum16(pp[q]), r = sum16(rr[q]), qv = sum16(qq[q]), kv = sum16(kk[q]);
        if (l16 == 0) {
          const int i = w * 16 + 4 * g4 + q;
          gs.sp[i] = p;
          gs.sr[i] = r;
          gs.sq[i] = qv;
          gs.sk[i] = kv;
        }
      }
    }
    lds_barrier();  // S4: per-token dots visible; reads of L, Sn, Xt-for-dx done

    {
      // dalpha partial, tokens of this wave's block; lane = (token, quarter of the chunk)
      const int i = wave * 16 + l16, qd = g4;
      const float lqi = gs.lq[i], lii = gs.li[i];
      float s2 = 0.f, s3 = 0.f, s4 = 0.f;
#pragma unroll 4
      for (int e = 0; e < 16; ++e) {
        const int j = qd * 16 + e;
        if (j < i) s2 += exp2f(lqi - gs.li[j]) * gs.neta[j] * gs.sp[j];
        if (j > i) {
          s3 += exp2f(gs.lq[j] - lii) * gs.sr[j];
          s4 += gs.sq[j];
        }
        if (j >= i) s4 -= gs.sk[j];
      }
      s2 += __shfl_xor(s2, 16, 64);
      s2 += __shfl_xor(s2, 32, 64);
      s3 += __shfl_xor(s3, 16, 64);
      s3 += __shfl_xor(s3, 32, 64);
      s4 += __shfl_xor(s4, 16, 64);
      s4 += __shfl_xor(s4, 32, 64);
      if (qd == 0 && i < cv) {
        const float c0 = gs.red[0] + gs.red[1] + gs.red[2] + gs.red[3];
        const float ll = gs.llast;
        const float t1 = exp2f(ll - lii + lqi) * c0;
        const float t2 = exp2f(ll - lii) * s2;
        const float t3 = exp2f(lqi) * s3;
        const float t4 = s4 / gs.al[i];
        pa[t0 + i] = t1 + t2 + t3 + t4;
      }
    }
    // adjoint columns: Lam[:, K] = Gamma Lam + sum_u e(lq_u) dy_u x_u[K]^T
    const float gam = gs.gam;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int b = wave + 4 * s, rb = b >> 1, cb = b & 1;
      lam[s] = lam[s] * gam;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 av;
        const int u0 = kb * 32 + 8 * g4;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          av[e] = static_cast<__bf16>(static_cast<float>(sm.Dy[u0 + e][rb * 16 + l16]) * gs.eq[u0 + e]);
        lam[s] = mfma16x16x32(av, frag(&sm.Xt[0][0], TP, cb * 16, kb * 32, lane), lam[s]);
      }
      uint2 pk;
      pk.x = bf16_bits(lam[s][0]) | (bf16_bits(lam[s][1]) << 16);
      pk.y = bf16_bits(lam[s][2]) | (bf16_bits(lam[s][3]) << 16);
      *reinterpret_cast<uint2*>(&sm.L[cb * 16 + l16][rb * 16 + 4 * g4]) = pk;
    }
    lds_barrier();  // S5
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
