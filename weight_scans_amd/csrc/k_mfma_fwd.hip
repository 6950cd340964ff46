// k_mfma_fwd.hip -- matrix-core forward scan for bf16 io, d_in = d_out = D
// in {64, 128} (gfx950, wave64, v_mfma_f32_16x16x32_bf16).
//
// One work-group = one sequence-head (b, h) x one tile of kTN = 32 rows of
// the adaptation D_t (rows are independent chains because y reduces over
// columns only).  The tile's fp32 state lives in MFMA accumulators for the
// whole sequence; chunks of kC = 64 tokens are streamed through LDS with a
// one-chunk register prefetch.  Per chunk (l = chunk-local inclusive cumsum
// of log2 alpha, e(.) = 2^(.)):
//   A_ij  = (x_i . x_j) e(l_{i-1} - l_j) (-eta_j)      j < i  (else 0)
//   y_i   = W0 x_i + e(l_{i-1}) D_in x_i + sum_j A_ij g_j
//   D_out = e(l_last) D_in + sum_j e(l_last - l_j)(-eta_j) g_j x_j^T
// i.e. the discounted sum of rank-one updates of "Parallelize the Training,
// Keep the Learning Serial" (cognaptus.com, section "Once the gradient signals
// are known, the weight trajectory becomes parallelizable") composed as an
// affine scan across chunks.  Every exponent is <= 0.
//
// `states` (optional) receives D_in of every chunk, transposed and rounded to
// bf16: [B*H][n_chunks][D (column c)][D (row r)] -- the layout the matrix-core
// backward reads as an MFMA operand.
#include <algorithm>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kC = 64;    // tokens per chunk
constexpr int kTN = 32;   // rows of the adaptation per work-group
constexpr int kNT = 256;  // threads (4 waves)

template <int D>
struct FwdSmem {
  static constexpr int XP = D + 8;   // row stride of token-major tiles (elements)
  static constexpr int TP = kC + 8;  // row stride of token-contiguous tiles
  __bf16 X[kC][XP];                  // x of the chunk          [token][feature]
  __bf16 Xt[D][TP];                  // x transposed            [feature][token]
  __bf16 Gt[kTN][TP];                // g of the tile, transposed [row][token]
  __bf16 A[kC][TP];                  // masked, decayed scores  [i][j]
  __bf16 S[kTN][XP];                 // D_in of the tile (bf16) [row][col]
  __bf16 W[kTN][XP];                 // W0 of the tile          [row][col]
  __bf16 Y[kC][kTN + 8];             // y staging               [token][row]
  float lq[kC], li[kC], eq[kC], bk[kC], neta[kC];
  float eta_raw[kC], alpha_raw[kC];
  float gam;
};

template <int D>
struct Prefetch {
  static constexpr int RPT = kC * D / (8 * kNT);  // x rows per thread (4 or 2)
  uint4 x[RPT];
  uint4 g;
  float eta, alpha;
};

template <int D>
__device__ __forceinline__ void load_chunk(Prefetch<D>& p, const uint16_t* x, const uint16_t* g,
                                           const float* eta, const float* alpha, int64_t t0,
                                           int cv, int r0, int tid) {
  constexpr int CG = D / 8;
  const int cg = tid % CG, rg = tid / CG;
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int s = 0; s < Prefetch<D>::RPT; ++s) {
    const int j = rg * Prefetch<D>::RPT + s;
    p.x[s] = (j < cv) ? *reinterpret_cast<const uint4*>(x + (t0 + j) * D + 8 * cg) : z;
  }
  const int jg = tid >> 2;
  p.g = (jg < cv) ? *reinterpret_cast<const uint4*>(g + (t0 + jg) * D + r0 + 8 * (tid & 3)) : z;
  if (tid < kC) {
    p.eta = (tid < cv) ? eta[t0 + tid] : 0.f;
    p.alpha = (tid < cv) ? alpha[t0 + tid] : 1.f;
  }
}

template <int D>
__device__ __forceinline__ void stage_chunk(FwdSmem<D>& sm, const Prefetch<D>& p, int tid) {
  constexpr int CG = D / 8, RPT = Prefetch<D>::RPT;
  const int cg = tid % CG, rg = tid / CG;
#pragma unroll
  for (int s = 0; s < RPT; ++s)
    *reinterpret_cast<uint4*>(&sm.X[rg * RPT + s][8 * cg]) = p.x[s];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(&sm.Xt[8 * cg + q][rg * RPT]);
    if constexpr (RPT == 4) {
      uint2 v;
      v.x = half_of(p.x[0], q) | (half_of(p.x[1], q) << 16);
      v.y = half_of(p.x[2], q) | (half_of(p.x[3], q) << 16);
      *reinterpret_cast<uint2*>(dst) = v;
    } else {
      *reinterpret_cast<uint32_t*>(dst) = half_of(p.x[0], q) | (half_of(p.x[1], q) << 16);
    }
  }
  const int jg = tid >> 2, c8 = 8 * (tid & 3);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    reinterpret_cast<uint16_t*>(&sm.Gt[c8 + q][0])[jg] = static_cast<uint16_t>(half_of(p.g, q));
  if (tid < kC) {
    sm.eta_raw[tid] = p.eta;
    sm.alpha_raw[tid] = p.alpha;
  }
}

// Block (i-block, j-block) list of the causal lower triangle of the 4x4 grid
// of 16x16 score blocks, dealt round-robin to the 4 waves.
__constant__ int kBlkI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kBlkJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <int D>
__global__ __launch_bounds__(kNT) void fwd_mfma(FwdArgs a) {
  static_assert(D == 64 || D == 128, "D");
  constexpr int NTILE = D / kTN;
  constexpr int XP = FwdSmem<D>::XP, TP = FwdSmem<D>::TP;
  constexpr int NS = (2 * (D / 16)) / 4;  // state blocks per wave
  __shared__ FwdSmem<D> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = blockIdx.x / (8 * NTILE), within = blockIdx.x % (8 * NTILE);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  const int tile = within >> 3;
  const int64_t BH = a.B * a.H;
  if (bh >= BH) return;
  const int r0 = tile * kTN;
  const int h = static_cast<int>(bh % a.H);
  const int64_t T = a.T;
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * D;
  const uint16_t* g = static_cast<const uint16_t*>(a.g) + bh * T * D;
  const float* eta = static_cast<const float*>(a.eta) + bh * T;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * D * D;
  uint16_t* y = a.y ? static_cast<uint16_t*>(a.y) + bh * T * D : nullptr;
  uint16_t* st = a.states ? static_cast<uint16_t*>(a.states) + bh * a.n_chunks * D * D : nullptr;
  const int g4 = lane >> 4, l16 = lane & 15;

  for (int idx = tid; idx < kTN * (D / 8); idx += kNT) {
    const int r = idx / (D / 8), c8 = 8 * (idx % (D / 8));
    *reinterpret_cast<uint4*>(&sm.W[r][c8]) =
        *reinterpret_cast<const uint4*>(W0 + static_cast<int64_t>(r0 + r) * D + c8);
    *reinterpret_cast<uint4*>(&sm.S[r][c8]) = make_uint4(0, 0, 0, 0);
  }
  for (int idx = tid; idx < kC * TP; idx += kNT) (&sm.A[0][0])[idx] = static_cast<__bf16>(0.f);

  f32x4 sacc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) sacc[s] = zero4();

  Prefetch<D> pf;
  load_chunk<D>(pf, x, g, eta, alpha, 0, static_cast<int>(std::min<int64_t>(kC, T)), r0, tid);

  for (int c = 0; c < a.n_chunks; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = static_cast<int>(std::min<int64_t>(kC, T - t0));
    stage_chunk<D>(sm, pf, tid);
    lds_barrier();  // S1: chunk tiles visible
    if (c + 1 < a.n_chunks) {
      const int64_t t1 = t0 + kC;
      load_chunk<D>(pf, x, g, eta, alpha, t1, static_cast<int>(std::min<int64_t>(kC, T - t1)),
                    r0, tid);
    }

    // gates: wave 0, lane = token
    if (wave == 0) {
      const float et = sm.eta_raw[lane];
      const ChunkGates cg = chunk_gates(sm.alpha_raw[lane], lane);
      const float l = cg.l, lp = cg.lq, ll = cg.llast;
      sm.lq[lane] = lp;
      sm.li[lane] = l;
      sm.eq[lane] = exp2f(lp);
      sm.bk[lane] = -et * exp2f(ll - l);
      sm.neta[lane] = -et;
      if (lane == 0) sm.gam = exp2f(ll);
    }

    // causal score blocks x_i . x_j (no gate needed yet)
    f32x4 xx[3];
    if (y) {
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        const int b = wave + 4 * s;
        xx[s] = zero4();
        if (b < 10) {
          const int ib = kBlkI[b], jb = kBlkJ[b];
#pragma unroll
          for (int kb = 0; kb < D / 32; ++kb)
            xx[s] = mfma16x16x32(frag(&sm.X[0][0], XP, ib * 16, kb * 32, lane),
                                 frag(&sm.X[0][0], XP, jb * 16, kb * 32, lane), xx[s]);
        }
      }
    }
    lds_barrier();  // S2: gates visible

    if (y) {
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        const int b = wave + 4 * s;
        if (b < 10) {
          const int ib = kBlkI[b], jb = kBlkJ[b];
          const int j = jb * 16 + l16;
          const float lj = sm.li[j], nj = sm.neta[j];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = ib * 16 + 4 * g4 + q;
            const float v = (j < i) ? xx[s][q] * exp2f(sm.lq[i] - lj) * nj : 0.f;
            sm.A[i][j] = static_cast<__bf16>(v);
          }
        }
      }
    }
    // chunk-start state for the backward (transposed, bf16)
    if (st) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int b = wave + 4 * s, rb = b / (D / 16), cb = b % (D / 16);
        uint2 v;
        v.x = bf16_bits(sacc[s][0]) | (bf16_bits(sacc[s][1]) << 16);
        v.y = bf16_bits(sacc[s][2]) | (bf16_bits(sacc[s][3]) << 16);
        *reinterpret_cast<uint2*>(st + (static_cast<int64_t>(c) * D + cb * 16 + l16) * D + r0 +
                                  rb * 16 + 4 * g4) = v;
      }
    }
    lds_barrier();  // S3: scores visible

    if (y) {
      const int ib = wave;
      f32x4 ya[2] = {zero4(), zero4()}, yb[2] = {zero4(), zero4()};
      const int nka = (ib + 2) / 2;
      for (int kb = 0; kb < nka; ++kb) {
        const bf16x8 af = frag(&sm.A[0][0], TP, ib * 16, kb * 32, lane);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          ya[nb] = mfma16x16x32(af, frag(&sm.Gt[0][0], TP, nb * 16, kb * 32, lane), ya[nb]);
      }
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8 xf = frag(&sm.X[0][0], XP, ib * 16, kb * 32, lane);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          ya[nb] = mfma16x16x32(xf, frag(&sm.W[0][0], XP, nb * 16, kb * 32, lane), ya[nb]);
          yb[nb] = mfma16x16x32(xf, frag(&sm.S[0][0], XP, nb * 16, kb * 32, lane), yb[nb]);
        }
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = ib * 16 + 4 * g4 + q;
          sm.Y[i][nb * 16 + l16] = static_cast<__bf16>(ya[nb][q] + sm.eq[i] * yb[nb][q]);
        }
    }
    lds_barrier();  // S4: y staged; every read of S done

    if (y) {
      const int i = tid >> 2, c8 = 8 * (tid & 3);
      if (i < cv)
        *reinterpret_cast<uint4*>(y + (t0 + i) * D + r0 + c8) =
            *reinterpret_cast<const uint4*>(&sm.Y[i][c8]);
    }
    // state update: D_out = Gamma D_in + (bk o G)^T X
    const float gam = sm.gam;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int b = wave + 4 * s, rb = b / (D / 16), cb = b % (D / 16);
      sacc[s] = sacc[s] * gam;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 ga = frag(&sm.Gt[0][0], TP, rb * 16, kb * 32, lane);
        const int j0 = kb * 32 + 8 * g4;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          ga[e] = static_cast<__bf16>(static_cast<float>(ga[e]) * sm.bk[j0 + e]);
        sacc[s] = mfma16x16x32(ga, frag(&sm.Xt[0][0], TP, cb * 16, kb * 32, lane), sacc[s]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sm.S[rb * 16 + 4 * g4 + q][cb * 16 + l16] = static_cast<__bf16>(sacc[s][q]);
    }
    lds_barrier();  // S5: new state visible; chunk tiles free
  }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const int64_t BH = a.B * a.H;
  const int64_t groups = (BH + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (D / kTN)));
  hipLaunchKernelGGL(fwd_mfma<D>, grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_fwd(const FwdArgs& a, hipStream_t s) {
  return a.d_in == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace gls
