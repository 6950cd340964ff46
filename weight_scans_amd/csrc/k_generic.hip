// k_generic.hip -- portable chunked scan kernels (VALU arithmetic, LDS tiles).
//
// These evaluate the same chunked associative scan as the matrix-core kernels
// for any 1 <= d_in, d_out <= 128 and every io type (fp64 and fp32 throughout,
// bf16 io with fp32 arithmetic).  They are the fp64/fp32 path and the
// cross-check for the matrix-core path.
//
// Notation (one sequence-head, one chunk of cv <= C tokens, local index i):
//   l_i   = sum_{r <= i} log alpha_r  (inclusive, chunk-local), l_{-1} = 0
//   Mf_ij = exp(l_{i-1} - l_j)         decay from the update at j to the read
//                                      at i (j < i), every exponent <= 0
//   Gamma = exp(l_{cv-1})              decay across the whole chunk
// The adaptation read by token i and the adjoint after token i are
//   D_i   = e^{l_{i-1}} D_in + sum_{j<i} Mf_ij (-eta_j) g_j x_j^T
//   Lam_i = e^{l_{cv-1}-l_i} Lam_out + sum_{u>i} Mf_ui dy_u x_u^T
// i.e. the correction is a sum of the earlier rank-one updates, each damped by
// the retention gates applied after it ("Parallelize the Training, Keep the
// Learning Serial", cognaptus.com, section
// "Once the gradient signals are known, the weight trajectory becomes
// parallelizable"), composed chunk to chunk as an affine scan:
//   D_out  = Gamma D_in  + sum_j e^{l_{cv-1}-l_j} (-eta_j) g_j x_j^T
//   Lam_in = Gamma Lam_out + sum_u e^{l_{u-1}} dy_u x_u^T
#include <algorithm>

#include "dev_common.hpp"
#include "internal.hpp"

namespace gls {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Forward: grid (B*H, ceil(d_out / TN)).  The row tile [r0, r0+TN) of D lives
// in LDS across chunks; each chunk forms the causal decayed score matrix
// A_ij = Mf_ij (q_i . x_j)(-eta_j) and emits
//   y_i = W0 q_i + e^{l_{i-1}} D_in q_i + sum_{j<i} A_ij g_j,
// with q = x (the scan) or, with QK, a read vector of its own (x is then
// only the write key).  OT is the type y is stored in.
// ---------------------------------------------------------------------------
template <typename T, typename IO, typename OT, int C, int TN, bool QK>
__global__ __launch_bounds__(kThreads) void fwd_generic(FwdArgs a) {
  constexpr int DM = kGenericMaxD, P = DM + 1;
  __shared__ T sX[C][P];
  __shared__ T sQv[QK ? C : 1][QK ? P : 1];
  __shared__ T sG[C][TN];
  __shared__ T sA[C][C + 1];
  __shared__ T sS[TN][P];
  __shared__ T sW[TN][P];
  __shared__ T sL[C], sQ[C], sBk[C], sEta[C];
  __shared__ T sGam;

  const int tid = threadIdx.x;
  const int r0 = blockIdx.y * TN;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int din = a.d_in, dout = a.d_out;
  const int nr = min(TN, dout - r0);
  const IO* x = static_cast<const IO*>(a.x) + bh * a.T * din;
  const IO* q = QK ? static_cast<const IO*>(a.q) + bh * a.T * din : x;
  const IO* g = static_cast<const IO*>(a.g) + bh * a.T * dout;
  const T* eta = static_cast<const T*>(a.eta) + bh * a.T;
  const T* alpha = static_cast<const T*>(a.alpha) + bh * a.T;
  const IO* W0 = static_cast<const IO*>(a.W0) + static_cast<int64_t>(h) * dout * din;
  OT* y = a.y ? static_cast<OT*>(a.y) + bh * a.T * dout : nullptr;
  // the read vectors: the key tile itself, or a tile of their own
  const auto QT = [&](int i, int k) -> T {
    if constexpr (QK) return sQv[i][k]; else return sX[i][k];
  };

  for (int idx = tid; idx < TN * din; idx += kThreads) {
    const int r = idx / din, k = idx % din;
    sS[r][k] = T(0);
    const int64_t wi = a.w0_t ? static_cast<int64_t>(k) * dout + r0 + r
                              : static_cast<int64_t>(r0 + r) * din + k;
    sW[r][k] = (r < nr) ? load_as<T>(W0, wi) : T(0);
  }
  __syncthreads();

  for (int c = 0; c < a.n_chunks; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * C;
    const int cv = static_cast<int>(min(static_cast<int64_t>(C), a.T - t0));
    if (a.states && (c % a.ckpt_every) == 0) {
      T* st = static_cast<T*>(a.states) +
              ((bh * a.n_ckpt + c / a.ckpt_every) * dout + r0) * static_cast<int64_t>(din);
      for (int idx = tid; idx < nr * din; idx += kThreads) st[idx] = sS[idx / din][idx % din];
    }
    for (int idx = tid; idx < cv * din; idx += kThreads) {
      sX[idx / din][idx % din] = load_as<T>(x, (t0 + idx / din) * din + idx % din);
      if constexpr (QK) sQv[idx / din][idx % din] = load_as<T>(q, (t0 + idx / din) * din + idx % din);
    }
    for (int idx = tid; idx < cv * TN; idx += kThreads) {
      const int i = idx / TN, r = idx % TN;
      sG[i][r] = (r < nr) ? load_as<T>(g, (t0 + i) * dout + r0 + r) : T(0);
    }
    if (tid < cv) sEta[tid] = eta[t0 + tid];
    if (tid == 0) {
      T l = T(0);
      for (int i = 0; i < cv; ++i) {
        sQ[i] = exp(l);  // e^{l_{i-1}}
        l += log(alpha[t0 + i]);
        sL[i] = l;
      }
      sGam = exp(l);
      for (int j = 0; j < cv; ++j) sBk[j] = -eta[t0 + j] * exp(l - sL[j]);
    }
    __syncthreads();

    for (int idx = tid; y && idx < C * C; idx += kThreads) {
      const int i = idx / C, j = idx % C;
      T v = T(0);
      if (j < i && i < cv) {
        T dot = T(0);
        for (int k = 0; k < din; ++k) dot += QT(i, k) * sX[j][k];
        v = dot * exp(sL[i - 1] - sL[j]) * (-sEta[j]);
      }
      sA[i][j] = v;
    }
    __syncthreads();

    if (y) {
      for (int idx = tid; idx < cv * TN; idx += kThreads) {
        const int i = idx / TN, r = idx % TN;
        if (r >= nr) continue;
        T a0 = T(0), a1 = T(0), a2 = T(0);
        for (int k = 0; k < din; ++k) {
          a0 += sW[r][k] * QT(i, k);
          a1 += sS[r][k] * QT(i, k);
        }
        for (int j = 0; j < i; ++j) a2 += sA[i][j] * sG[j][r];
        store_from<T>(y, (t0 + i) * dout + r0 + r, a0 + sQ[i] * a1 + a2);
      }
    }
    __syncthreads();

    for (int idx = tid; idx < nr * din; idx += kThreads) {
      const int r = idx / din, k = idx % din;
      T s = sGam * sS[r][k];
      for (int j = 0; j < cv; ++j) s += sG[j][r] * sBk[j] * sX[j][k];
      sS[r][k] = s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Backward: grid (B*H, n_tiles), reverse over chunks.  Work-group k holds
//   columns K = [k0, k0+TK) of D_in (from the stored chunk states) and of Lam,
//   rows    R = [k0, k0+TK) of Lam,  and the columns K of dW0.
// With q the read vector and x the write key (q = x for the scan), per chunk,
// for j < i:  Be_ij = Mf_ij (dy_i . g_j)(-eta_j),  P_ij = Mf_ij (q_i . x_j):
//   dq_i[K]  = W0[:,K]^T dy_i + e^{l_{i-1}} D_in[:,K]^T dy_i + sum_{j<i} Be_ij x_j[K]
//   dx_i[K]  = -eta_i e^{l_{cv-1}-l_i} Lam_out[:,K]^T g_i + sum_{u>i} Be_ui q_u[K]
//              (the scan returns dq + dx as dx)
//   u_i[R]   = e^{l_{cv-1}-l_i} Lam_out[R,:] x_i + sum_{u>i} P_ui dy_u[R]
//   dg_i[R]  = -eta_i u_i[R],  deta_i partial = -g_i[R] . u_i[R]
//   dalpha_i = <Lam_i, D_i> = e^{l_{cv-1}-l_i+l_{i-1}} <Lam_out, D_in>
//              + e^{l_{cv-1}-l_i} sum_{j<i} Mf_ij (-eta_j) x_j.(Lam_out^T g_j)
//              + e^{l_{i-1}} sum_{u>i} Mf_ui q_u.(D_in^T dy_u)
//              + (1/alpha_i) sum_{u>i, j<i} Be_uj (q_u . x_j)
//   (the first three split over column tiles; the last is added by tile 0),
//   Lam_in = Gamma Lam_out + sum_u e^{l_{u-1}} dy_u q_u^T,  dW0 += dy_u q_u^T.
// OT is the type dx, dg and dq are stored in.
// ---------------------------------------------------------------------------
template <typename T, typename IO, typename OT, int C, int TK, bool QK>
__global__ __launch_bounds__(kThreads) void bwd_generic(BwdArgs a) {
  constexpr int DM = kGenericMaxD, P = DM + 1, PK = TK + 1;
  __shared__ T sX[C][P], sG[C][P], sD[C][P];
  __shared__ T sQv[QK ? C : 1][QK ? P : 1];
  __shared__ T sPm[C][C + 1], sBe[C][C + 1], sZ[C][C + 1];
  __shared__ T sSin[DM][PK], sLk[DM][PK], sW[DM][PK], sdW[DM][PK];
  __shared__ T sLr[TK][P];
  __shared__ T sLg[C][PK], sSd[C][PK], sLx[C][PK];
  __shared__ T sL[C], sE1[C], sE2[C], sEta[C], sAl[C], sPj[C], sRu[C];
  __shared__ T sRed[kThreads];
  __shared__ T sC0, sGam;

  const int tid = threadIdx.x;
  const int k = blockIdx.y;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int din = a.d_in, dout = a.d_out;
  const int k0 = k * TK;
  const int nk = max(0, min(TK, din - k0));   // columns of this tile
  const int nrr = max(0, min(TK, dout - k0));  // rows of this tile
  const int64_t BHT = a.B * a.H * a.T;
  const IO* x = static_cast<const IO*>(a.x) + bh * a.T * din;
  const IO* q = QK ? static_cast<const IO*>(a.q) + bh * a.T * din : x;
  const IO* g = static_cast<const IO*>(a.g) + bh * a.T * dout;
  const IO* dy = static_cast<const IO*>(a.dy) + bh * a.T * dout;
  const T* eta = static_cast<const T*>(a.eta) + bh * a.T;
  const T* alpha = static_cast<const T*>(a.alpha) + bh * a.T;
  const IO* W0 = static_cast<const IO*>(a.W0) + static_cast<int64_t>(h) * dout * din;
  OT* dx = static_cast<OT*>(a.dx) + bh * a.T * din;
  OT* dq = QK ? static_cast<OT*>(a.dq) + bh * a.T * din : nullptr;
  OT* dg = static_cast<OT*>(a.dg) + bh * a.T * dout;
  T* pe = static_cast<T*>(a.part_eta) + k * BHT + bh * a.T;
  T* pa = static_cast<T*>(a.part_alpha) + k * BHT + bh * a.T;
  const auto QT = [&](int i, int kk) -> T {
    if constexpr (QK) return sQv[i][kk]; else return sX[i][kk];
  };

  for (int idx = tid; idx < dout * TK; idx += kThreads) {
    const int r = idx / TK, kk = idx % TK;
    sLk[r][kk] = T(0);
    sdW[r][kk] = T(0);
    const int64_t wi = a.w0_t ? static_cast<int64_t>(k0 + kk) * dout + r
                              : static_cast<int64_t>(r) * din + k0 + kk;
    sW[r][kk] = (kk < nk) ? load_as<T>(W0, wi) : T(0);
  }
  for (int idx = tid; idx < TK * din; idx += kThreads) sLr[idx / din][idx % din] = T(0);
  __syncthreads();

  for (int c = a.n_chunks - 1; c >= 0; --c) {
    const int64_t t0 = static_cast<int64_t>(c) * C;
    const int cv = static_cast<int>(min(static_cast<int64_t>(C), a.T - t0));
    for (int idx = tid; idx < cv * din; idx += kThreads) {
      sX[idx / din][idx % din] = load_as<T>(x, (t0 + idx / din) * din + idx % din);
      if constexpr (QK) sQv[idx / din][idx % din] = load_as<T>(q, (t0 + idx / din) * din + idx % din);
    }
    for (int idx = tid; idx < cv * dout; idx += kThreads) {
      const int i = idx / dout, r = idx % dout;
      sG[i][r] = load_as<T>(g, (t0 + i) * dout + r);
      sD[i][r] = load_as<T>(dy, (t0 + i) * dout + r);
    }
    if (tid < cv) {
      sEta[tid] = eta[t0 + tid];
      sAl[tid] = alpha[t0 + tid];
    }
    {
      // D_in[:, K] for this chunk (ckpt_every == 1 for this kernel)
      const T* st = static_cast<const T*>(a.states) +
                    (bh * a.n_ckpt + c / a.ckpt_every) * static_cast<int64_t>(dout) * din;
      for (int idx = tid; idx < dout * TK; idx += kThreads) {
        const int r = idx / TK, kk = idx % TK;
        sSin[r][kk] = (kk < nk) ? st[static_cast<int64_t>(r) * din + k0 + kk] : T(0);
      }
    }
    __syncthreads();

    if (tid == 0) {
      T l = T(0);
      for (int i = 0; i < cv; ++i) {
        sE1[i] = exp(l);  // e^{l_{i-1}}
        l += log(sAl[i]);
        sL[i] = l;
      }
      sGam = exp(l);
      for (int i = 0; i < cv; ++i) sE2[i] = exp(l - sL[i]);  // e^{l_{cv-1}-l_i}
    }
    __syncthreads();

    for (int idx = tid; idx < C * C; idx += kThreads) {
      const int i = idx / C, j = idx % C;
      T p = T(0), be = T(0), z = T(0);
      if (j < i && i < cv) {
        T xx = T(0), dgd = T(0);
        for (int qq = 0; qq < din; ++qq) xx += QT(i, qq) * sX[j][qq];
        for (int qq = 0; qq < dout; ++qq) dgd += sD[i][qq] * sG[j][qq];
        const T mf = exp(sL[i - 1] - sL[j]);
        p = mf * xx;
        be = mf * dgd * (-sEta[j]);
        z = be * xx;
      }
      sPm[i][j] = p;
      sBe[i][j] = be;
      sZ[i][j] = z;
    }
    for (int idx = tid; idx < cv * TK; idx += kThreads) {
      const int i = idx / TK, kk = idx % TK;
      T lg = T(0), sd = T(0), lx = T(0);
      if (kk < nk) {
        for (int r = 0; r < dout; ++r) {
          lg += sLk[r][kk] * sG[i][r];
          sd += sSin[r][kk] * sD[i][r];
        }
      }
      if (kk < nrr)
        for (int qq = 0; qq < din; ++qq) lx += sLr[kk][qq] * sX[i][qq];
      sLg[i][kk] = lg;
      sSd[i][kk] = sd;
      sLx[i][kk] = lx;
    }
    {
      T part = T(0);
      if (nk > 0)
        for (int idx = tid; idx < dout * nk; idx += kThreads) {
          const int r = idx / nk, kk = idx % nk;
          part += sLk[r][kk] * sSin[r][kk];
        }
      sRed[tid] = part;
    }
    __syncthreads();

    if (tid == 0) {
      T sm = T(0);
      for (int qq = 0; qq < kThreads; ++qq) sm += sRed[qq];
      sC0 = sm;
    }
    if (tid < cv) {
      T pj = T(0), ru = T(0);
      for (int kk = 0; kk < nk; ++kk) {
        pj += sX[tid][k0 + kk] * sLg[tid][kk];
        ru += QT(tid, k0 + kk) * sSd[tid][kk];
      }
      sPj[tid] = pj;
      sRu[tid] = ru;
    }
    __syncthreads();

    for (int idx = tid; idx < cv * TK; idx += kThreads) {
      const int i = idx / TK, kk = idx % TK;
      if (kk >= nk) continue;
      const int col = k0 + kk;
      T vq = T(0);
      for (int r = 0; r < dout; ++r) vq += sW[r][kk] * sD[i][r];
      vq += sE1[i] * sSd[i][kk];
      for (int j = 0; j < i; ++j) vq += sBe[i][j] * sX[j][col];
      T vk = -sEta[i] * sE2[i] * sLg[i][kk];
      for (int j = i + 1; j < cv; ++j) vk += sBe[j][i] * QT(j, col);
      if constexpr (QK) {
        store_from<T>(dq, (t0 + i) * din + col, vq);
        store_from<T>(dx, (t0 + i) * din + col, vk);
      } else {
        store_from<T>(dx, (t0 + i) * din + col, vq + vk);
      }
    }
    if (tid < cv) {
      const int i = tid;
      T de = T(0);
      for (int rr = 0; rr < nrr; ++rr) {
        const int r = k0 + rr;
        T u = sE2[i] * sLx[i][rr];
        for (int v = i + 1; v < cv; ++v) u += sPm[v][i] * sD[v][r];
        store_from<T>(dg, (t0 + i) * dout + r, -sEta[i] * u);
        de -= sG[i][r] * u;
      }
      pe[t0 + i] = de;
      const T lim1 = (i > 0) ? sL[i - 1] : T(0);
      T t1 = exp(sL[cv - 1] - sL[i] + lim1) * sC0;
      T t2 = T(0), t3 = T(0), t4 = T(0);
      for (int j = 0; j < i; ++j) t2 += exp(sL[i - 1] - sL[j]) * (-sEta[j]) * sPj[j];
      for (int v = i + 1; v < cv; ++v) t3 += exp(sL[v - 1] - sL[i]) * sRu[v];
      if (k == 0) {
        for (int v = i + 1; v < cv; ++v)
          for (int j = 0; j < i; ++j) t4 += sZ[v][j];
        t4 = t4 / sAl[i];
      }
      pa[t0 + i] = t1 + sE2[i] * t2 + sE1[i] * t3 + t4;
    }
    __syncthreads();

    for (int idx = tid; nk > 0 && idx < dout * nk; idx += kThreads) {
      const int r = idx / nk, kk = idx % nk;
      const int col = k0 + kk;
      T s1 = T(0), s2 = T(0);
      for (int u = 0; u < cv; ++u) {
        const T pr = sD[u][r] * QT(u, col);
        s1 += sE1[u] * pr;
        s2 += pr;
      }
      sLk[r][kk] = sGam * sLk[r][kk] + s1;
      sdW[r][kk] += s2;
    }
    for (int idx = tid; nrr > 0 && idx < nrr * din; idx += kThreads) {
      const int rr = idx / din, qq = idx % din;
      const int r = k0 + rr;
      T s1 = T(0);
      for (int u = 0; u < cv; ++u) s1 += sE1[u] * sD[u][r] * QT(u, qq);
      sLr[rr][qq] = sGam * sLr[rr][qq] + s1;
    }
    __syncthreads();
  }

  T* pw = static_cast<T*>(a.part_dW0) + bh * static_cast<int64_t>(dout) * din;
  for (int idx = tid; nk > 0 && idx < dout * nk; idx += kThreads) {
    const int r = idx / nk, kk = idx % nk;
    const int64_t wi = a.w0_t ? static_cast<int64_t>(k0 + kk) * dout + r
                              : static_cast<int64_t>(r) * din + k0 + kk;
    pw[wi] = sdW[r][kk];
  }
}

// Fixed-order sums of the per-tile / per-batch partials.
template <typename T>
__global__ __launch_bounds__(kThreads) void finalize_kernel(FinArgs a) {
  const int64_t BHT = a.B * a.H * a.T;
  const int64_t dd = static_cast<int64_t>(a.d_in) * a.d_out;
  const int64_t HD = a.H * dd;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const T* pe = static_cast<const T*>(a.part_eta);
  const T* pa = static_cast<const T*>(a.part_alpha);
  const T* pw = static_cast<const T*>(a.part_dW0);
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
       !(a.eta_done && a.alpha_done) && i < BHT; i += stride) {
    T se = T(0), sa = T(0);
    for (int k = 0; k < a.n_tiles; ++k) {
      if (!a.eta_done) se += pe[k * BHT + i];
      if (!a.alpha_done) sa += pa[k * BHT + i];
    }
    if (!a.eta_done) static_cast<T*>(a.deta)[i] = se;
    if (!a.alpha_done) static_cast<T*>(a.dalpha)[i] = sa;
  }
  const int64_t nb = a.B * a.n_seg;  // partials [n_seg][B][H][.]
  if constexpr (sizeof(T) == 4) {
    if ((HD & 3) == 0) {
      // four elements per lane group of L = a.lanes lanes (a power of two up
      // to 64): lane j of a group sums partials j, j + L, ... in that order,
      // then the group folds by xor-shuffles over 1, 2, .., L / 2 -- a fixed
      // order, so the result is the same from run to run
      typedef float f4 __attribute__((ext_vector_type(4)));
      const f4* pw4 = reinterpret_cast<const f4*>(pw);
      const int64_t HD4 = HD >> 2;
      const int L = a.lanes, lg = __builtin_ctz(static_cast<unsigned>(L));
      const int gpw = 64 >> lg;  // groups per wave
      const int lane = static_cast<int>(threadIdx.x) & 63, j = lane & (L - 1);
      const int64_t wave = (blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x) >> 6;
      const int64_t n_waves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
      // the loop bound is the same for every lane of a wave (the shuffles
      // below need the whole wave)
      for (int64_t base = wave * gpw; base < HD4; base += n_waves * gpw) {
        const int64_t gi = base + (lane >> lg);
        const bool on = gi < HD4;
        f4 s = {0.f, 0.f, 0.f, 0.f};
        if (on)
          for (int64_t b = j; b < nb; b += L) s += pw4[b * HD4 + gi];
        for (int o = 1; o < L; o <<= 1) {
          s[0] += __shfl_xor(s[0], o, 64);
          s[1] += __shfl_xor(s[1], o, 64);
          s[2] += __shfl_xor(s[2], o, 64);
          s[3] += __shfl_xor(s[3], o, 64);
        }
        if (on && j == 0) reinterpret_cast<f4*>(a.dW0)[gi] = s;
      }
      return;
    }
  }
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < HD; i += stride) {
    T s = T(0);
    for (int64_t b = 0; b < nb; ++b) s += pw[b * HD + i];
    static_cast<T*>(a.dW0)[i] = s;
  }
}

// Zero fill of n 4-byte words (a kernel rather than a memset node, so that a
// captured graph replays it like any other launch).
__global__ __launch_bounds__(kThreads) void clear_kernel(uint32_t* p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n; i += stride)
    p[i] = 0u;
}

template <typename T, typename IO, typename OT, int C, bool QK>
hipError_t fwd_c(const FwdArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(a.B * a.H), (a.d_out + kGenericTile - 1) / kGenericTile);
  hipLaunchKernelGGL((fwd_generic<T, IO, OT, C, kGenericTile, QK>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, typename IO, typename OT, int C, bool QK>
hipError_t bwd_c(const BwdArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(a.B * a.H), a.n_tiles);
  hipLaunchKernelGGL((bwd_generic<T, IO, OT, C, kGenericTile, QK>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// chunk dispatch (the host has checked the chunk against generic_chunk_ok)
template <typename T, typename IO, typename OT, bool QK>
hipError_t fwd_q(const FwdArgs& a, hipStream_t s) {
  if (a.chunk == 8) return fwd_c<T, IO, OT, 8, QK>(a, s);
  if constexpr (sizeof(T) == 8) {
    return fwd_c<T, IO, OT, 16, QK>(a, s);
  } else {
    if (a.chunk == 16) return fwd_c<T, IO, OT, 16, QK>(a, s);
    return fwd_c<T, IO, OT, 32, QK>(a, s);
  }
}
template <typename T, typename IO, typename OT, bool QK>
hipError_t bwd_q(const BwdArgs& a, hipStream_t s) {
  if (a.chunk == 8) return bwd_c<T, IO, OT, 8, QK>(a, s);
  if constexpr (sizeof(T) == 8) {
    // fp64 with a read vector of its own fits LDS at chunk 8 only
    if constexpr (QK) return hipErrorInvalidValue;
    else return bwd_c<T, IO, OT, 16, QK>(a, s);
  } else {
    if (a.chunk == 16) return bwd_c<T, IO, OT, 16, QK>(a, s);
    return bwd_c<T, IO, OT, 32, QK>(a, s);
  }
}

}  // namespace

bool generic_chunk_ok(int io, int chunk) {
  if (io == IO_F64) return chunk == 8 || chunk == 16;
  return chunk == 8 || chunk == 16 || chunk == 32;
}

int generic_default_chunk(int io) { return io == IO_F64 ? 16 : 32; }

hipError_t launch_generic_fwd(int io, const FwdArgs& a, hipStream_t s) {
  const bool qk = a.q != nullptr;
  switch (io) {
    case IO_F64:
      return qk ? fwd_q<double, double, double, true>(a, s) : fwd_q<double, double, double, false>(a, s);
    case IO_F32:
      return qk ? fwd_q<float, float, float, true>(a, s) : fwd_q<float, float, float, false>(a, s);
    default:
      if (a.out_f32)
        return qk ? fwd_q<float, bf16, float, true>(a, s) : fwd_q<float, bf16, float, false>(a, s);
      return qk ? fwd_q<float, bf16, bf16, true>(a, s) : fwd_q<float, bf16, bf16, false>(a, s);
  }
}

hipError_t launch_generic_bwd(int io, const BwdArgs& a, hipStream_t s) {
  const bool qk = a.q != nullptr;
  switch (io) {
    case IO_F64:
      return qk ? bwd_q<double, double, double, true>(a, s) : bwd_q<double, double, double, false>(a, s);
    case IO_F32:
      return qk ? bwd_q<float, float, float, true>(a, s) : bwd_q<float, float, float, false>(a, s);
    default:
      if (a.out_f32)
        return qk ? bwd_q<float, bf16, float, true>(a, s) : bwd_q<float, bf16, float, false>(a, s);
      return qk ? bwd_q<float, bf16, bf16, true>(a, s) : bwd_q<float, bf16, bf16, false>(a, s);
  }
}

hipError_t launch_clear(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 4);
  if (n == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(std::min<int64_t>(1024, (n + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(kThreads), 0, s, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_finalize(int io, const FinArgs& a0, hipStream_t s) {
  FinArgs a = a0;
  // lanes per dW0 element group: the partial count rounded up to a power of
  // two, at most 64
  const int64_t nb = a.B * a.n_seg;
  a.lanes = 1;
  while (a.lanes < 64 && a.lanes < nb) a.lanes <<= 1;
  // threads: the per-token sums, the lane groups of the 4-wide dW0 sums, or
  // one per dW0 element (the element-wise path: fp64, or H d_in d_out not a
  // multiple of 4)
  const int64_t HD = a.H * static_cast<int64_t>(a.d_in) * a.d_out;
  const int64_t n = std::max<int64_t>({(a.eta_done && a.alpha_done) ? 0 : a.B * a.H * a.T, HD,
                                       (HD + 3) / 4 * a.lanes});
  const unsigned blocks = static_cast<unsigned>(std::min<int64_t>(4096, (n + kThreads - 1) / kThreads));
  if (blocks == 0) return hipSuccess;
  if (io == IO_F64)
    hipLaunchKernelGGL(finalize_kernel<double>, dim3(blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(finalize_kernel<float>, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace gls
