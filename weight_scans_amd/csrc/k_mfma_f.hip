// k_mfma_f.hip -- matrix-core scans in fp32 and fp64 (gfx950,
// v_mfma_f32_16x16x4_f32 and v_mfma_f64_16x16x4_f64), chunk of 64 tokens,
// any 1 <= d_in, d_out <= DM with DM = 64 (fp32) or 32 (fp64), io dtype =
// compute dtype.
//
// The same chunked form of the recurrence as the bf16 kernels ("Parallelize
// the Training, Keep the Learning Serial", cognaptus.com, section "Once the
// gradient signals are known, the weight trajectory becomes parallelizable";
// its exact adjoint, GradLev abstract, omanscience.com), with every product
// on the matrix cores in the compute precision.  Per chunk (l = chunk-local
// inclusive cumsum of log2 alpha, lq_i = l_{i-1}, e(.) = 2^(.)):
//   A_ij  = (x_i . x_j) e(lq_i - l_j)(-eta_j)                    (j < i)
//   y_i   = W0 x_i + e(lq_i) D_in x_i + sum_j A_ij g_j
//   D_out = e(l_last) D_in + sum_j e(l_last - l_j)(-eta_j) g_j x_j^T
// and, walking the chunks backwards with Lam_out = dL/dD after the chunk,
//   u_i   = e(l_last - l_i) Lam_out x_i + sum_{u>i} P_ui dy_u,  P_ui = e(lq_u - l_i)(x_u . x_i)
//   dx_i  = W0^T dy_i + e(lq_i) D_in^T dy_i + sum_j M_ij x_j - eta_i e(l_last - l_i) Lam_out^T g_i
//   dg_i  = -eta_i u_i,  deta_i = -g_i . u_i,  M = Be + Be^T,  Be_ij = e(lq_i - l_j)(-eta_j)(dy_i . g_j)
//   Lam_in = e(l_last) Lam_out + sum_u e(lq_u) dy_u x_u^T,   dW0 += sum_u dy_u x_u^T
//   dalpha_i = e(l_last - l_i) e(lq_i) <Lam_out, D_in> + e(l_last - l_i) sum_{j<i} e(lq_i - l_j)(-eta_j) pp_j
//            + e(lq_i) sum_{u>i} e(lq_u - l_i) rr_u + (sum_{u>i} qq_u - sum_{j>=i} kk_j) / alpha_i
// (pp_j = g_j . (Lam_out x_j), rr_u = x_u . (D_in^T dy_u), qq / kk the row /
// column sums of Be o XX).  The forward runs one work-group per sequence-head
// and 16-row tile of D; the backward one work-group per sequence-head with the
// whole adjoint.  Tiles live in LDS in the compute type (row stride padded by
// one element); a 16 x 16 output block takes K / 4 MFMAs, each lane
// supplying one element of A and of B.
#include <algorithm>
#include <cstdint>

#include "dev_common.hpp"
#include "internal.hpp"

namespace gls {
namespace {

constexpr int kC = 64;      // tokens per chunk
constexpr int kNT = 256;    // threads (four waves)
constexpr int kCP = kC + 1; // padded row of a [64][64] tile

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

// One MFMA of a 16 x 16 block with K = 4: lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16]; it receives D[row(l, q)][l % 16], q = 0..3 (layouts
// measured on the device: fp32 rows 4 (l / 16) + q, fp64 rows l / 16 + 4 q).
template <typename T>
struct Mx;
template <>
struct Mx<float> {
  using acc = f32x4;
  static __device__ __forceinline__ acc mma(float a, float b, const acc& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int row(int lane, int q) { return 4 * (lane >> 4) + q; }
  static __device__ __forceinline__ acc zero() { return acc{0.f, 0.f, 0.f, 0.f}; }
};
template <>
struct Mx<double> {
  using acc = f64x4;
  static __device__ __forceinline__ acc mma(double a, double b, const acc& c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int row(int lane, int q) { return (lane >> 4) + 4 * q; }
  static __device__ __forceinline__ acc zero() { return acc{0.0, 0.0, 0.0, 0.0}; }
};

// c += sum_{k < K} A(m0 + m, k) B(k, n0 + n) over one 16 x 16 block; fa(m, k)
// and fb(k, n) read the operands (m, n in 0..15), K a multiple of 4.
template <typename T, typename FA, typename FB>
__device__ __forceinline__ typename Mx<T>::acc mm(typename Mx<T>::acc c, int K, FA fa, FB fb,
                                                  int lane) {
  const int i = lane & 15, k = lane >> 4;
  for (int k0 = 0; k0 < K; k0 += 4) c = Mx<T>::mma(fa(i, k0 + k), fb(k0 + k, i), c);
  return c;
}

__device__ __forceinline__ float xlog2(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ double xlog2(double v) { return log2(v); }
__device__ __forceinline__ float xexp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ double xexp2(double v) { return exp2(v); }

// Wave-level scans (lane = token) in the compute type, by shuffles.
template <typename T>
__device__ __forceinline__ T scan_add(T v, int lane) {  // inclusive prefix sum
  for (int o = 1; o < 64; o <<= 1) {
    const T p = __shfl_up(v, o, 64);
    if (lane >= o) v += p;
  }
  return v;
}
template <typename T>
__device__ __forceinline__ T suffix_add(T v, int lane) {  // inclusive suffix sum
  for (int o = 1; o < 64; o <<= 1) {
    const T p = __shfl_down(v, o, 64);
    if (lane + o < 64) v += p;
  }
  return v;
}
// Inclusive affine scans: prefix B_i = sum_{j<=i} (prod_{j<r<=i} a_r) b_j,
// suffix B_i = sum_{u>=i} (prod_{i<=r<u} a_r) b_u.
template <typename T>
__device__ __forceinline__ T scan_affine(T a, T b, int lane) {
  for (int o = 1; o < 64; o <<= 1) {
    const T ap = __shfl_up(a, o, 64), bp = __shfl_up(b, o, 64);
    if (lane >= o) {
      b = b + a * bp;
      a = a * ap;
    }
  }
  return b;
}
template <typename T>
__device__ __forceinline__ T suffix_affine(T a, T b, int lane) {
  for (int o = 1; o < 64; o <<= 1) {
    const T an = __shfl_down(a, o, 64), bn = __shfl_down(b, o, 64);
    if (lane + o < 64) {
      b = b + a * bn;
      a = a * an;
    }
  }
  return b;
}

// Gates of a chunk (one wave, lane = token; padding tokens alpha = 1, eta = 0).
template <typename T>
struct GatesF {
  T lq[kC], li[kC], nb[kC], eq[kC], e2[kC], al[kC];
  T gam;
};
template <typename T>
__device__ __forceinline__ void gates_mf(const T* eta, const T* alpha, int64_t t0, int cv,
                                         GatesF<T>& g, int lane) {
  const T al = lane < cv ? alpha[t0 + lane] : T(1);
  const T et = lane < cv ? eta[t0 + lane] : T(0);
  const T l = scan_add<T>(xlog2(al), lane);
  const T lq = __shfl_up(l, 1, 64);
  const T lqi = lane == 0 ? T(0) : lq;
  const T llast = __shfl(l, 63, 64);
  g.lq[lane] = lqi;
  g.li[lane] = l;
  g.nb[lane] = -et;
  g.eq[lane] = xexp2(lqi);
  g.e2[lane] = xexp2(llast - l);
  g.al[lane] = al;
  if (lane == 0) g.gam = xexp2(llast);
}

// ------------------------------------------------------------------ forward
template <typename T, int DM>
__global__ __launch_bounds__(kNT) void fwd_mf(FwdArgs a) {
  constexpr int DP = DM + 1;
  using M = Mx<T>;
  __shared__ T sX[kC][DP];     // x of the chunk (columns past d_in zero)
  __shared__ T sG[kC][17];     // g of the row tile
  __shared__ T sA[kC][kCP];    // decayed scores (upper blocks stay zero)
  __shared__ T sS[16][DP];     // D_in of the row tile
  __shared__ T sW[16][DP];     // W0 rows of the tile
  __shared__ GatesF<T> gt;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bh = blockIdx.x;
  const int r0 = blockIdx.y * 16;
  const int h = static_cast<int>(bh % a.H);
  const int din = a.d_in, dout = a.d_out;
  const int64_t T_ = a.T;
  const T* x = static_cast<const T*>(a.x) + bh * T_ * din;
  const T* g = static_cast<const T*>(a.g) + bh * T_ * dout;
  const T* eta = static_cast<const T*>(a.eta) + bh * T_;
  const T* alpha = static_cast<const T*>(a.alpha) + bh * T_;
  const T* W0 = static_cast<const T*>(a.W0) + static_cast<int64_t>(h) * dout * din;
  T* y = a.y ? static_cast<T*>(a.y) + bh * T_ * dout : nullptr;
  T* st = a.states ? static_cast<T*>(a.states) + bh * static_cast<int64_t>(a.n_chunks) * dout * din
                   : nullptr;

  for (int idx = tid; idx < 16 * DP; idx += kNT) {
    const int r = idx / DP, k = idx % DP;
    sS[r][k] = T(0);
    sW[r][k] = (r0 + r < dout && k < din) ? W0[static_cast<int64_t>(r0 + r) * din + k] : T(0);
  }
  for (int idx = tid; idx < kC * kCP; idx += kNT) sA[idx / kCP][idx % kCP] = T(0);
  // this wave's block of the state (rows r0.., columns 16 wave..), in registers
  typename M::acc sacc = M::zero();
  __syncthreads();

  for (int c = 0; c < a.n_chunks; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = static_cast<int>(std::min<int64_t>(kC, T_ - t0));
    for (int idx = tid; idx < kC * DM; idx += kNT) {
      const int i = idx / DM, k = idx % DM;
      sX[i][k] = (i < cv && k < din) ? x[(t0 + i) * din + k] : T(0);
    }
    for (int idx = tid; idx < kC * 16; idx += kNT) {
      const int i = idx >> 4, r = idx & 15;
      sG[i][r] = (i < cv && r0 + r < dout) ? g[(t0 + i) * dout + r0 + r] : T(0);
    }
    if (wave == 0) gates_mf<T>(eta, alpha, t0, cv, gt, lane);
    __syncthreads();
    if (st) {  // D_in of this chunk (rows of the tile; sS was published by the barrier)
      T* sp = st + static_cast<int64_t>(c) * dout * din;
      for (int idx = tid; idx < 16 * din; idx += kNT) {
        const int r = idx / din, k = idx % din;
        if (r0 + r < dout) sp[static_cast<int64_t>(r0 + r) * din + k] = sS[r][k];
      }
    }

    // scores: causal blocks (ib >= jb) of the 4 x 4 grid, blocks w, w + 4, w + 8
    const int KX = (din + 3) & ~3;
    if (y) {
      for (int b = wave; b < 10; b += 4) {
        const int ib = static_cast<int>((0x3333222110ull >> (4 * b)) & 0xf);
        const int jb = static_cast<int>((0x3210210100ull >> (4 * b)) & 0xf);
        typename M::acc xx = mm<T>(
            M::zero(), KX, [&](int m, int k) { return sX[ib * 16 + m][k]; },
            [&](int k, int n) { return sX[jb * 16 + n][k]; }, lane);
        const int j = jb * 16 + (lane & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = ib * 16 + M::row(lane, q);
          sA[i][j] = j < i ? xx[q] * xexp2(gt.lq[i] - gt.li[j]) * gt.nb[j] : T(0);
        }
      }
    }
    __syncthreads();

    if (y) {
      // y^T[r][i] for token block `wave`: W0 x_i + sum_j A_ij g_j, and D_in x_i
      const int ib = wave;
      typename M::acc ya = mm<T>(
          M::zero(), KX, [&](int m, int k) { return sW[m][k]; },
          [&](int k, int n) { return sX[ib * 16 + n][k]; }, lane);
      ya = mm<T>(
          ya, kC, [&](int m, int k) { return sG[k][m]; },
          [&](int k, int n) { return sA[ib * 16 + n][k]; }, lane);
      const typename M::acc yb = mm<T>(
          M::zero(), KX, [&](int m, int k) { return sS[m][k]; },
          [&](int k, int n) { return sX[ib * 16 + n][k]; }, lane);
      const int i = ib * 16 + (lane & 15);
      if (i < cv) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = r0 + M::row(lane, q);
          if (r < dout) y[(t0 + i) * dout + r] = ya[q] + gt.eq[i] * yb[q];
        }
      }
    }
    // state update of this wave's block: D[r][k] = Gamma D + sum_j bk_j g_j[r] x_j[k]
    if (wave * 16 < din) {
      const T gam = gt.gam;
#pragma unroll
      for (int q = 0; q < 4; ++q) sacc[q] *= gam;
      sacc = mm<T>(
          sacc, kC, [&](int m, int k) { return sG[k][m] * (gt.nb[k] * gt.e2[k]); },
          [&](int k, int n) { return sX[k][wave * 16 + n]; }, lane);
    }
    __syncthreads();
    if (wave * 16 < din) {
#pragma unroll
      for (int q = 0; q < 4; ++q) sS[M::row(lane, q)][wave * 16 + (lane & 15)] = sacc[q];
    }
    // (the next chunk's loads write other tiles; the barrier after them
    // publishes sS)
  }
}

// ------------------------------------------------------------------ backward
template <typename T, int DM>
struct alignas(16) BwdLds {
  T X[kC][DM + 1], G[kC][DM + 1], DY[kC][DM + 1];
  T S[DM][DM + 1], L[DM][DM + 1], W[DM][DM + 1];
  T P[kC][kCP], Mm[kC][kCP];
  T qq[10][16], kk[10][16];
  T pp[DM / 16][kC], rr[DM / 16][kC], de[DM / 16][kC];
  T c0[4];
  GatesF<T> gt;
};

template <typename T, int DM>
__global__ __launch_bounds__(kNT) void bwd_mf(BwdArgs a) {
  using M = Mx<T>;
  constexpr int NB = DM / 16;             // 16-blocks per side of D
  constexpr int NL = NB * NB;             // blocks of Lam / dW0
  constexpr int LPW = (NL + 3) / 4;       // of which per wave
  __shared__ BwdLds<T, DM> L;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int din = a.d_in, dout = a.d_out;
  const int64_t T_ = a.T;
  const T* x = static_cast<const T*>(a.x) + bh * T_ * din;
  const T* g = static_cast<const T*>(a.g) + bh * T_ * dout;
  const T* dy = static_cast<const T*>(a.dy) + bh * T_ * dout;
  const T* eta = static_cast<const T*>(a.eta) + bh * T_;
  const T* alpha = static_cast<const T*>(a.alpha) + bh * T_;
  const T* W0 = static_cast<const T*>(a.W0) + static_cast<int64_t>(h) * dout * din;
  const T* st = static_cast<const T*>(a.states) + bh * static_cast<int64_t>(a.n_chunks) * dout * din;
  T* dx = static_cast<T*>(a.dx) + bh * T_ * din;
  T* dg = static_cast<T*>(a.dg) + bh * T_ * dout;
  T* deta = static_cast<T*>(a.deta_out) + bh * T_;
  T* dalpha = static_cast<T*>(a.dalpha_out) + bh * T_;
  const int KI = (din + 3) & ~3, KO = (dout + 3) & ~3;

  for (int idx = tid; idx < DM * (DM + 1); idx += kNT) {
    const int r = idx / (DM + 1), k = idx % (DM + 1);
    L.W[r][k] = (r < dout && k < din) ? W0[static_cast<int64_t>(r) * din + k] : T(0);
    L.L[r][k] = T(0);
  }
  for (int idx = tid; idx < kC * kCP; idx += kNT) {
    L.P[idx / kCP][idx % kCP] = T(0);
    L.Mm[idx / kCP][idx % kCP] = T(0);
  }
  // this wave's blocks of Lam and dW0 (block e = wave + 4 j: rows 16 (e / NB), cols 16 (e % NB))
  typename M::acc lam[LPW], dw[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) lam[j] = dw[j] = M::zero();
  __syncthreads();

  for (int c = a.n_chunks - 1; c >= 0; --c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = static_cast<int>(std::min<int64_t>(kC, T_ - t0));
    for (int idx = tid; idx < kC * DM; idx += kNT) {
      const int i = idx / DM, k = idx % DM;
      const bool in = i < cv;
      L.X[i][k] = (in && k < din) ? x[(t0 + i) * din + k] : T(0);
      L.G[i][k] = (in && k < dout) ? g[(t0 + i) * dout + k] : T(0);
      L.DY[i][k] = (in && k < dout) ? dy[(t0 + i) * dout + k] : T(0);
    }
    const T* sp = st + static_cast<int64_t>(c) * dout * din;
    for (int idx = tid; idx < DM * DM; idx += kNT) {
      const int r = idx / DM, k = idx % DM;
      L.S[r][k] = (r < dout && k < din) ? sp[static_cast<int64_t>(r) * din + k] : T(0);
    }
    if (wave == 0) gates_mf<T>(eta, alpha, t0, cv, L.gt, lane);
    __syncthreads();

    // ---- causal blocks: P, M = Be + Be^T and the Be o XX sums (blocks w, w + 4, w + 8)
    for (int b = wave; b < 10; b += 4) {
      const int ib = static_cast<int>((0x3333222110ull >> (4 * b)) & 0xf);
      const int jb = static_cast<int>((0x3210210100ull >> (4 * b)) & 0xf);
      const typename M::acc xx = mm<T>(
          M::zero(), KI, [&](int m, int k) { return L.X[ib * 16 + m][k]; },
          [&](int k, int n) { return L.X[jb * 16 + n][k]; }, lane);
      const typename M::acc be = mm<T>(
          M::zero(), KO, [&](int m, int k) { return L.DY[ib * 16 + m][k]; },
          [&](int k, int n) { return L.G[jb * 16 + n][k]; }, lane);
      const int n = lane & 15, j = jb * 16 + n;
      T zq[4];
      T zcol = T(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = M::row(lane, q), i = ib * 16 + m;
        const bool on = j < i;
        const T e = on ? xexp2(L.gt.lq[i] - L.gt.li[j]) : T(0);
        const T bev = be[q] * e * L.gt.nb[j];
        L.P[i][j] = xx[q] * e;
        // M only where Be lives (j < i) and its mirror: the diagonal stays
        // at its initial zero, and no lane zeroes a mirrored element
        if (on) {
          L.Mm[i][j] = bev;
          L.Mm[j][i] = bev;
        }
        zq[q] = bev * xx[q];
        zcol += zq[q];
      }
      // row sums over the 16 columns n (lanes of equal l / 16), column sums
      // over the 16 rows (q and the four lane groups)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        T v = zq[q];
        for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
        if (n == 0) L.qq[b][M::row(lane, q)] = v;
      }
      zcol += __shfl_xor(zcol, 16, 64);
      zcol += __shfl_xor(zcol, 32, 64);
      if (lane < 16) L.kk[b][n] = zcol;
    }
    // ---- <Lam_out, D_in> over this wave's blocks
    {
      T cp = T(0);
#pragma unroll
      for (int jx = 0; jx < LPW; ++jx) {
        const int e = wave + 4 * jx;
        if (e < NL) {
          const int rb = e / NB, kb = e % NB;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            cp += lam[jx][q] * L.S[rb * 16 + M::row(lane, q)][kb * 16 + (lane & 15)];
        }
      }
      for (int o = 1; o < 64; o <<= 1) cp += __shfl_xor(cp, o, 64);
      if (lane == 0) L.c0[wave] = cp;
    }
    __syncthreads();

    // ---- u (rows r, tokens i) and dx (columns k, tokens i): block e = wave + 4 j of
    // the NB x 4 grid (r or k block e / 4, token block e % 4)
    for (int e = wave; e < NB * 4; e += 4) {
      const int ob = e >> 2, ib = e & 3;
      const int ii = ib * 16 + (lane & 15);
      // u = e2 Lam_out x + P^T dy: pp, dg, deta shares
      const typename M::acc ain = mm<T>(
          M::zero(), KI, [&](int m, int k) { return L.L[ob * 16 + m][k]; },
          [&](int k, int n) { return L.X[ib * 16 + n][k]; }, lane);
      const typename M::acc apd = mm<T>(
          M::zero(), kC, [&](int m, int k) { return L.DY[k][ob * 16 + m]; },
          [&](int k, int n) { return L.P[k][ib * 16 + n]; }, lane);
      T dsum = T(0), psum = T(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = ob * 16 + M::row(lane, q);
        const T u = ain[q] * L.gt.e2[ii] + apd[q];
        const T gv = L.G[ii][r];
        dsum += gv * u;
        psum += gv * ain[q];
        if (ii < cv && r < dout) dg[(t0 + ii) * dout + r] = L.gt.nb[ii] * u;
      }
      dsum += __shfl_xor(dsum, 16, 64);
      dsum += __shfl_xor(dsum, 32, 64);
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      if (lane < 16) {
        L.de[ob][ii] = -dsum;
        L.pp[ob][ii] = psum;
      }
      // dx: W0^T dy + M X (acc), D_in^T dy (t), Lam_out^T g (tl)
      typename M::acc acc = mm<T>(
          M::zero(), KO, [&](int m, int k) { return L.W[k][ob * 16 + m]; },
          [&](int k, int n) { return L.DY[ib * 16 + n][k]; }, lane);
      acc = mm<T>(
          acc, kC, [&](int m, int k) { return L.X[k][ob * 16 + m]; },
          [&](int k, int n) { return L.Mm[ib * 16 + n][k]; }, lane);
      const typename M::acc t = mm<T>(
          M::zero(), KO, [&](int m, int k) { return L.S[k][ob * 16 + m]; },
          [&](int k, int n) { return L.DY[ib * 16 + n][k]; }, lane);
      const typename M::acc tl = mm<T>(
          M::zero(), KO, [&](int m, int k) { return L.L[k][ob * 16 + m]; },
          [&](int k, int n) { return L.G[ib * 16 + n][k]; }, lane);
      T rsum = T(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = ob * 16 + M::row(lane, q);
        rsum += L.X[ii][k] * t[q];
        const T v = acc[q] + L.gt.eq[ii] * t[q] + L.gt.nb[ii] * L.gt.e2[ii] * tl[q];
        if (ii < cv && k < din) dx[(t0 + ii) * din + k] = v;
      }
      rsum += __shfl_xor(rsum, 16, 64);
      rsum += __shfl_xor(rsum, 32, 64);
      if (lane < 16) L.rr[ob][ii] = rsum;
    }
    // ---- Lam <- Gamma Lam + sum_u e(lq_u) dy_u x_u^T, dW0 += sum_u dy_u x_u^T
    {
      const T gam = L.gt.gam;
#pragma unroll
      for (int jx = 0; jx < LPW; ++jx) {
        const int e = wave + 4 * jx;
        if (e < NL) {
          const int rb = e / NB, kb = e % NB;
#pragma unroll
          for (int q = 0; q < 4; ++q) lam[jx][q] *= gam;
          lam[jx] = mm<T>(
              lam[jx], kC, [&](int m, int k) { return L.DY[k][rb * 16 + m] * L.gt.eq[k]; },
              [&](int k, int n) { return L.X[k][kb * 16 + n]; }, lane);
          dw[jx] = mm<T>(
              dw[jx], kC, [&](int m, int k) { return L.DY[k][rb * 16 + m]; },
              [&](int k, int n) { return L.X[k][kb * 16 + n]; }, lane);
        }
      }
    }
    __syncthreads();

    // ---- deta and dalpha of the chunk (wave 0, lane = token)
    if (wave == 0) {
      const int i = lane;
      T pp = T(0), rr = T(0), de = T(0);
#pragma unroll
      for (int ob = 0; ob < NB; ++ob) {
        pp += L.pp[ob][i];
        rr += L.rr[ob][i];
        de += L.de[ob][i];
      }
      T qq = T(0), kk = T(0);
      const int R = i >> 4;
      for (int cc = 0; cc <= R; ++cc) qq += L.qq[R * (R + 1) / 2 + cc][i & 15];
      for (int Rr = R; Rr < 4; ++Rr) kk += L.kk[Rr * (Rr + 1) / 2 + R][i & 15];
      const T c0 = L.c0[0] + L.c0[1] + L.c0[2] + L.c0[3];
      const T al = L.gt.al[i];
      const T s2 = __shfl_up(scan_affine<T>(al, L.gt.nb[i] * pp, lane), 1, 64);
      const T s3 = __shfl_down(suffix_affine<T>(al, rr, lane), 1, 64);
      const T zs = __shfl_down(suffix_add<T>(qq - kk, lane), 1, 64);
      const T s2i = i == 0 ? T(0) : s2;
      const T s3i = i == 63 ? T(0) : s3;
      const T zsi = i == 63 ? T(0) : zs;
      const T e2 = L.gt.e2[i], eq = L.gt.eq[i];
      const T da = e2 * eq * c0 + e2 * s2i + eq * s3i + (zsi - kk) / al;
      if (i < cv) {
        dalpha[t0 + i] = da;
        deta[t0 + i] = de;
      }
    }
    // Lam_in becomes the next chunk's Lam_out (bf16-free: the compute type)
#pragma unroll
    for (int jx = 0; jx < LPW; ++jx) {
      const int e = wave + 4 * jx;
      if (e < NL) {
        const int rb = e / NB, kb = e % NB;
#pragma unroll
        for (int q = 0; q < 4; ++q) L.L[rb * 16 + M::row(lane, q)][kb * 16 + (lane & 15)] = lam[jx][q];
      }
    }
    __syncthreads();
  }
  // dW0 partial of this sequence-head: [d_out][d_in]
  T* pw = static_cast<T*>(a.part_dW0) + bh * static_cast<int64_t>(dout) * din;
#pragma unroll
  for (int jx = 0; jx < LPW; ++jx) {
    const int e = wave + 4 * jx;
    if (e < NL) {
      const int rb = e / NB, kb = e % NB;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = rb * 16 + M::row(lane, q), k = kb * 16 + (lane & 15);
        if (r < dout && k < din) pw[static_cast<int64_t>(r) * din + k] = dw[jx][q];
      }
    }
  }
}

}  // namespace

bool mf_shape_ok(int io, int d_in, int d_out) {
  const int dm = io == IO_F64 ? 32 : io == IO_F32 ? 64 : 0;
  return d_in <= dm && d_out <= dm;
}

hipError_t launch_mf_fwd(int io, const FwdArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B * a.H), static_cast<unsigned>((a.d_out + 15) / 16));
  if (io == IO_F64) {
    hipLaunchKernelGGL((fwd_mf<double, 32>), grid, dim3(kNT), 0, s, a);
  } else {
    if (a.d_in <= 32 && a.d_out <= 32)
      hipLaunchKernelGGL((fwd_mf<float, 32>), grid, dim3(kNT), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_mf<float, 64>), grid, dim3(kNT), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_mf_bwd(int io, const BwdArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B * a.H));
  if (io == IO_F64) {
    hipLaunchKernelGGL((bwd_mf<double, 32>), grid, dim3(kNT), 0, s, a);
  } else {
    if (a.d_in <= 32 && a.d_out <= 32)
      hipLaunchKernelGGL((bwd_mf<float, 32>), grid, dim3(kNT), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_mf<float, 64>), grid, dim3(kNT), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace gls
