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
// inclusive cumsum of log2 alpha, lq_i = l_{i-1}, e(.) = 2^(.), gam = e(l_last)):
//   A_ij  = (x_i . x_j) e(lq_i - l_j)(-eta_j)                    (j < i)
//   y_i   = W0 x_i + e(lq_i) D_in x_i + sum_j A_ij g_j
//   D_out = gam D_in + U,  U = sum_j e(l_last - l_j)(-eta_j) g_j x_j^T
// and, with Lam_out = dL/dD after the chunk,
//   Lam_in = gam Lam_out + V,  V = sum_u e(lq_u) dy_u x_u^T,  dW0 += sum_u dy_u x_u^T
//   u_i   = e(l_last - l_i) Lam_out x_i + sum_{u>i} P_ui dy_u,  P_ui = e(lq_u - l_i)(x_u . x_i)
//   dx_i  = W0^T dy_i + e(lq_i) D_in^T dy_i + sum_j M_ij x_j - eta_i e(l_last - l_i) Lam_out^T g_i
//   dg_i  = -eta_i u_i,  deta_i = -g_i . u_i,  M = Be + Be^T,  Be_ij = e(lq_i - l_j)(-eta_j)(dy_i . g_j)
//   dalpha_i = e(l_last - l_i) e(lq_i) <Lam_out, D_in> + e(l_last - l_i) sum_{j<i} e(lq_i - l_j)(-eta_j) pp_j
//            + e(lq_i) sum_{u>i} e(lq_u - l_i) rr_u + (sum_{u>i} qq_u - sum_{j>=i} kk_j) / alpha_i
// (pp_j = g_j . (Lam_out x_j), rr_u = x_u . (D_in^T dy_u), qq / kk the row /
// column sums of Be o XX).
//
// Only the carries D and Lam chain the chunks, and they are affine in each
// other, so each direction runs in three launches with one work-group per
// (sequence-head, chunk): the chunk's own increment (U, or V and its dW0
// share) from its tokens alone; an element-wise scan of the increments over
// the chunks (D_in of every chunk, Lam_out of every chunk); then every chunk's
// outputs from its carry.  Tiles live in LDS in the compute type with rows
// padded by one element; a 16 x 16 output block takes K / 4 MFMAs.
#include <algorithm>
#include <cstdint>

#include "dev_common.hpp"
#include "internal.hpp"

namespace gls {
namespace {

constexpr int kC = 64;      // tokens per chunk
constexpr int kNT = 256;    // threads of the increment kernels (four waves)
constexpr int kNT8 = 512;   // threads of the output kernels (eight waves)
constexpr int kCP = kC + 1; // padded row of a [64][64] tile
constexpr int kCarryThreads = 256;

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

// c += sum_{k < K} A(m, k) B(k, n) over one 16 x 16 block; fa(m, k) and
// fb(k, n) read the operands (m, n in 0..15).  K is a multiple of 4 known at
// compile time; at step s lane group g = lane / 16 supplies k = g K / 4 + s,
// so that each lane walks one contiguous run of k (with rows padded to an odd
// number of 4-byte words, the 64 lanes of a step read distinct banks).
// Every operand is read before the first MFMA of the block is issued (the
// reads of one block stream in while its MFMAs run in order).
template <typename T, int K, typename FA, typename FB>
__device__ __forceinline__ typename Mx<T>::acc mmk(typename Mx<T>::acc c, FA fa, FB fb, int lane) {
  constexpr int S = K / 4;
  const int i = lane & 15, k0 = (lane >> 4) * S;
  T av[S], bv[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    av[s] = fa(i, k0 + s);
    bv[s] = fb(k0 + s, i);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * S, 0);  // LDS reads
  __builtin_amdgcn_sched_group_barrier(0x002, 2 * S, 0);  // VALU (operand scaling)
  __builtin_amdgcn_sched_group_barrier(0x008, S, 0);      // MFMA
#pragma unroll
  for (int s = 0; s < S; ++s) c = Mx<T>::mma(av[s], bv[s], c);
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

// Gates of a chunk (one wave, lane = token; padding tokens alpha = 1, eta = 0),
// in two steps so that the loads can be issued ahead of the tile loads.
template <typename T>
struct GatesF {
  T lq[kC], li[kC], nb[kC], eq[kC], e2[kC], al[kC];
  T gam;
};
template <typename T>
struct GateIn {
  T al, et;
};
template <typename T>
__device__ __forceinline__ GateIn<T> gate_load(const T* eta, const T* alpha, int64_t t0, int cv,
                                                int lane) {
  GateIn<T> in;
  in.al = lane < cv ? alpha[t0 + lane] : T(1);
  in.et = lane < cv ? eta[t0 + lane] : T(0);
  return in;
}
template <typename T>
__device__ __forceinline__ void gates_mf(const GateIn<T>& in, GatesF<T>& g, int lane) {
  const T l = scan_add<T>(xlog2(in.al), lane);
  const T lq = __shfl_up(l, 1, 64);
  const T lqi = lane == 0 ? T(0) : lq;
  const T llast = __shfl(l, 63, 64);
  g.lq[lane] = lqi;
  g.li[lane] = l;
  g.nb[lane] = -in.et;
  g.eq[lane] = xexp2(lqi);
  g.e2[lane] = xexp2(llast - l);
  g.al[lane] = in.al;
  if (lane == 0) g.gam = xexp2(llast);
}

// A [ROWS][DM] tile of a row-major source (row stride ld; rows >= nr or
// columns >= nc read as zero), moved into LDS rows padded to DM + 1 by NT
// threads in two steps: fetch() issues the thread's global loads into
// registers, store() writes them to LDS, so that the loads of several tiles
// are in flight together.  Each thread moves 16-byte pieces of rows: FULL
// (every tile of the launch is full width, nc = ld = DM, so the source rows
// are the tile's rows and 16-byte aligned) with one load per piece, otherwise
// element by element.  Loads are unconditional (an address inside the tile
// stands in for a piece outside it, whose value is then dropped), so that no
// branch separates a load from the next.
template <typename T, int DM, int ROWS, int NT, bool FULL>
struct Tile {
  static constexpr int V = 16 / sizeof(T), RV = DM / V, TOT = ROWS * RV;
  static constexpr int N = (TOT + NT - 1) / NT;
  typedef T vec_t __attribute__((ext_vector_type(V)));
  vec_t v[N];

  // nr, nc >= 1
  __device__ __forceinline__ void fetch(const T* src, int64_t ld, int nr, int nc, int tid) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = tid + j * NT, r = idx / RV, k = (idx % RV) * V;
      const bool in = idx < TOT && r < nr;
      if constexpr (FULL) {
        const vec_t x = *reinterpret_cast<const vec_t*>(src + (in ? r * ld + k : 0));
#pragma unroll
        for (int e = 0; e < V; ++e) v[j][e] = in ? x[e] : T(0);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const bool ok = in && k + e < nc;
          const T x = src[ok ? r * ld + k + e : 0];
          v[j][e] = ok ? x : T(0);
        }
      }
    }
  }
  __device__ __forceinline__ void store(T (*dst)[DM + 1], int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = tid + j * NT;
      if (idx < TOT) {
#pragma unroll
        for (int e = 0; e < V; ++e) dst[idx / RV][(idx % RV) * V + e] = v[j][e];
      }
    }
  }
};

// ------------------------------------------------- chunk increments (pass 1)
// Forward: U of chunk c into the state slot c + 1 (c < n_chunks - 1) and gam
// of the chunk.  Work-group = (sequence-head, chunk), blockIdx.x = bh n + c.
template <typename T, int DM, bool FULL>
__global__ __launch_bounds__(kNT) void fwd_inc(FwdArgs a, int n_launch) {
  using M = Mx<T>;
  constexpr int DP = DM + 1, NB = DM / 16, NL = NB * NB;
  __shared__ T sG[kC][DP], sX[kC][DP];
  __shared__ T sw[kC];
  __shared__ T sgam;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bh = blockIdx.x / n_launch;
  const int c = static_cast<int>(blockIdx.x % n_launch);
  const int n = a.n_chunks, din = a.d_in, dout = a.d_out;
  const int64_t t0 = static_cast<int64_t>(c) * kC;
  const int cv = static_cast<int>(std::min<int64_t>(kC, a.T - t0));
  GateIn<T> gin{};
  if (wave == 0)
    gin = gate_load<T>(static_cast<const T*>(a.eta) + bh * a.T,
                       static_cast<const T*>(a.alpha) + bh * a.T, t0, cv, lane);
  Tile<T, DM, kC, kNT, FULL> tg, tx;
  tg.fetch(static_cast<const T*>(a.g) + (bh * a.T + t0) * dout, dout, cv, dout, tid);
  tx.fetch(static_cast<const T*>(a.x) + (bh * a.T + t0) * din, din, cv, din, tid);
  if (wave == 0) {
    const T l = scan_add<T>(xlog2(gin.al), lane);
    const T llast = __shfl(l, 63, 64);
    sw[lane] = -gin.et * xexp2(llast - l);
    if (lane == 0) sgam = xexp2(llast);
  }
  tg.store(sG, tid);
  tx.store(sX, tid);
  __syncthreads();
  T* out = static_cast<T*>(a.states) + (bh * n + c + 1) * static_cast<int64_t>(dout) * din;
#pragma unroll
  for (int e = wave; e < NL; e += 4) {
    const int rb = e / NB, kb = e % NB;
    const typename M::acc u = mmk<T, kC>(
        M::zero(), [&](int m, int k) { return sG[k][rb * 16 + m] * sw[k]; },
        [&](int k, int nn) { return sX[k][kb * 16 + nn]; }, lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = rb * 16 + M::row(lane, q), k = kb * 16 + (lane & 15);
      if (r < dout && k < din) out[r * din + k] = u[q];
    }
  }
  if (tid == 0) static_cast<T*>(a.mf_gam)[bh * n + c] = sgam;
}

// Backward: V of chunk c into the adjoint slot c - 1 (c >= 1), the chunk's
// dW0 share into part_dW0[c][bh], and gam of the chunk.
template <typename T, int DM, bool FULL>
__global__ __launch_bounds__(kNT) void bwd_inc(BwdArgs a) {
  using M = Mx<T>;
  constexpr int DP = DM + 1, NB = DM / 16, NL = NB * NB;
  __shared__ T sD[kC][DP], sX[kC][DP];
  __shared__ T sw[kC];
  __shared__ T sgam;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.n_chunks, din = a.d_in, dout = a.d_out;
  const int64_t bh = blockIdx.x / n;
  const int c = static_cast<int>(blockIdx.x % n);
  const int64_t BH = a.B * a.H;
  const int64_t dd = static_cast<int64_t>(dout) * din;
  const int64_t t0 = static_cast<int64_t>(c) * kC;
  const int cv = static_cast<int>(std::min<int64_t>(kC, a.T - t0));
  T al = T(1);
  if (wave == 0 && lane < cv) al = static_cast<const T*>(a.alpha)[bh * a.T + t0 + lane];
  Tile<T, DM, kC, kNT, FULL> td, tx;
  td.fetch(static_cast<const T*>(a.dy) + (bh * a.T + t0) * dout, dout, cv, dout, tid);
  tx.fetch(static_cast<const T*>(a.x) + (bh * a.T + t0) * din, din, cv, din, tid);
  if (wave == 0) {
    const T l = scan_add<T>(xlog2(al), lane);
    const T lq = __shfl_up(l, 1, 64);
    const T llast = __shfl(l, 63, 64);
    sw[lane] = lane == 0 ? T(1) : xexp2(lq);
    if (lane == 0) sgam = xexp2(llast);
  }
  td.store(sD, tid);
  tx.store(sX, tid);
  __syncthreads();
  T* pw = static_cast<T*>(a.part_dW0) + (static_cast<int64_t>(c) * BH + bh) * dd;
  T* pv = c > 0 ? static_cast<T*>(a.mf_lam) + (bh * n + c - 1) * dd : nullptr;
#pragma unroll
  for (int e = wave; e < NL; e += 4) {
    const int rb = e / NB, kb = e % NB;
    const int i = lane & 15, k0 = (lane >> 4) * (kC / 4);
    typename M::acc w = M::zero(), v = M::zero();
#pragma unroll
    for (int s = 0; s < kC / 4; ++s) {
      const int k = k0 + s;
      const T av = sD[k][rb * 16 + i], bv = sX[k][kb * 16 + i];
      w = M::mma(av, bv, w);
      v = M::mma(av * sw[k], bv, v);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = rb * 16 + M::row(lane, q), k = kb * 16 + i;
      if (r < dout && k < din) {
        pw[r * din + k] = w[q];
        if (pv) pv[r * din + k] = v[q];
      }
    }
  }
  if (tid == 0) static_cast<T*>(a.mf_gam)[bh * n + c] = sgam;
}

// ---------------------------------------------- carries over chunks (pass 2)
// buf [BH][n][dd]: on entry slot c holds the increment arriving at chunk c
// from the chunk visited before it (forward: from c - 1, reverse: from c + 1;
// the slot of the chunk visited first is ignored); on exit the carry at chunk
// c: zero for the first, then carry = gam[prev] carry + increment.
template <typename T>
__global__ __launch_bounds__(kCarryThreads) void mf_carry(T* buf, const T* gam, int n, int dd,
                                                          int n_eb, int reverse) {
  const int64_t bh = blockIdx.x / n_eb;
  const int e = static_cast<int>(blockIdx.x % n_eb) * kCarryThreads + threadIdx.x;
  if (e >= dd) return;
  T* p = buf + bh * n * static_cast<int64_t>(dd) + e;
  const T* gm = gam + bh * n;
  // chunks in groups of sixteen: the group's loads are issued together
  constexpr int kG = 16;
  T carry = T(0);
  for (int k0 = 0; k0 < n; k0 += kG) {
    T inc[kG], dec[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int k = k0 + j;
      const int c = reverse ? n - 1 - k : k;
      const int prev = reverse ? c + 1 : c - 1;
      const bool use = k >= 1 && k < n;
      inc[j] = use ? p[static_cast<int64_t>(c) * dd] : T(0);
      dec[j] = use ? gm[prev] : T(0);
    }
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int k = k0 + j;
      if (k >= n) break;
      const int c = reverse ? n - 1 - k : k;
      carry = dec[j] * carry + inc[j];
      p[static_cast<int64_t>(c) * dd] = carry;
    }
  }
}

// ------------------------------------------------------- forward (pass 3)
// y of chunk c from D_in = state slot c.  blockIdx.x = bh n + c.
template <typename T, int DM>
struct alignas(16) FwdLds {
  T X[kC][DM + 1], G[kC][DM + 1], S[DM][DM + 1], W[DM][DM + 1];
  T A[kC][kCP];
  GatesF<T> gt;
};

template <typename T, int DM, bool FULL>
__global__ __launch_bounds__(kNT8) void fwd_chunk(FwdArgs a) {
  using M = Mx<T>;
  constexpr int NB = DM / 16;
  __shared__ FwdLds<T, DM> L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.n_chunks, din = a.d_in, dout = a.d_out;
  const int64_t bh = blockIdx.x / n;
  const int c = static_cast<int>(blockIdx.x % n);
  const int h = static_cast<int>(bh % a.H);
  const int64_t dd = static_cast<int64_t>(dout) * din;
  const int64_t t0 = static_cast<int64_t>(c) * kC;
  const int cv = static_cast<int>(std::min<int64_t>(kC, a.T - t0));
  // the six blocks above the diagonal of A: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
  for (int idx = tid; idx < 6 * 256; idx += kNT8) {
    const int u = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
    const int ib = static_cast<int>((0x211000u >> (4 * u)) & 0xf);
    const int jb = static_cast<int>((0x332321u >> (4 * u)) & 0xf);
    L.A[ib * 16 + r][jb * 16 + cc] = T(0);
  }
  GateIn<T> gin{};
  if (wave == 0)
    gin = gate_load<T>(static_cast<const T*>(a.eta) + bh * a.T,
                       static_cast<const T*>(a.alpha) + bh * a.T, t0, cv, lane);
  Tile<T, DM, kC, kNT8, FULL> tx, tg;
  Tile<T, DM, DM, kNT8, FULL> ts, tw;
  tx.fetch(static_cast<const T*>(a.x) + (bh * a.T + t0) * din, din, cv, din, tid);
  tg.fetch(static_cast<const T*>(a.g) + (bh * a.T + t0) * dout, dout, cv, dout, tid);
  ts.fetch(static_cast<const T*>(a.states) + (bh * n + c) * dd, din, dout, din, tid);
  tw.fetch(static_cast<const T*>(a.W0) + h * dd, din, dout, din, tid);
  if (wave == 0) gates_mf<T>(gin, L.gt, lane);
  tx.store(L.X, tid);
  tg.store(L.G, tid);
  ts.store(L.S, tid);
  tw.store(L.W, tid);
  __syncthreads();

  // scores: causal blocks (ib >= jb) of the 4 x 4 token grid, blocks w and
  // w + 8 of the ten (the six above the diagonal were zeroed)
  for (int b = wave; b < 10; b += 8) {
    const int ib = static_cast<int>((0x3333222110ull >> (4 * b)) & 0xf);
    const int jb = static_cast<int>((0x3210210100ull >> (4 * b)) & 0xf);
    const int j = jb * 16 + (lane & 15);
    const typename M::acc xx = mmk<T, DM>(
        M::zero(), [&](int m, int k) { return L.X[ib * 16 + m][k]; },
        [&](int k, int nn) { return L.X[jb * 16 + nn][k]; }, lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = ib * 16 + M::row(lane, q);
      L.A[i][j] = j < i ? xx[q] * xexp2(L.gt.lq[i] - L.gt.li[j]) * L.gt.nb[j] : T(0);
    }
  }
  __syncthreads();

  // y^T[r][i]: tokens ib = wave % 4, rows rb = wave / 4 + 2 j
  T* y = static_cast<T*>(a.y) + (bh * a.T + t0) * dout;
  const int ib = wave & 3, i = ib * 16 + (lane & 15);
  const T eqi = L.gt.eq[i];
#pragma unroll
  for (int jr = 0; jr < NB / 2; ++jr) {
    const int rb = (wave >> 2) + 2 * jr;
    typename M::acc acc = mmk<T, DM>(
        M::zero(), [&](int m, int k) { return L.W[rb * 16 + m][k]; },
        [&](int k, int nn) { return L.X[ib * 16 + nn][k]; }, lane);
    acc = mmk<T, DM>(
        acc, [&](int m, int k) { return L.S[rb * 16 + m][k]; },
        [&](int k, int nn) { return L.X[ib * 16 + nn][k] * eqi; }, lane);
    acc = mmk<T, kC>(
        acc, [&](int m, int k) { return L.G[k][rb * 16 + m]; },
        [&](int k, int nn) { return L.A[ib * 16 + nn][k]; }, lane);
    if (i < cv) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = rb * 16 + M::row(lane, q);
        if (r < dout) y[static_cast<int64_t>(i) * dout + r] = acc[q];
      }
    }
  }
}

// ------------------------------------------------------ backward (pass 3)
// dx, dg, deta, dalpha of chunk c from D_in = state slot c and Lam_out =
// adjoint slot c.  blockIdx.x = bh n + c.
template <typename T, int DM>
struct alignas(16) BwdLds {
  T X[kC][DM + 1], G[kC][DM + 1], DY[kC][DM + 1];
  T S[DM][DM + 1], L[DM][DM + 1], W[DM][DM + 1];
  T P[kC][kCP], Mm[kC][kCP];
  T qq[10][16], kk[10][16];
  T pp[DM / 16][kC], rr[DM / 16][kC], de[DM / 16][kC];
  T c0[8];
  GatesF<T> gt;
};

template <typename T, int DM, bool FULL>
__global__ __launch_bounds__(kNT8) void bwd_chunk(BwdArgs a) {
  using M = Mx<T>;
  constexpr int NB = DM / 16;  // 16-blocks per side of D
  __shared__ BwdLds<T, DM> L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.n_chunks, din = a.d_in, dout = a.d_out;
  const int64_t bh = blockIdx.x / n;
  const int c = static_cast<int>(blockIdx.x % n);
  const int h = static_cast<int>(bh % a.H);
  const int64_t dd = static_cast<int64_t>(dout) * din;
  const int64_t t0 = static_cast<int64_t>(c) * kC;
  const int cv = static_cast<int>(std::min<int64_t>(kC, a.T - t0));

  for (int idx = tid; idx < kC * kCP; idx += kNT8) {
    L.P[idx / kCP][idx % kCP] = T(0);
    L.Mm[idx / kCP][idx % kCP] = T(0);
  }
  GateIn<T> gin{};
  if (wave == 0)
    gin = gate_load<T>(static_cast<const T*>(a.eta) + bh * a.T,
                       static_cast<const T*>(a.alpha) + bh * a.T, t0, cv, lane);
  Tile<T, DM, kC, kNT8, FULL> tx, tg, td;
  Tile<T, DM, DM, kNT8, FULL> ts, tl, tw;
  tx.fetch(static_cast<const T*>(a.x) + (bh * a.T + t0) * din, din, cv, din, tid);
  tg.fetch(static_cast<const T*>(a.g) + (bh * a.T + t0) * dout, dout, cv, dout, tid);
  td.fetch(static_cast<const T*>(a.dy) + (bh * a.T + t0) * dout, dout, cv, dout, tid);
  ts.fetch(static_cast<const T*>(a.states) + (bh * n + c) * dd, din, dout, din, tid);
  tl.fetch(static_cast<const T*>(a.mf_lam) + (bh * n + c) * dd, din, dout, din, tid);
  tw.fetch(static_cast<const T*>(a.W0) + h * dd, din, dout, din, tid);
  if (wave == 0) gates_mf<T>(gin, L.gt, lane);
  tx.store(L.X, tid);
  tg.store(L.G, tid);
  td.store(L.DY, tid);
  ts.store(L.S, tid);
  tl.store(L.L, tid);
  tw.store(L.W, tid);
  __syncthreads();

  // ---- causal blocks: P, M = Be + Be^T and the Be o XX sums (blocks w, w + 8)
  for (int b = wave; b < 10; b += 8) {
    const int ib = static_cast<int>((0x3333222110ull >> (4 * b)) & 0xf);
    const int jb = static_cast<int>((0x3210210100ull >> (4 * b)) & 0xf);
    const typename M::acc xx = mmk<T, DM>(
        M::zero(), [&](int m, int k) { return L.X[ib * 16 + m][k]; },
        [&](int k, int nn) { return L.X[jb * 16 + nn][k]; }, lane);
    const typename M::acc be = mmk<T, DM>(
        M::zero(), [&](int m, int k) { return L.DY[ib * 16 + m][k]; },
        [&](int k, int nn) { return L.G[jb * 16 + nn][k]; }, lane);
    const int nn = lane & 15, j = jb * 16 + nn;
    T zq[4];
    T zcol = T(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = M::row(lane, q), i = ib * 16 + m;
      const bool on = j < i;
      const T e = on ? xexp2(L.gt.lq[i] - L.gt.li[j]) : T(0);
      const T bev = be[q] * e * L.gt.nb[j];
      L.P[i][j] = xx[q] * e;
      // M only where Be lives (j < i) and its mirror: the diagonal stays at
      // its initial zero, and no lane zeroes a mirrored element
      if (on) {
        L.Mm[i][j] = bev;
        L.Mm[j][i] = bev;
      }
      zq[q] = bev * xx[q];
      zcol += zq[q];
    }
    // row sums over the 16 columns (lanes of equal l / 16), column sums over
    // the 16 rows (q and the four lane groups)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      T v = zq[q];
      for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
      if (nn == 0) L.qq[b][M::row(lane, q)] = v;
    }
    zcol += __shfl_xor(zcol, 16, 64);
    zcol += __shfl_xor(zcol, 32, 64);
    if (lane < 16) L.kk[b][nn] = zcol;
  }
  // ---- <Lam_out, D_in>
  {
    T cp = T(0);
#pragma unroll
    for (int j = 0; j < DM * DM / kNT8; ++j) {
      const int idx = tid + j * kNT8;
      cp += L.L[idx / DM][idx % DM] * L.S[idx / DM][idx % DM];
    }
    for (int o = 1; o < 64; o <<= 1) cp += __shfl_xor(cp, o, 64);
    if (lane == 0) L.c0[wave] = cp;
  }
  __syncthreads();

  // ---- u (rows r, tokens i) and dx (columns k, tokens i): token block
  // ib = wave % 4, r or k block ob = wave / 4 + 2 j
  T* dx = static_cast<T*>(a.dx) + (bh * a.T + t0) * din;
  T* dg = static_cast<T*>(a.dg) + (bh * a.T + t0) * dout;
  const int ib = wave & 3, ii = ib * 16 + (lane & 15);
  const T e2i = L.gt.e2[ii], eqi = L.gt.eq[ii], nbi = L.gt.nb[ii];
#pragma unroll
  for (int jo = 0; jo < NB / 2; ++jo) {
    const int ob = (wave >> 2) + 2 * jo;
    // u = e2 Lam_out x + P^T dy: pp, dg, deta shares
    const typename M::acc ain = mmk<T, DM>(
        M::zero(), [&](int m, int k) { return L.L[ob * 16 + m][k]; },
        [&](int k, int nn) { return L.X[ib * 16 + nn][k]; }, lane);
    const typename M::acc apd = mmk<T, kC>(
        M::zero(), [&](int m, int k) { return L.DY[k][ob * 16 + m]; },
        [&](int k, int nn) { return L.P[k][ib * 16 + nn]; }, lane);
    T dsum = T(0), psum = T(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = ob * 16 + M::row(lane, q);
      const T u = ain[q] * e2i + apd[q];
      const T gv = L.G[ii][r];
      dsum += gv * u;
      psum += gv * ain[q];
      if (ii < cv && r < dout) dg[static_cast<int64_t>(ii) * dout + r] = nbi * u;
    }
    dsum += __shfl_xor(dsum, 16, 64);
    dsum += __shfl_xor(dsum, 32, 64);
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    if (lane < 16) {
      L.de[ob][ii] = -dsum;
      L.pp[ob][ii] = psum;
    }
    // dx: W0^T dy + M X + e(lq) D_in^T dy + (-eta e2) Lam_out^T g, with
    // D_in^T dy (t) kept apart for rr
    typename M::acc acc = mmk<T, DM>(
        M::zero(), [&](int m, int k) { return L.W[k][ob * 16 + m]; },
        [&](int k, int nn) { return L.DY[ib * 16 + nn][k]; }, lane);
    acc = mmk<T, kC>(
        acc, [&](int m, int k) { return L.X[k][ob * 16 + m]; },
        [&](int k, int nn) { return L.Mm[ib * 16 + nn][k]; }, lane);
    const T wl = nbi * e2i;
    acc = mmk<T, DM>(
        acc, [&](int m, int k) { return L.L[k][ob * 16 + m]; },
        [&](int k, int nn) { return L.G[ib * 16 + nn][k] * wl; }, lane);
    const typename M::acc t = mmk<T, DM>(
        M::zero(), [&](int m, int k) { return L.S[k][ob * 16 + m]; },
        [&](int k, int nn) { return L.DY[ib * 16 + nn][k]; }, lane);
    T rsum = T(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = ob * 16 + M::row(lane, q);
      rsum += L.X[ii][k] * t[q];
      if (ii < cv && k < din) dx[static_cast<int64_t>(ii) * din + k] = acc[q] + eqi * t[q];
    }
    rsum += __shfl_xor(rsum, 16, 64);
    rsum += __shfl_xor(rsum, 32, 64);
    if (lane < 16) L.rr[ob][ii] = rsum;
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
    T c0 = T(0);
#pragma unroll
    for (int w = 0; w < 8; ++w) c0 += L.c0[w];
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
      static_cast<T*>(a.dalpha_out)[bh * a.T + t0 + i] = da;
      static_cast<T*>(a.deta_out)[bh * a.T + t0 + i] = de;
    }
  }
}

template <typename T>
hipError_t carry(T* buf, const T* gam, int64_t BH, int n, int dd, bool reverse, hipStream_t s) {
  const int n_eb = (dd + kCarryThreads - 1) / kCarryThreads;
  hipLaunchKernelGGL(mf_carry<T>, dim3(static_cast<unsigned>(BH * n_eb)), dim3(kCarryThreads), 0,
                     s, buf, gam, n, dd, n_eb, reverse ? 1 : 0);
  return hipGetLastError();
}

template <typename T, int DM, bool FULL>
hipError_t fwd_passes(const FwdArgs& a, hipStream_t s) {
  const int64_t BH = a.B * a.H;
  const int n = a.n_chunks;
  if (n > 1)
    hipLaunchKernelGGL((fwd_inc<T, DM, FULL>), dim3(static_cast<unsigned>(BH * (n - 1))), dim3(kNT),
                       0, s, a, n - 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = carry<T>(static_cast<T*>(a.states), static_cast<const T*>(a.mf_gam), BH, n,
               a.d_in * a.d_out, false, s);
  if (e != hipSuccess || !a.y) return e;
  hipLaunchKernelGGL((fwd_chunk<T, DM, FULL>), dim3(static_cast<unsigned>(BH * n)), dim3(kNT8), 0,
                     s, a);
  return hipGetLastError();
}

template <typename T, int DM, bool FULL>
hipError_t bwd_passes(const BwdArgs& a, hipStream_t s) {
  const int64_t BH = a.B * a.H;
  const int n = a.n_chunks;
  hipLaunchKernelGGL((bwd_inc<T, DM, FULL>), dim3(static_cast<unsigned>(BH * n)), dim3(kNT), 0, s,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = carry<T>(static_cast<T*>(a.mf_lam), static_cast<const T*>(a.mf_gam), BH, n,
               a.d_in * a.d_out, true, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_chunk<T, DM, FULL>), dim3(static_cast<unsigned>(BH * n)), dim3(kNT8), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

bool mf_shape_ok(int io, int d_in, int d_out) {
  const int dm = io == IO_F64 ? 32 : io == IO_F32 ? 64 : 0;
  return d_in <= dm && d_out <= dm;
}

hipError_t launch_mf_fwd(int io, const FwdArgs& a, hipStream_t s) {
  const bool full32 = a.d_in == 32 && a.d_out == 32, full64 = a.d_in == 64 && a.d_out == 64;
  if (io == IO_F64)
    return full32 ? fwd_passes<double, 32, true>(a, s) : fwd_passes<double, 32, false>(a, s);
  if (a.d_in <= 32 && a.d_out <= 32)
    return full32 ? fwd_passes<float, 32, true>(a, s) : fwd_passes<float, 32, false>(a, s);
  return full64 ? fwd_passes<float, 64, true>(a, s) : fwd_passes<float, 64, false>(a, s);
}

hipError_t launch_mf_bwd(int io, const BwdArgs& a, hipStream_t s) {
  const bool full32 = a.d_in == 32 && a.d_out == 32, full64 = a.d_in == 64 && a.d_out == 64;
  if (io == IO_F64)
    return full32 ? bwd_passes<double, 32, true>(a, s) : bwd_passes<double, 32, false>(a, s);
  if (a.d_in <= 32 && a.d_out <= 32)
    return full32 ? bwd_passes<float, 32, true>(a, s) : bwd_passes<float, 32, false>(a, s);
  return full64 ? bwd_passes<float, 64, true>(a, s) : bwd_passes<float, 64, false>(a, s);
}

}  // namespace gls
