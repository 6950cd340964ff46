// k_qkv.hip -- the scan with a read vector q_t and a write key k_t of their
// own (any io dtype, 1 <= dk, dv <= 128):
//
//   y_t = (W0' + D_t) q_t,   D_{t+1} = alpha_t D_t - eta_t v_t k_t^T,  D_0 = 0
//
// With q = k = x and v = g it is the forward scan.  Two readings of the pages
// need it with q != k:
//  - the transpose read W_{t-1}^T u_t that carries a hidden costate back
//    through an adapted layer ("Parallelize the Training, Keep the Learning
//    Serial", cognaptus.com, section "The synthetic test checks the mechanism,
//    not model quality"): since D_t^T u = sum_s (decay)(-eta_s) x_s (g_s . u),
//    it is this scan with q = u, k = g, v = x and W0' = W0^T;
//  - a centered write key x_bar_t != x_t (section "Once the gradient signals
//    are known, the weight trajectory becomes parallelizable", where the
//    update is centered): q = x, k = x_bar, v = g.
//
// Tokens run in order (exactly the serial recurrence), the parallelism is
// over sequence-heads and rows: a work-group of four waves owns 16 rows of D
// (D is dv x dk), a wave 4 rows, each row split over the 16 lanes of a DPP
// row, which hold MC consecutive columns of D and of W0' in registers (MC = 4
// for dk <= 64, else 8; columns past dk are zero).  Per token a lane reads its
// q and k columns from LDS, the row's readout meets by four in-register DPP
// moves, and the lane updates its columns of D.
// The q, k, v, eta and alpha of a chunk of TC tokens are staged through LDS,
// the next chunk's loads in flight in registers.  Bound by the vector ALU
// (4 dk dv flops per token and head).
#include <algorithm>
#include <cstddef>

#include "dev_common.hpp"
#include "internal.hpp"

namespace gls {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesRow = 16;                        // lanes per row of D (one DPP row)
constexpr int kRowsWG = kThreads / kLanesRow;        // rows of D per work-group

template <typename S> struct QkvTile;
template <> struct QkvTile<float> { static constexpr int TC = 32; };   // tokens per chunk
template <> struct QkvTile<double> { static constexpr int TC = 16; };

template <int MC>
__device__ __forceinline__ void lds_vec(const float* p, float (&v)[MC]) {
#pragma unroll
  for (int i = 0; i < MC / 4; ++i) {
    const float4 t = reinterpret_cast<const float4*>(p)[i];
    v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
  }
}
template <int MC>
__device__ __forceinline__ void lds_vec(const double* p, double (&v)[MC]) {
#pragma unroll
  for (int i = 0; i < MC / 2; ++i) {
    const double2 t = reinterpret_cast<const double2*>(p)[i];
    v[2 * i] = t.x; v[2 * i + 1] = t.y;
  }
}

// Sum over the 16 lanes of a DPP row, in registers: quad permutations
// [1,0,3,2] and [2,3,0,1] (quad sums), the half-row mirror (lane i <- 7 - i
// within 8: the other quad), the row mirror (lane i <- 15 - i: the other 8).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  const int2 h = __builtin_bit_cast(int2, v);
  int2 o;
  o.x = __builtin_amdgcn_mov_dpp(h.x, CTRL, 0xF, 0xF, true);
  o.y = __builtin_amdgcn_mov_dpp(h.y, CTRL, 0xF, 0xF, true);
  return __builtin_bit_cast(double, o);
}
template <typename S>
__device__ __forceinline__ S row16_sum(S v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

template <typename IO, typename S, int MC, bool W0T>
__global__ __launch_bounds__(kThreads) void qkv_fwd_k(QkvArgs a) {
  constexpr int TC = QkvTile<S>::TC;
  constexpr int KP = kLanesRow * MC;               // padded columns
  constexpr int QPER = TC * KP / kThreads;         // q (and k) values staged per thread
  constexpr int VPER = TC * kRowsWG / kThreads;    // v values staged per thread
  __shared__ __attribute__((aligned(16))) S qs[TC][KP];
  __shared__ __attribute__((aligned(16))) S ks[TC][KP];
  __shared__ S vs[TC][kRowsWG], ys[TC][kRowsWG], es[TC], as[TC];

  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int r0 = blockIdx.y * kRowsWG;
  const int dk = a.dk, dv = a.dv;
  const int64_t T = a.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = wave * (64 / kLanesRow) + lane / kLanesRow;  // row within the work-group
  const int cg = lane % kLanesRow, cbase = cg * MC;
  const int r = min(r0 + rl, dv - 1);      // rows past dv compute row dv-1 and store nothing
  const IO* q = static_cast<const IO*>(a.q) + bh * T * dk;
  const IO* k = static_cast<const IO*>(a.k) + bh * T * dk;
  const IO* v = static_cast<const IO*>(a.v) + bh * T * dv;
  const S* eta = static_cast<const S*>(a.eta) + bh * T;
  const S* alpha = static_cast<const S*>(a.alpha) + bh * T;
  IO* y = static_cast<IO*>(a.y) + bh * T * dv;
  const IO* w0 = static_cast<const IO*>(a.W0) + static_cast<int64_t>(h) * dv * dk;

  S w0r[MC], dr[MC];
#pragma unroll
  for (int j = 0; j < MC; ++j) {
    const int c = cbase + j;
    const int cc = min(c, dk - 1);
    const S wv = W0T ? load_as<S>(w0, static_cast<int64_t>(cc) * dv + r)
                     : load_as<S>(w0, static_cast<int64_t>(r) * dk + cc);
    w0r[j] = c < dk ? wv : S(0);
    dr[j] = S(0);
  }

  S rq[QPER], rk[QPER], rv[VPER], re = S(0), ra = S(1);
  // loads of the chunk [t0, t0 + n): positions past n repeat token t0 + n - 1
  const auto fetch = [&](int64_t t0, int n) {
#pragma unroll
    for (int i = 0; i < QPER; ++i) {
      const int idx = tid + i * kThreads, j = idx / KP, c = idx % KP;
      const int64_t o = (t0 + min(j, n - 1)) * dk + min(c, dk - 1);
      rq[i] = load_as<S>(q, o);
      rk[i] = load_as<S>(k, o);
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int idx = tid + i * kThreads, j = idx / kRowsWG, rr = idx % kRowsWG;
      rv[i] = load_as<S>(v, (t0 + min(j, n - 1)) * dv + min(r0 + rr, dv - 1));
    }
    if (tid < TC) {
      re = eta[t0 + min(tid, n - 1)];
      ra = alpha[t0 + min(tid, n - 1)];
    }
  };
  // registers -> LDS; key columns past dk are zero (so D stays zero there),
  // padding tokens get eta = 0, alpha = 1 (they leave D unchanged)
  const auto stash = [&](int n) {
#pragma unroll
    for (int i = 0; i < QPER; ++i) {
      const int idx = tid + i * kThreads, j = idx / KP, c = idx % KP;
      qs[j][c] = rq[i];
      ks[j][c] = c < dk ? rk[i] : S(0);
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int idx = tid + i * kThreads;
      vs[idx / kRowsWG][idx % kRowsWG] = rv[i];
    }
    if (tid < TC) {
      es[tid] = tid < n ? re : S(0);
      as[tid] = tid < n ? ra : S(1);
    }
  };

  if (T > 0) fetch(0, static_cast<int>(std::min<int64_t>(TC, T)));
  for (int64_t t0 = 0; t0 < T; t0 += TC) {
    const int n = static_cast<int>(std::min<int64_t>(TC, T - t0));
    __syncthreads();  // the previous chunk's LDS reads (and y writes out) are done
    stash(n);
    __syncthreads();
    const int64_t t1 = t0 + TC;
    if (t1 < T) fetch(t1, static_cast<int>(std::min<int64_t>(TC, T - t1)));
#pragma unroll 2
    for (int t = 0; t < TC; ++t) {
      S qv[MC], kv[MC];
      lds_vec<MC>(&qs[t][cbase], qv);
      lds_vec<MC>(&ks[t][cbase], kv);
      S pa[4] = {S(0), S(0), S(0), S(0)};  // four independent chains
#pragma unroll
      for (int j = 0; j < MC; ++j) pa[j & 3] += (w0r[j] + dr[j]) * qv[j];
      const S part = row16_sum((pa[0] + pa[1]) + (pa[2] + pa[3]));
      if (cg == 0) ys[t][rl] = part;
      const S ne = -es[t] * vs[t][rl];
      const S al = as[t];
#pragma unroll
      for (int j = 0; j < MC; ++j) dr[j] = al * dr[j] + ne * kv[j];
    }
    __syncthreads();  // the chunk's readouts are in LDS
    for (int idx = tid; idx < n * kRowsWG; idx += kThreads) {
      const int j = idx / kRowsWG, rr = idx % kRowsWG;
      if (r0 + rr < dv) store_from(y, (t0 + j) * dv + r0 + rr, ys[j][rr]);
    }
  }
}

template <typename IO, typename S>
hipError_t qkv_t(const QkvArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B * a.H), (a.dv + kRowsWG - 1) / kRowsWG);
  const dim3 block(kThreads);
  if (a.dk <= 64) {
    if (a.w0_transposed)
      hipLaunchKernelGGL((qkv_fwd_k<IO, S, 4, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((qkv_fwd_k<IO, S, 4, false>), grid, block, 0, s, a);
  } else {
    if (a.w0_transposed)
      hipLaunchKernelGGL((qkv_fwd_k<IO, S, 8, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((qkv_fwd_k<IO, S, 8, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_fwd(int io, const QkvArgs& a, hipStream_t s) {
  if (a.B * a.H * a.T == 0) return hipSuccess;
  if (io == IO_F64) return qkv_t<double, double>(a, s);
  if (io == IO_F32) return qkv_t<float, float>(a, s);
  return qkv_t<bf16, float>(a, s);
}

}  // namespace gls
