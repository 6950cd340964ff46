// k_decode.hip -- deployment: one token at a time against the cached
// adaptation (any io dtype, 1 <= d_in, d_out <= 128).
//
// At deployment the learner runs token by token: the layer reads out with
// the cached weight, the network's backward pass returns the costate g of
// that token, and the cache is advanced by the recurrence's update for that
// one token ("Parallelize the Training, Keep the Learning Serial",
// cognaptus.com, section "The bottleneck appears before deployment"; ParaTTT
// news summary, section "Perspective": decoding needs no iteration, each
// token costs a single update of the cache).  With the cached adaptation
// D = W - W0:
//   readout:  y = (W0 + D) x
//   update:   D <- alpha D - eta g x^T
//   step:     the update of token t, then the readout of token t + 1 (the
//             steady state of serving: one pass over the state per token)
// and, to hand a prefill over to decoding, the adaptation after T tokens from
// zero:  D_T = sum_t (prod_{s>t} alpha_s) (-eta_t) g_t x_t^T.
//
// All three are bound by moving the d_out x d_in state (fp32, fp64 for fp64
// io): the readout reads it once, the update reads and writes it.  The final
// state is a hand-over pass (one work-group per sequence-head and block of
// rows, tokens from the right in chunks staged through LDS).
#include <algorithm>
#include <cstddef>

#include "dev_common.hpp"
#include "internal.hpp"

namespace gls {
namespace {

constexpr int kDecThreads = 256;
constexpr int kRowsPerBlock = kDecThreads / 64;  // readout: one wave per output row

template <typename S>
__device__ __forceinline__ S wave_sum64(S v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// y[bh][r] = sum_c (W0[h][r][c] + D[bh][r][c]) x[bh][c]
template <typename IO, typename S>
__global__ __launch_bounds__(kDecThreads) void decode_readout_k(DecArgs a) {
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.y * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= a.d_out) return;
  const IO* x = static_cast<const IO*>(a.x) + bh * a.d_in;
  const IO* w0 = static_cast<const IO*>(a.W0) + (static_cast<int64_t>(h) * a.d_out + r) * a.d_in;
  const S* d = static_cast<const S*>(a.state) + (bh * a.d_out + r) * a.d_in;
  S acc = S(0);
  for (int c = lane; c < a.d_in; c += 64)
    acc += (load_as<S>(w0, c) + d[c]) * load_as<S>(x, c);
  acc = wave_sum64(acc);
  if (lane == 0) store_from(static_cast<IO*>(a.y), bh * a.d_out + r, acc);
}

// Four consecutive elements (16-byte aligned for fp32 / fp64, 8-byte for
// bf16: the base pointers are 16-byte aligned and every offset here is a
// multiple of four elements).
__device__ __forceinline__ void ld4(const float* p, int64_t i, float (&v)[4]) {
  const float4 t = *reinterpret_cast<const float4*>(p + i);
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void ld4(const double* p, int64_t i, double (&v)[4]) {
  const double2 t0 = *reinterpret_cast<const double2*>(p + i);
  const double2 t1 = *reinterpret_cast<const double2*>(p + i + 2);
  v[0] = t0.x; v[1] = t0.y; v[2] = t1.x; v[3] = t1.y;
}
__device__ __forceinline__ void ld4(const bf16* p, int64_t i, float (&v)[4]) {
  const uint2 t = *reinterpret_cast<const uint2*>(p + i);
  v[0] = bf16_to_f32(t.x & 0xffffu); v[1] = bf16_to_f32(t.x >> 16);
  v[2] = bf16_to_f32(t.y & 0xffffu); v[3] = bf16_to_f32(t.y >> 16);
}
__device__ __forceinline__ void st4(float* p, int64_t i, const float (&v)[4]) {
  *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st4(double* p, int64_t i, const double (&v)[4]) {
  *reinterpret_cast<double2*>(p + i) = make_double2(v[0], v[1]);
  *reinterpret_cast<double2*>(p + i + 2) = make_double2(v[2], v[3]);
}

constexpr int kVecGroups = 4;  // 4-element groups per thread in the vector kernels

// Readout with d_in a multiple of 4 and L = d_in / 4 a power of two: L lanes
// per row (four elements each), 64 / L rows per wave and pass, kVecGroups
// passes; the row's partial sums meet by butterfly within its L lanes.  With
// UPD, each lane first takes the update of the previous token on its four
// state elements (x_prev, g_prev, eta_prev, alpha_prev), stores them and reads
// out the new token from the updated state: one pass over the state per token.
template <typename IO, typename S, bool UPD>
__global__ __launch_bounds__(kDecThreads) void decode_readout_v(DecArgs a) {
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int L = a.d_in / 4, RW = 64 / L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = (lane % L) * 4;
  const int r_base = (blockIdx.y * (kDecThreads / 64) + wave) * RW * kVecGroups + lane / L;
  const IO* w0 = static_cast<const IO*>(a.W0) + static_cast<int64_t>(h) * a.d_out * a.d_in;
  S* d = static_cast<S*>(a.state) + bh * a.d_out * a.d_in;
  S xv[4], xp[4] = {}, al = S(0), ne = S(0);
  ld4(static_cast<const IO*>(a.x), bh * a.d_in + c, xv);
  if constexpr (UPD) {
    ld4(static_cast<const IO*>(a.x_prev), bh * a.d_in + c, xp);
    al = static_cast<const S*>(a.alpha)[bh];
    ne = -static_cast<const S*>(a.eta)[bh];
  }
  S acc[kVecGroups];
#pragma unroll
  for (int k = 0; k < kVecGroups; ++k) {
    const int r = r_base + k * RW;
    acc[k] = S(0);
    if (r < a.d_out) {
      S wv[4], dv[4];
      ld4(w0, static_cast<int64_t>(r) * a.d_in + c, wv);
      ld4(d, static_cast<int64_t>(r) * a.d_in + c, dv);
      if constexpr (UPD) {
        const S gr = ne * load_as<S>(static_cast<const IO*>(a.g), bh * a.d_out + r);
#pragma unroll
        for (int q = 0; q < 4; ++q) dv[q] = al * dv[q] + gr * xp[q];
        st4(d, static_cast<int64_t>(r) * a.d_in + c, dv);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[k] += (wv[q] + dv[q]) * xv[q];
    }
  }
#pragma unroll
  for (int k = 0; k < kVecGroups; ++k) {
    for (int m = L / 2; m >= 1; m >>= 1) acc[k] += __shfl_xor(acc[k], m, 64);
    const int r = r_base + k * RW;
    if (lane % L == 0 && r < a.d_out) store_from(static_cast<IO*>(a.y), bh * a.d_out + r, acc[k]);
  }
}

// Update with d_in a multiple of 4: each thread takes kVecGroups groups of
// four elements of one row (block y: a run of 256 kVecGroups groups).
template <typename IO, typename S>
__global__ __launch_bounds__(kDecThreads) void decode_update_v(DecArgs a) {
  const int64_t bh = blockIdx.x;
  const int n4 = a.d_in * a.d_out / 4;
  const int L = a.d_in / 4;
  const IO* x = static_cast<const IO*>(a.x) + bh * a.d_in;
  const IO* g = static_cast<const IO*>(a.g) + bh * a.d_out;
  const S al = static_cast<const S*>(a.alpha)[bh];
  const S ne = -static_cast<const S*>(a.eta)[bh];
  S* d = static_cast<S*>(a.state) + bh * a.d_in * a.d_out;
  const int e0 = blockIdx.y * kDecThreads * kVecGroups + threadIdx.x;
  S dv[kVecGroups][4];
#pragma unroll
  for (int k = 0; k < kVecGroups; ++k) {
    const int e = e0 + k * kDecThreads;
    if (e < n4) ld4(d, 4 * static_cast<int64_t>(e), dv[k]);
  }
#pragma unroll
  for (int k = 0; k < kVecGroups; ++k) {
    const int e = e0 + k * kDecThreads;
    if (e < n4) {
      const int r = e / L, c = (e - r * L) * 4;
      const S gr = ne * load_as<S>(g, r);
      S xv[4];
      ld4(x, c, xv);
#pragma unroll
      for (int q = 0; q < 4; ++q) dv[k][q] = al * dv[k][q] + gr * xv[q];
      st4(d, 4 * static_cast<int64_t>(e), dv[k]);
    }
  }
}

// D[bh][r][c] <- alpha[bh] D[bh][r][c] - eta[bh] g[bh][r] x[bh][c]
// (block x: the sequence-head, block y: a run of 256 elements of its state)
template <typename IO, typename S>
__global__ __launch_bounds__(kDecThreads) void decode_update_k(DecArgs a) {
  const int64_t bh = blockIdx.x;
  const int dd = a.d_in * a.d_out;
  const IO* x = static_cast<const IO*>(a.x) + bh * a.d_in;
  const IO* g = static_cast<const IO*>(a.g) + bh * a.d_out;
  const S al = static_cast<const S*>(a.alpha)[bh];
  const S ne = -static_cast<const S*>(a.eta)[bh];
  S* d = static_cast<S*>(a.state) + bh * dd;
  for (int e = blockIdx.y * kDecThreads + threadIdx.x; e < dd; e += gridDim.y * kDecThreads) {
    const int r = e / a.d_in, c = e - r * a.d_in;
    d[e] = al * d[e] + ne * load_as<S>(g, r) * load_as<S>(x, c);
  }
}

// D_T of one sequence-head from zero, one work-group per block of kRT rows
// (block x: the sequence-head, block y: the row block).  Thread t owns column
// c = t % d_in and the RPT = ceil(kRT / RG) consecutive rows from
// rg RPT of the block (rg = t / d_in, RG = 256 / d_in >= 2; threads with
// rg >= RG hold nothing).  Tokens are taken from the right in chunks of kCT:
// each thread keeps its own column of x for the chunk in registers, the g
// rows of the block, eta and alpha go through LDS, and the next chunk's loads
// are in flight while this one is folded in.  Every thread forms the weights
// w_t = (prod_{s>t} alpha_s)(-eta_t) itself from the chunk's gates and the
// running product of the gates already taken; a short chunk is padded with
// neutral gates (eta = 0, alpha = 1), so every chunk folds in kCT tokens
// without branches.  NR accumulators per thread (NR >= RPT); with VEC
// (RG NR == kRT) a thread's g values of a token are read from LDS as one
// vector.
constexpr int kMaxD = 128;
constexpr int kRT = 16;                              // rows per work-group
constexpr int kCT = 32;                              // tokens per chunk
constexpr int kGPer = kCT * kRT / kDecThreads;       // g values staged per thread

// NR consecutive values from 16-byte aligned LDS, 16 bytes per read
template <int NR>
__device__ __forceinline__ void lds_row(const float* p, float (&v)[NR]) {
#pragma unroll
  for (int i = 0; i < NR / 4; ++i) {
    const float4 t = reinterpret_cast<const float4*>(p)[i];
    v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
  }
}
template <int NR>
__device__ __forceinline__ void lds_row(const double* p, double (&v)[NR]) {
#pragma unroll
  for (int i = 0; i < NR / 2; ++i) {
    const double2 t = reinterpret_cast<const double2*>(p)[i];
    v[2 * i] = t.x; v[2 * i + 1] = t.y;
  }
}

template <typename IO, typename S, int NR, bool VEC>
__global__ __launch_bounds__(kDecThreads) void final_state_k(DecArgs a) {
  __shared__ S es[kCT], as[kCT];
  __shared__ __attribute__((aligned(16))) S gs[kCT][kRT];
  const int64_t bh = blockIdx.x;
  const int r0 = blockIdx.y * kRT;
  const int rows = min(kRT, a.d_out - r0);
  const int tid = threadIdx.x;
  const int64_t T = a.T;
  const int d_in = a.d_in;
  const int RG = kDecThreads / d_in;
  const int RPT = (kRT + RG - 1) / RG;
  const int c = tid % d_in, rg = tid / d_in;
  // first row of this thread (idle threads fold in row 0 and store nothing)
  const int rbase = rg < RG ? rg * RPT : 0;
  const int nrow = rg < RG ? max(0, min(RPT, rows - rbase)) : 0;
  const IO* x = static_cast<const IO*>(a.x) + bh * T * d_in + c;
  const IO* g = static_cast<const IO*>(a.g) + bh * T * a.d_out + r0;
  const S* eta = static_cast<const S*>(a.eta) + bh * T;
  const S* alpha = static_cast<const S*>(a.alpha) + bh * T;

  S xn[kCT], rgv[kGPer], re = S(0), ra = S(1);
  const auto fetch = [&](int64_t lo, int n) {
    // padding positions load the chunk's last token (its weight is zero)
#pragma unroll
    for (int j = 0; j < kCT; ++j) xn[j] = load_as<S>(x, (lo + min(j, n - 1)) * d_in);
#pragma unroll
    for (int i = 0; i < kGPer; ++i) {
      const int idx = tid + i * kDecThreads, j = idx / kRT, r = idx % kRT;
      rgv[i] = load_as<S>(g, (lo + min(j, n - 1)) * a.d_out + min(r, rows - 1));
    }
    if (tid < kCT) {
      re = eta[lo + min(tid, n - 1)];
      ra = alpha[lo + min(tid, n - 1)];
    }
  };
  const auto stash = [&](int n) {
#pragma unroll
    for (int i = 0; i < kGPer; ++i) {
      const int idx = tid + i * kDecThreads, j = idx / kRT, r = idx % kRT;
      gs[j][r] = r < rows ? rgv[i] : S(0);
    }
    if (tid < kCT) {
      es[tid] = tid < n ? re : S(0);
      as[tid] = tid < n ? ra : S(1);
    }
  };

  S acc[NR];
  int grow[NR];  // this thread's rows within the block, clamped into it
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    acc[k] = S(0);
    grow[k] = min(rbase + k, kRT - 1);
  }
  S carry = S(1);  // prod of alpha over the tokens already taken
  int64_t hi = T, lo = T - kCT > 0 ? T - kCT : 0;
  if (T > 0) fetch(lo, static_cast<int>(hi - lo));
  while (hi > 0) {
    const int n = static_cast<int>(hi - lo);
    __syncthreads();  // the previous chunk is folded in by every thread
    stash(n);
    __syncthreads();
    S xc[kCT];
#pragma unroll
    for (int j = 0; j < kCT; ++j) xc[j] = xn[j];
    const int64_t hi2 = lo, lo2 = lo - kCT > 0 ? lo - kCT : 0;
    if (hi2 > 0) fetch(lo2, static_cast<int>(hi2 - lo2));
    // every thread folds in NR rows (rows past its own read a valid entry of
    // the block and are never stored)
    S p = carry;
#pragma unroll
    for (int j = kCT - 1; j >= 0; --j) {
      const S wx = -p * es[j] * xc[j];
      if constexpr (VEC) {
        S gv[NR];
        lds_row<NR>(&gs[j][rbase], gv);
#pragma unroll
        for (int k = 0; k < NR; ++k) acc[k] += wx * gv[k];
      } else {
#pragma unroll
        for (int k = 0; k < NR; ++k) acc[k] += wx * gs[j][grow[k]];
      }
      p *= as[j];
    }
    carry = p;
    hi = hi2;
    lo = lo2;
  }
  S* d = static_cast<S*>(a.state) + (bh * a.d_out + r0) * static_cast<int64_t>(d_in);
#pragma unroll
  for (int k = 0; k < NR; ++k)
    if (k < nrow) d[static_cast<int64_t>(rbase + k) * d_in + c] = acc[k];
}

bool readout_vec(const DecArgs& a) {
  const int L = a.d_in / 4;
  return a.d_in % 4 == 0 && (L & (L - 1)) == 0;
}

template <typename IO, typename S>
hipError_t readout_t(const DecArgs& a, hipStream_t s) {
  if (readout_vec(a)) {
    const int rows = (kDecThreads / 64) * (64 / (a.d_in / 4)) * kVecGroups;  // per work-group
    const dim3 grid(static_cast<unsigned>(a.B * a.H), (a.d_out + rows - 1) / rows);
    hipLaunchKernelGGL((decode_readout_v<IO, S, false>), grid, dim3(kDecThreads), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(a.B * a.H), (a.d_out + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL((decode_readout_k<IO, S>), grid, dim3(kDecThreads), 0, s, a);
  return hipGetLastError();
}

template <typename IO, typename S>
hipError_t update_t(const DecArgs& a, hipStream_t s) {
  if (a.d_in % 4 == 0) {
    const int per = kDecThreads * kVecGroups;  // groups per work-group
    const dim3 grid(static_cast<unsigned>(a.B * a.H), (a.d_in * a.d_out / 4 + per - 1) / per);
    hipLaunchKernelGGL((decode_update_v<IO, S>), grid, dim3(kDecThreads), 0, s, a);
    return hipGetLastError();
  }
  const int dd = a.d_in * a.d_out;
  const dim3 grid(static_cast<unsigned>(a.B * a.H), (dd + kDecThreads - 1) / kDecThreads);
  hipLaunchKernelGGL((decode_update_k<IO, S>), grid, dim3(kDecThreads), 0, s, a);
  return hipGetLastError();
}

// update of the previous token (a.x_prev, a.g, a.eta, a.alpha), then readout
// of a.x: one launch where the vector layout applies, else the two kernels
template <typename IO, typename S>
hipError_t step_t(const DecArgs& a, hipStream_t s) {
  if (readout_vec(a)) {
    const int rows = (kDecThreads / 64) * (64 / (a.d_in / 4)) * kVecGroups;
    const dim3 grid(static_cast<unsigned>(a.B * a.H), (a.d_out + rows - 1) / rows);
    hipLaunchKernelGGL((decode_readout_v<IO, S, true>), grid, dim3(kDecThreads), 0, s, a);
    return hipGetLastError();
  }
  DecArgs u = a;
  u.x = a.x_prev;
  const hipError_t e = update_t<IO, S>(u, s);
  if (e != hipSuccess) return e;
  return readout_t<IO, S>(a, s);
}

template <typename IO, typename S>
hipError_t final_t(const DecArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B * a.H), (a.d_out + kRT - 1) / kRT);
  const int RG = kDecThreads / a.d_in, RPT = (kRT + RG - 1) / RG;
  if (RG * 8 == kRT)
    hipLaunchKernelGGL((final_state_k<IO, S, 8, true>), grid, dim3(kDecThreads), 0, s, a);
  else if (RG * 4 == kRT)
    hipLaunchKernelGGL((final_state_k<IO, S, 4, true>), grid, dim3(kDecThreads), 0, s, a);
  else if (RPT > 4)
    hipLaunchKernelGGL((final_state_k<IO, S, 8, false>), grid, dim3(kDecThreads), 0, s, a);
  else
    hipLaunchKernelGGL((final_state_k<IO, S, 4, false>), grid, dim3(kDecThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_readout(int io, const DecArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  if (io == IO_F64) return readout_t<double, double>(a, s);
  if (io == IO_F32) return readout_t<float, float>(a, s);
  return readout_t<bf16, float>(a, s);
}

hipError_t launch_decode_update(int io, const DecArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  if (io == IO_F64) return update_t<double, double>(a, s);
  if (io == IO_F32) return update_t<float, float>(a, s);
  return update_t<bf16, float>(a, s);
}

hipError_t launch_decode_step(int io, const DecArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  if (io == IO_F64) return step_t<double, double>(a, s);
  if (io == IO_F32) return step_t<float, float>(a, s);
  return step_t<bf16, float>(a, s);
}

hipError_t launch_final_state(int io, const DecArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  if (io == IO_F64) return final_t<double, double>(a, s);
  if (io == IO_F32) return final_t<float, float>(a, s);
  return final_t<bf16, float>(a, s);
}

}  // namespace gls
