// k_costate.hip -- costate reconstruction under a quadratic token loss and
// the consistency residual (any io dtype, 1 <= d_out <= 128).
//
// GradLev trains the predicted costates g^ toward the costates the primary
// model reconstructs on the proposed trajectory ("Parallelize the Training,
// Keep the Learning Serial", cognaptus.com, section "The predictor is
// constrained by the learner it is supposed to reproduce").  With the
// quadratic token loss l_t = |y_t - r_t|^2 / 2 of the pages' synthetic test
// (section "The synthetic test checks the mechanism, not model quality"), the
// reconstructed costate is the loss gradient at the scan's output,
//   g~_t = y_t - r_t,
// and the consistency residual of token t compares it with the proposal:
//   res_sq_t = |g^_t - g~_t|^2,   res_max_t = max_r |g^_t[r] - g~_t[r]|.
// The causal map g^ -> g~ has the serial learner's costates as its unique
// fixed point; a Picard sweep (scan, then this kernel, then g^ <- g~) fixes
// at least one more token each time.
//
// Bound by HBM: y, r and g^ are read once and g~ is written once.  The
// residuals use g~ in the compute type, before it is rounded to the io type.
#include <algorithm>
#include <cstddef>

#include "dev_common.hpp"
#include "internal.hpp"

namespace gls {
namespace {

constexpr int kThreads = 256;
constexpr int kPasses = 4;  // token rows per lane group and work-group pass

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
__device__ __forceinline__ void st4(bf16* p, int64_t i, const float (&v)[4]) {
  uint2 t;
  t.x = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
  t.y = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
  *reinterpret_cast<uint2*>(p + i) = t;
}

// Token rows of d_out elements.  VEC (d_out a multiple of 4, L = d_out / 4 a
// power of two): L lanes per row, four elements each, 64 / L rows per wave and
// pass; otherwise one row per wave and pass, lanes striding the row.  The
// row's sums and maxima meet by butterfly within its lanes.
template <typename IO, typename S, bool VEC>
__global__ __launch_bounds__(kThreads) void costate_k(CostArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = a.d_out;
  const int L = VEC ? d / 4 : 64;
  const int RW = 64 / L;  // rows per wave and pass
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wave) * RW * kPasses +
                       lane / L;
  const IO* y = static_cast<const IO*>(a.y);
  const IO* r = static_cast<const IO*>(a.target);
  const IO* gh = static_cast<const IO*>(a.g_hat);
  IO* gt = static_cast<IO*>(a.g_tilde);
  S sq[kPasses], mx[kPasses];
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int64_t row = row0 + static_cast<int64_t>(k) * RW;
    sq[k] = S(0);
    mx[k] = S(0);
    if (row >= a.rows) continue;
    if constexpr (VEC) {
      const int64_t i = row * d + (lane % L) * 4;
      S yv[4], rv[4], hv[4], gv[4];
      ld4(y, i, yv);
      ld4(r, i, rv);
      ld4(gh, i, hv);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        gv[q] = yv[q] - rv[q];
        const S e = hv[q] - gv[q];
        sq[k] += e * e;
        mx[k] = max(mx[k], abs(e));
      }
      st4(gt, i, gv);
    } else {
      for (int c = lane; c < d; c += 64) {
        const int64_t i = row * d + c;
        const S g = load_as<S>(y, i) - load_as<S>(r, i);
        const S e = load_as<S>(gh, i) - g;
        sq[k] += e * e;
        mx[k] = max(mx[k], abs(e));
        store_from(gt, i, g);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    for (int m = L / 2; m >= 1; m >>= 1) {
      sq[k] += __shfl_xor(sq[k], m, 64);
      mx[k] = max(mx[k], __shfl_xor(mx[k], m, 64));
    }
    const int64_t row = row0 + static_cast<int64_t>(k) * RW;
    if (lane % L == 0 && row < a.rows) {
      static_cast<S*>(a.res_sq)[row] = sq[k];
      static_cast<S*>(a.res_max)[row] = mx[k];
    }
  }
}

template <typename IO, typename S>
hipError_t costate_t(const CostArgs& a, hipStream_t s) {
  const int L4 = a.d_out / 4;
  const bool vec = a.d_out % 4 == 0 && (L4 & (L4 - 1)) == 0;
  const int64_t per = (kThreads / 64) * (vec ? 64 / L4 : 1) * kPasses;  // rows per work-group
  const int64_t blocks = (a.rows + per - 1) / per;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL((costate_k<IO, S, true>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       s, a);
  else
    hipLaunchKernelGGL((costate_k<IO, S, false>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_costate(int io, const CostArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (io == IO_F64) return costate_t<double, double>(a, s);
  if (io == IO_F32) return costate_t<float, float>(a, s);
  return costate_t<bf16, float>(a, s);
}

}  // namespace gls
