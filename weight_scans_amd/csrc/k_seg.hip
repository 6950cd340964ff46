// k_seg.hip -- combine step of the segmented scan.
//
// A long sequence is cut into segments that separate work-groups scan from a
// zero state.  Each segment s reports its final state L_s and its summed
// log2 retention lg_s (so the whole segment scales a state by G_s = 2^lg_s).
// Because the per-token update is affine in the state, composing segments
// is the same associative combine as composing tokens ("Parallelize the
// Training, Keep the Learning Serial", cognaptus.com, section "Once the
// gradient signals are known, the weight trajectory becomes
// parallelizable"):
//   state entering segment 0 = 0,  entering s + 1 = G_s (entering s) + L_s.
// The reverse scan composes its adjoint the same way from the right end.
// This kernel replaces every L_s by the state entering segment s (an
// exclusive scan over segments, one thread per matrix element).  The segment
// the scan reaches last never contributes (segment n - 1 forwards, segment 0
// in reverse): its L_s need not have been computed.
#include "internal.hpp"

namespace gls {
namespace {

constexpr int kSegThreads = 256;

__global__ __launch_bounds__(kSegThreads) void seg_combine(float* buf, const float* lg,
                                                           int n_seg, int dd, int reverse) {
  const int64_t bh = blockIdx.y;
  const int e = blockIdx.x * kSegThreads + threadIdx.x;
  if (e >= dd) return;
  float* p = buf + bh * n_seg * static_cast<int64_t>(dd) + e;
  const float* l = lg + bh * n_seg;
  // segments in groups of eight: the group's loads are issued together, then
  // the scan runs through them (one memory round trip per group, not per
  // segment)
  constexpr int kGroup = 8;
  float carry = 0.f;
  for (int k0 = 0; k0 < n_seg; k0 += kGroup) {
    float local[kGroup], lgs[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int k = k0 + j;
      const int s = reverse ? n_seg - 1 - k : k;
      // the segment reached last: its own L_s is never needed (nor read)
      const bool use = k < n_seg - 1;
      local[j] = use ? p[static_cast<int64_t>(s) * dd] : 0.f;
      lgs[j] = use ? l[s] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int k = k0 + j;
      if (k >= n_seg) break;
      const int s = reverse ? n_seg - 1 - k : k;
      p[static_cast<int64_t>(s) * dd] = carry;
      carry = carry * __builtin_amdgcn_exp2f(lgs[j]) + local[j];
    }
  }
}

}  // namespace

hipError_t launch_seg_combine(float* buf, const float* lg, int64_t BH, int n_seg, int dd,
                              bool reverse, hipStream_t s) {
  if (BH == 0 || n_seg <= 1) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((dd + kSegThreads - 1) / kSegThreads),
                  static_cast<unsigned>(BH));
  hipLaunchKernelGGL(seg_combine, grid, dim3(kSegThreads), 0, s, buf, lg, n_seg, dd,
                     reverse ? 1 : 0);
  return hipGetLastError();
}

}  // namespace gls
