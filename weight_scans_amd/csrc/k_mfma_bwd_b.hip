// k_mfma_bwd_b.hip -- the column-tile pass of the matrix-core reverse scan as
// a kernel of its own (used where it does not share a CU with the row-tile
// pass; see bwd_b.hpp for the mathematics and the pipeline).
#include "bwd_b.hpp"

namespace gls {
namespace {

template <int D>
__global__ __launch_bounds__(kNT) void bwd_b(BwdArgs a) {
  constexpr int NTILE = D / kT;
  __shared__ SlotB<D> ring0, ring1;
  __shared__ __bf16 BeT_s[kC * kC];
  __shared__ __bf16 L0_s[D * kT], L1_s[D * kT];
  __shared__ __bf16 XS_s[kC * kT];
  __shared__ GatesB gs[3];
  __shared__ float dots_s[2 * 2 * 4 * kC];
  __shared__ float c0_s[2 * kNW];
  // (segment is the slowest index, so the XCD of a head does not change)
  const int per_seg = static_cast<int>((a.B * a.H + 7) / 8) * 8 * NTILE;
  const int seg = blockIdx.x / per_seg, bid = blockIdx.x % per_seg;
  const int grp = bid / (8 * NTILE), within = bid % (8 * NTILE);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  if (bh >= a.B * a.H) return;
  const SmemB<D> m{ring0, ring1, BeT_s, L0_s, L1_s, XS_s, gs, dots_s, c0_s};
  role_b_body<D>(a, bh, within >> 3, seg, m);
}

template <int D>
hipError_t launch_b(const BwdArgs& a, hipStream_t s) {
  const int64_t groups = (a.B * a.H + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (D / kT) * a.n_seg));
  hipLaunchKernelGGL(bwd_b<D>, grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_bwd_b(const BwdArgs& a, hipStream_t s) {
  return a.d_in == 128 ? launch_b<128>(a, s) : launch_b<64>(a, s);
}

}  // namespace gls
