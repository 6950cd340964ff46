// k_mfma_bwd.hip -- matrix-core reverse scan at d = 128: the two kernels that
// make it (d = 64 has a fused kernel of its own, k_mfma_bwd_f.hip).
//
// The backward needs the adjoint Lam = dL/dD both by rows (u_i = Lam_i x_i
// reduces over columns: dg, deta, dW0) and by columns (dx reduces over rows,
// dalpha over both), so every (b, h) is covered twice:
//   bwd_a (k_mfma_bwd_a.hip): row tiles of Lam    -> dg, deta partial, dW0 rows
//   bwd_b (k_mfma_bwd_b.hip): column tiles of Lam -> dx, dalpha partial
// the row tiles first, then the column tiles.  Per-token partials (one per
// tile) and the per-(segment, b, h) dW0 partials are summed by the finalize
// kernel in a fixed order.
#include "internal.hpp"

namespace gls {

namespace {
constexpr int kTileRows = 32;  // rows (columns) of Lam per work-group in both kernels
}  // namespace

int mfma_bwd_tiles(int d) { return d / kTileRows; }

hipError_t launch_mfma_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.d_in != 128) return hipErrorInvalidValue;
  const hipError_t e = launch_mfma_bwd_a(a, s);
  if (e != hipSuccess) return e;
  return launch_mfma_bwd_b(a, s);
}

}  // namespace gls
