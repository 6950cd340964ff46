// k_mfma_bwd.hip -- matrix-core reverse scan: the two kernels that make it.
//
// The backward needs the adjoint Lam = dL/dD both by rows (u_i = Lam_i x_i
// reduces over columns: dg, deta, dW0) and by columns (dx reduces over rows,
// dalpha over both), so every (b, h) is covered twice:
//   bwd_a (k_mfma_bwd_a.hip): row tiles of Lam    -> dg, deta partial, dW0 rows
//   bwd_b (k_mfma_bwd_b.hip): column tiles of Lam -> dx, dalpha partial
// At D = 64 both kinds fit two work-groups per CU, and one launch holds
// both (k_mfma_bwd_ab.hip) so that the two chains of a head run side by side;
// at D = 128 the row tiles run first, then the column tiles.
// Per-token partials (one per tile) and the per-(b, h) dW0 partials are
// summed by the finalize kernel in a fixed order.
#include "internal.hpp"

namespace gls {

namespace {
constexpr int kTileRows = 32;  // rows (columns) of Lam per work-group in both kernels
}  // namespace

int mfma_bwd_tiles(int d) { return d / kTileRows; }

hipError_t launch_mfma_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.d_in == 64) return launch_mfma_bwd_ab64(a, s);
  const hipError_t e = launch_mfma_bwd_a(a, s);
  if (e != hipSuccess) return e;
  return launch_mfma_bwd_b(a, s);
}

}  // namespace gls
