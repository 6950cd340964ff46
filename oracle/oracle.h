/*
 * oracle.h -- serial fp64 CPU oracle for the GradLev fast-weight scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code; only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code with the HIP library.
 *
 * What it computes (one sequence-head; tokens t = 0..T-1; 0-based):
 *   adaptive linear map with persistent weight W0 (d_out x d_in) and temporary
 *   adaptation D_t = W_t - W0, D_0 = 0 ("Parallelize the Training, Keep the
 *   Learning Serial", cognaptus.com, section "Once the gradient signals are
 *   known, the weight trajectory becomes parallelizable": centered per-token
 *   update with eta = update size, alpha = retention of previous adaptation,
 *   g = costate = gradient of the token loss w.r.t. the layer output):
 *
 *       y_t     = (W0 + D_t) x_t                 (read before token t's update;
 *                                                 section "The bottleneck appears
 *                                                 before deployment")
 *       D_{t+1} = alpha_t D_t - eta_t g_t x_t^T  (online gradient-descent step)
 *
 * The backward pass is the exact adjoint of that loop for the scalar
 * L = sum_t <dy_t, y_t>, i.e. it returns dL/dx, dL/dg, dL/deta, dL/dalpha and
 * dL/dW0 (GradLev abstract, omanscience.com: "exact parallel scans for both
 * forward evaluation and reverse backpropagation"; the serial loop is the
 * definition those scans reproduce).
 *
 * Layouts (row-major, last index fastest):
 *   x, dx            [B][H][T][d_in]
 *   g, y, dy, dg     [B][H][T][d_out]
 *   eta, alpha, deta, dalpha  [B][H][T]
 *   W0, dW0          [H][d_out][d_in]   (one W0 per head, shared by the batch)
 * All arrays are host fp64, owned by the caller.  Outputs are overwritten.
 */
#ifndef GL_ORACLE_H
#define GL_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Single sequence forward.  S_init (d_out x d_in) may be NULL (= zero start).
 * S_final (may be NULL) receives D_T, the adaptation after the last token. */
void oracle_seq_fwd(int64_t T, int64_t d_in, int64_t d_out,
                    const double* x, const double* g, const double* eta,
                    const double* alpha, const double* W0, const double* S_init,
                    double* y, double* S_final);

/* Single sequence backward.  dW0 is ACCUMULATED into (caller zeroes it).
 * ckpt = number of tokens between stored states (>= 1); the states inside a
 * segment are recomputed with the same operations, so every ckpt gives
 * bit-identical results.  variant = 0: exact adjoint.  variant = 1: the
 * control of the synthetic test on page 1 (section "The synthetic test checks
 * the mechanism, not model quality"): the input gradient uses W0^T instead of
 * the adapted transpose (W0 + D_t)^T.  Used only to show that the pins bite. */
void oracle_seq_bwd(int64_t T, int64_t d_in, int64_t d_out,
                    const double* x, const double* g, const double* eta,
                    const double* alpha, const double* W0, const double* dy,
                    int64_t ckpt, int variant,
                    double* dx, double* dg, double* deta, double* dalpha,
                    double* dW0);

/* Batched [B][H] versions; nthreads <= 1 runs serially.  dW0 is summed over
 * the batch in a fixed order, so results do not depend on nthreads. */
void oracle_fwd(int64_t B, int64_t H, int64_t T, int64_t d_in, int64_t d_out,
                const double* x, const double* g, const double* eta,
                const double* alpha, const double* W0, double* y, int nthreads);

void oracle_bwd(int64_t B, int64_t H, int64_t T, int64_t d_in, int64_t d_out,
                const double* x, const double* g, const double* eta,
                const double* alpha, const double* W0, const double* dy,
                int64_t ckpt, int variant,
                double* dx, double* dg, double* deta, double* dalpha,
                double* dW0, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
