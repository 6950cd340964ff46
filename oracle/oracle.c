/*
 * oracle.c -- serial fp64 CPU oracle for the GradLev fast-weight scan.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).  The
 * product path never includes, links or calls it, and it shares no code with
 * the HIP library.
 *
 * The oracle is the plain definition of the learner: a token-by-token loop
 * that materialises the adaptation D_t = W_t - W0 and reads the pre-update
 * weight, followed by the exact serial adjoint.  Sources (page titles and
 * sections; the update formula itself was lost from the page text and is
 * restated from the surrounding prose):
 *  - "Parallelize the Training, Keep the Learning Serial" (cognaptus.com),
 *    section "Once the gradient signals are known, the weight trajectory
 *    becomes parallelizable": adaptive linear map W_t started from W0, a
 *    centered update with update size eta_t, retention alpha_t of the previous
 *    adaptation and costate g_t (gradient of the token loss w.r.t. the layer
 *    output); the correction is a discounted sum of rank-one gradient updates.
 *  - same page, section "The bottleneck appears before deployment": token t+1
 *    uses the weights changed by token t (so y_t reads D_t, not D_{t+1}).
 *  - GradLev abstract (omanscience.com): online gradient descent, exact scans
 *    for forward evaluation and reverse backpropagation.
 * Nothing here is blocked, fused or reordered beyond the loop itself.
 */
#include "oracle.h"

#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* D <- alpha * D - eta * g x^T   (one online gradient-descent step on the
 * adaptation; the minus sign is descent, the alpha factor decays the
 * adaptation toward W0 -- "centered"). */
static void adapt_step(int64_t d_in, int64_t d_out, double* D, double alpha,
                       double eta, const double* g, const double* x) {
  for (int64_t r = 0; r < d_out; ++r)
    for (int64_t c = 0; c < d_in; ++c)
      D[r * d_in + c] = alpha * D[r * d_in + c] - eta * g[r] * x[c];
}

void oracle_seq_fwd(int64_t T, int64_t d_in, int64_t d_out, const double* x,
                    const double* g, const double* eta, const double* alpha,
                    const double* W0, const double* S_init, double* y,
                    double* S_final) {
  const int64_t dd = d_in * d_out;
  double* D = (double*)calloc((size_t)dd, sizeof(double));
  if (S_init) memcpy(D, S_init, sizeof(double) * (size_t)dd);
  for (int64_t t = 0; t < T; ++t) {
    const double* xt = x + t * d_in;
    /* readout from the pre-update weight W0 + D_t */
    for (int64_t r = 0; r < d_out; ++r) {
      double acc = 0.0;
      for (int64_t c = 0; c < d_in; ++c)
        acc += (W0[r * d_in + c] + D[r * d_in + c]) * xt[c];
      y[t * d_out + r] = acc;
    }
    adapt_step(d_in, d_out, D, alpha[t], eta[t], g + t * d_out, xt);
  }
  if (S_final) memcpy(S_final, D, sizeof(double) * (size_t)dd);
  free(D);
}

/* Exact adjoint of oracle_seq_fwd for L = sum_t <dy_t, y_t>.
 * Lam holds dL/dD_{t+1} (the adaptation after token t); it is zero after the
 * last token because that update is never read.  Per token, walking back:
 *   u        = Lam x_t
 *   deta_t   = -<g_t, u>            dg_t = -eta_t u
 *   dx_t     = (W0 + D_t)^T dy_t - eta_t Lam^T g_t
 *   dalpha_t = <Lam, D_t>_F
 *   dW0     += dy_t x_t^T
 *   Lam     <- alpha_t Lam + dy_t x_t^T          (becomes dL/dD_t)
 * D_t is recovered from stored states every `ckpt` tokens plus a forward
 * recomputation of the segment with the same operations. */
void oracle_seq_bwd(int64_t T, int64_t d_in, int64_t d_out, const double* x,
                    const double* g, const double* eta, const double* alpha,
                    const double* W0, const double* dy, int64_t ckpt,
                    int variant, double* dx, double* dg, double* deta,
                    double* dalpha, double* dW0) {
  const int64_t dd = d_in * d_out;
  if (T <= 0) return;
  if (ckpt < 1) ckpt = 1;
  if (ckpt > T) ckpt = T;
  const int64_t nseg = (T + ckpt - 1) / ckpt;
  double* ck = (double*)malloc(sizeof(double) * (size_t)(nseg * dd));
  double* seg = (double*)malloc(sizeof(double) * (size_t)(ckpt * dd));
  double* Lam = (double*)calloc((size_t)dd, sizeof(double));
  double* u = (double*)malloc(sizeof(double) * (size_t)d_out);

  /* forward pass, keeping D at the start of every segment */
  double* D = (double*)calloc((size_t)dd, sizeof(double));
  for (int64_t t = 0; t < T; ++t) {
    if (t % ckpt == 0) memcpy(ck + (t / ckpt) * dd, D, sizeof(double) * (size_t)dd);
    adapt_step(d_in, d_out, D, alpha[t], eta[t], g + t * d_out, x + t * d_in);
  }
  free(D);

  for (int64_t s = nseg - 1; s >= 0; --s) {
    const int64_t t0 = s * ckpt;
    const int64_t t1 = (t0 + ckpt < T) ? t0 + ckpt : T;
    /* seg[k] = D_{t0+k}: the adaptation read by token t0+k */
    memcpy(seg, ck + s * dd, sizeof(double) * (size_t)dd);
    for (int64_t t = t0; t + 1 < t1; ++t) {
      double* nxt = seg + (t - t0 + 1) * dd;
      memcpy(nxt, seg + (t - t0) * dd, sizeof(double) * (size_t)dd);
      adapt_step(d_in, d_out, nxt, alpha[t], eta[t], g + t * d_out, x + t * d_in);
    }
    for (int64_t t = t1 - 1; t >= t0; --t) {
      const double* Dt = seg + (t - t0) * dd;
      const double* xt = x + t * d_in;
      const double* gt = g + t * d_out;
      const double* dyt = dy + t * d_out;
      double dn = 0.0;
      for (int64_t r = 0; r < d_out; ++r) {
        double acc = 0.0;
        for (int64_t c = 0; c < d_in; ++c) acc += Lam[r * d_in + c] * xt[c];
        u[r] = acc;
        dn -= gt[r] * acc;
      }
      deta[t] = dn;
      for (int64_t r = 0; r < d_out; ++r) dg[t * d_out + r] = -eta[t] * u[r];
      for (int64_t c = 0; c < d_in; ++c) {
        double a = 0.0, b = 0.0;
        for (int64_t r = 0; r < d_out; ++r) {
          const double w = (variant == 1) ? W0[r * d_in + c]
                                          : W0[r * d_in + c] + Dt[r * d_in + c];
          a += w * dyt[r];
          b += Lam[r * d_in + c] * gt[r];
        }
        dx[t * d_in + c] = a - eta[t] * b;
      }
      double da = 0.0;
      for (int64_t k = 0; k < dd; ++k) da += Lam[k] * Dt[k];
      dalpha[t] = da;
      for (int64_t r = 0; r < d_out; ++r)
        for (int64_t c = 0; c < d_in; ++c) {
          dW0[r * d_in + c] += dyt[r] * xt[c];
          Lam[r * d_in + c] = alpha[t] * Lam[r * d_in + c] + dyt[r] * xt[c];
        }
    }
  }
  free(u);
  free(Lam);
  free(seg);
  free(ck);
}

/* ---------------- batched drivers (one work item = one (b,h)) ------------ */
typedef struct {
  int64_t B, H, T, d_in, d_out, ckpt;
  int variant, nthreads, tid, bwd;
  const double *x, *g, *eta, *alpha, *W0, *dy;
  double *y, *dx, *dg, *deta, *dalpha, *dW0part;
} job_t;

static void* run_items(void* arg) {
  job_t* j = (job_t*)arg;
  const int64_t n = j->B * j->H, dd = j->d_in * j->d_out;
  for (int64_t i = j->tid; i < n; i += j->nthreads) {
    const int64_t h = i % j->H;
    const double* x = j->x + i * j->T * j->d_in;
    const double* g = j->g + i * j->T * j->d_out;
    const double* e = j->eta + i * j->T;
    const double* a = j->alpha + i * j->T;
    const double* W = j->W0 + h * dd;
    if (!j->bwd) {
      oracle_seq_fwd(j->T, j->d_in, j->d_out, x, g, e, a, W, NULL,
                     j->y + i * j->T * j->d_out, NULL);
    } else {
      double* part = j->dW0part + i * dd;
      memset(part, 0, sizeof(double) * (size_t)dd);
      oracle_seq_bwd(j->T, j->d_in, j->d_out, x, g, e, a, W,
                     j->dy + i * j->T * j->d_out, j->ckpt, j->variant,
                     j->dx + i * j->T * j->d_in, j->dg + i * j->T * j->d_out,
                     j->deta + i * j->T, j->dalpha + i * j->T, part);
    }
  }
  return NULL;
}

static void run_all(job_t* base) {
  int nt = base->nthreads < 1 ? 1 : base->nthreads;
  if (nt > base->B * base->H) nt = (int)(base->B * base->H);
  if (nt < 1) nt = 1;
  job_t* jobs = (job_t*)malloc(sizeof(job_t) * (size_t)nt);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
  for (int k = 0; k < nt; ++k) {
    jobs[k] = *base;
    jobs[k].tid = k;
    jobs[k].nthreads = nt;
  }
  for (int k = 1; k < nt; ++k) pthread_create(&th[k], NULL, run_items, &jobs[k]);
  run_items(&jobs[0]);
  for (int k = 1; k < nt; ++k) pthread_join(th[k], NULL);
  free(th);
  free(jobs);
}

void oracle_fwd(int64_t B, int64_t H, int64_t T, int64_t d_in, int64_t d_out,
                const double* x, const double* g, const double* eta,
                const double* alpha, const double* W0, double* y, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof(j));
  j.B = B; j.H = H; j.T = T; j.d_in = d_in; j.d_out = d_out;
  j.x = x; j.g = g; j.eta = eta; j.alpha = alpha; j.W0 = W0; j.y = y;
  j.nthreads = nthreads; j.bwd = 0;
  if (B * H * T > 0) run_all(&j);
}

void oracle_bwd(int64_t B, int64_t H, int64_t T, int64_t d_in, int64_t d_out,
                const double* x, const double* g, const double* eta,
                const double* alpha, const double* W0, const double* dy,
                int64_t ckpt, int variant, double* dx, double* dg, double* deta,
                double* dalpha, double* dW0, int nthreads) {
  const int64_t dd = d_in * d_out;
  memset(dW0, 0, sizeof(double) * (size_t)(H * dd));
  if (B * H * T <= 0) return;
  double* part = (double*)malloc(sizeof(double) * (size_t)(B * H * dd));
  job_t j;
  memset(&j, 0, sizeof(j));
  j.B = B; j.H = H; j.T = T; j.d_in = d_in; j.d_out = d_out; j.ckpt = ckpt;
  j.variant = variant; j.x = x; j.g = g; j.eta = eta; j.alpha = alpha;
  j.W0 = W0; j.dy = dy; j.dx = dx; j.dg = dg; j.deta = deta; j.dalpha = dalpha;
  j.dW0part = part; j.nthreads = nthreads; j.bwd = 1;
  run_all(&j);
  /* dW0 = sum over the batch, b ascending (fixed order) */
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t k = 0; k < dd; ++k) dW0[h * dd + k] += part[(b * H + h) * dd + k];
  free(part);
}
