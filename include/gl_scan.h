/*
 * gl_scan.h -- C ABI of the GradLev fast-weight scan library (libglscan.so).
 *
 * The operation ("Parallelize the Training, Keep the Learning Serial",
 * cognaptus.com, section "Once the gradient signals are known, the weight
 * trajectory becomes parallelizable"; GradLev abstract, omanscience.com):
 * an adaptive linear map with persistent weight W0 and temporary adaptation
 * D_t = W_t - W0 is updated after every token by one online gradient-descent
 * step with update size eta_t and retention alpha_t of the previous
 * adaptation, driven by the costate g_t (gradient of the token loss w.r.t. the
 * layer output).  Per sequence-head, tokens t = 0..T-1, D_0 = 0:
 *
 *     y_t     = (W0 + D_t) x_t            read from the pre-update weight
 *     D_{t+1} = alpha_t D_t - eta_t g_t x_t^T
 *
 * Because the recurrence is affine in D, the library evaluates it as a chunked
 * associative prefix scan (gl_scan_fwd) and its exact adjoint as the matching
 * reverse-time scan (gl_scan_bwd), which returns the gradients of
 * L = sum_t <dy_t, y_t> w.r.t. x, g, eta, alpha and W0.
 *
 * Layouts: dense, row-major, last index fastest.
 *   x, dx                    [B][H][T][d_in]     io dtype
 *   g, y, dy, dg             [B][H][T][d_out]    io dtype
 *   eta, alpha, deta, dalpha [B][H][T]           gate dtype (fp64 if io is
 *                                                F64, else fp32)
 *   W0                       [H][d_out][d_in]    io dtype (shared by the batch)
 *   dW0                      [H][d_out][d_in]    gate dtype (sum over batch)
 *
 * Ownership: every data pointer is a DEVICE pointer allocated and owned by
 * the caller; the library keeps no state between calls and allocates no
 * memory.  Scratch memory is passed in as `ws` (size from
 * gl_scan_workspace_size).  Outputs are overwritten, never accumulated, and
 * must not alias inputs.  Calls are asynchronous on `stream` (a hipStream_t;
 * NULL = the default stream); the caller synchronises.
 *
 * Errors: every argument check runs before anything is launched; on error the
 * call returns a status and touches no output.  GL_ERROR_HIP reports a failed
 * launch (text via gl_last_error()).  Nothing aborts, prints or throws.
 *
 * Numerical preconditions of every path (documented, not checked on the
 * device): inputs are finite and 0 < alpha_t <= 1.  The scans work with
 * log alpha, and the matrix-core kernels build their decay factors on the
 * assumption that every product of gates is at most one (the rank-one factors
 * of the off-diagonal score blocks are clamped at one); an alpha above one
 * gives results that are silently wrong there.  The oracle and the serial
 * recurrence accept any alpha.
 */
#ifndef GL_SCAN_H
#define GL_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GL_DTYPE_F64 = 0,  /* fp64 everywhere                                   */
  GL_DTYPE_F32 = 1,  /* fp32 io, gates, state                             */
  GL_DTYPE_BF16 = 2  /* bf16 io; fp32 gates, accumulation and state       */
} gl_dtype_t;

typedef enum {
  GL_SUCCESS = 0,
  GL_ERROR_INVALID_VALUE = 1,        /* NULL pointer, negative size, bad enum   */
  GL_ERROR_NOT_SUPPORTED = 2,        /* shape / dtype / chunk not implemented    */
  GL_ERROR_MISALIGNED = 3,           /* a data pointer is not 16-byte aligned    */
  GL_ERROR_WORKSPACE_TOO_SMALL = 4,  /* ws_bytes below gl_scan_workspace_size    */
  GL_ERROR_HIP = 5                   /* a HIP runtime call or launch failed      */
} gl_status_t;

/* Flags for gl_scan_desc_t.flags */
#define GL_FLAG_GENERIC 1u  /* use the portable VALU kernels even where a matrix-
                               core kernel exists (cross-checking only)        */
#define GL_FLAG_OUT_F32 2u  /* gl_scan_fwd / gl_scan_bwd: y, dx and dg are fp32
                               (the accumulators, not rounded to the io type)
                               although io is BF16; no effect with F32 io;
                               F64 io: GL_ERROR_NOT_SUPPORTED.  Inputs keep
                               the io dtype.                                   */

typedef struct {
  int64_t B, H, T;      /* batch, heads, tokens; any may be 0 (no-op)          */
  int64_t d_in, d_out;  /* 1..128 each; the matrix-core kernels take
                           d_in == d_out in {64, 128} with BF16 io            */
  int32_t io_dtype;     /* gl_dtype_t                                          */
  int32_t chunk;        /* tokens per chunk; 0 = default of the chosen kernels.
                           The result does not depend on it (the chunked form
                           is exact).  Taken: 8, 16, 32 by the VALU kernels
                           (F64: 8, 16), 64 by the matrix-core kernels; any
                           other value (128 included: its 128 x 128 score
                           tiles do not fit LDS beside the d = 128 state) is
                           GL_ERROR_NOT_SUPPORTED                             */
  uint32_t flags;       /* GL_FLAG_*                                           */
  uint32_t segments;    /* matrix-core kernels: 0 = automatic (long sequences
                           with few heads are cut into segments so that a pass
                           fills the GPU), 1 = one segment per sequence, n > 1
                           = n segments (at most one per chunk); the generic
                           kernels take 0 or 1 only                         */
} gl_scan_desc_t;

/* Bytes of the optional `saved` buffer that gl_scan_fwd can fill with chunk-
 * boundary adaptation states for gl_scan_bwd (opaque layout; the same desc
 * must be used for both calls). */
gl_status_t gl_scan_saved_size(const gl_scan_desc_t* desc, size_t* saved_bytes);

/* Workspace bytes for gl_scan_fwd and gl_scan_bwd.  have_saved != 0: the fwd
 * call receives a `saved` buffer and the bwd call the same buffer; 0: neither
 * does, and the bwd recomputes the chunk-boundary states itself inside its
 * workspace.  The fwd needs a workspace when the sequences are cut into
 * segments, and on the fp32 / fp64 matrix-core kernels (per-chunk decays, plus
 * the chunk-boundary states when there is no `saved`); otherwise 0 bytes and
 * ws may be NULL. */
gl_status_t gl_scan_workspace_size(const gl_scan_desc_t* desc, int have_saved,
                                   size_t* fwd_ws_bytes, size_t* bwd_ws_bytes);

/* Forward prefix scan: y.  `saved` may be NULL; otherwise it receives
 * gl_scan_saved_size bytes of chunk-boundary states. */
gl_status_t gl_scan_fwd(const gl_scan_desc_t* desc, const void* x, const void* g,
                        const void* eta, const void* alpha, const void* W0,
                        void* y, void* saved, void* ws, size_t ws_bytes,
                        void* stream);

/* Reverse scan: dx, dg, deta, dalpha, dW0 for upstream gradient dy.
 * `saved` is NULL or the buffer filled by gl_scan_fwd with the same inputs. */
gl_status_t gl_scan_bwd(const gl_scan_desc_t* desc, const void* x, const void* g,
                        const void* eta, const void* alpha, const void* W0,
                        const void* dy, const void* saved, void* dx, void* dg,
                        void* deta, void* dalpha, void* dW0, void* ws,
                        size_t ws_bytes, void* stream);

/* gl_scan_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same reverse scan, arguments and results as gl_scan_bwd, without a
 * workspace argument.  Its scratch memory is a static device buffer of 64 MiB
 * per GPU that the library holds until the process ends; nothing is
 * allocated or freed by the call.  A descriptor whose backward needs more
 * scratch than that (gl_scan_workspace_size's bwd figure; passing the
 * forward's `saved` keeps it small) returns GL_ERROR_WORKSPACE_TOO_SMALL before
 * anything is launched.  Every call on one GPU shares that GPU's buffer:
 * calls that overlap in time on one GPU (two streams, two threads) race and
 * must be serialised by the caller.  The buffer keeps the last call's
 * contents; no kernel relies on it being zero. */
gl_status_t gl_scan_bwd_static(const gl_scan_desc_t* desc, const void* x, const void* g,
                               const void* eta, const void* alpha, const void* W0,
                               const void* dy, const void* saved, void* dx, void* dg,
                               void* deta, void* dalpha, void* dW0, void* stream);

/* ---- Deployment: one token at a time, and the prefill -> decode handoff.
 *
 * Once trained, the learner runs token by token: the layer reads out with its
 * cached weight, the costate g of that token comes back, and the cache is
 * advanced by the recurrence's update for that token ("Parallelize the Training, Keep the
 * Learning Serial", cognaptus.com, section "The bottleneck appears before
 * deployment"; ParaTTT news summary, section "Perspective").  The cache is the
 * adaptation D = W - W0 of every sequence-head:
 *
 *   state                    [B][H][d_out][d_in]  state dtype (fp64 if io is
 *                                                 F64, else fp32)
 *
 * These calls take the same descriptor as the scans (B, H, d_in, d_out,
 * io_dtype; chunk, flags and segments are ignored) and follow the same rules:
 * device pointers owned by the caller, 16-byte aligned, outputs must not alias
 * inputs (gl_decode_update updates `state` in place), asynchronous on
 * `stream`, every check before any launch, nothing allocated.  B*H == 0 is a
 * no-op. */

/* Readout of one token against the cache, from the pre-update weight:
 * y = (W0 + D) x.   x [B][H][d_in] io, W0 [H][d_out][d_in] io,
 * y [B][H][d_out] io.  desc->T is ignored. */
gl_status_t gl_decode_readout(const gl_scan_desc_t* desc, const void* x, const void* W0,
                              const void* state, void* y, void* stream);

/* One exact gradient step of the cache: D <- alpha D - eta g x^T (the scan's
 * recurrence for one token).  x [B][H][d_in] io, g [B][H][d_out] io,
 * eta, alpha [B][H] gate dtype.  desc->T is ignored. */
gl_status_t gl_decode_update(const gl_scan_desc_t* desc, const void* x, const void* g,
                             const void* eta, const void* alpha, void* state, void* stream);

/* The steady state of serving, fused: the update of the previous token (once
 * its costate has come back), then the readout of the next one,
 *   D <- alpha_prev D - eta_prev g_prev x_prev^T;   y = (W0 + D) x,
 * in one pass over the state where the shape allows (d_in a multiple of 4
 * with d_in / 4 a power of two), else as gl_decode_update followed by
 * gl_decode_readout.  x_prev, x [B][H][d_in] io, g_prev [B][H][d_out] io,
 * eta_prev, alpha_prev [B][H] gate dtype, W0 [H][d_out][d_in] io,
 * y [B][H][d_out] io; `state` is updated in place.  desc->T is ignored. */
gl_status_t gl_decode_step(const gl_scan_desc_t* desc, const void* x_prev, const void* g_prev,
                           const void* eta_prev, const void* alpha_prev, const void* x,
                           const void* W0, void* state, void* y, void* stream);

/* Hand-over from a prefill of desc->T tokens (the inputs of gl_scan_fwd) to
 * decoding: writes the adaptation after the last token,
 * D_T = sum_t (prod_{s>t} alpha_s)(-eta_t) g_t x_t^T, into `state` (zero for
 * T == 0).  BF16 io with d_in == d_out in {64, 128}: the forward scan's
 * matrix-core arithmetic (bf16 operands, fp32 accumulation: the state the
 * prefill's own readouts used); GL_FLAG_GENERIC or other shapes: fp32 (fp64)
 * vector arithmetic. */
gl_status_t gl_scan_final_state(const gl_scan_desc_t* desc, const void* x, const void* g,
                                const void* eta, const void* alpha, void* state,
                                void* stream);

/* ---- Costate reconstruction and the consistency residual.
 *
 * GradLev trains proposed costates g^ toward the costates the model
 * reconstructs on the trajectory they propose ("Parallelize the Training, Keep
 * the Learning Serial", cognaptus.com, section "The predictor is constrained by
 * the learner it is supposed to reproduce").  For the quadratic token loss
 * l_t = |y_t - r_t|^2 / 2 of the pages' synthetic test, with y the output of
 * gl_scan_fwd driven by g^:
 *
 *   g~_t = y_t - r_t,  res_sq_t = |g^_t - g~_t|^2,  res_max_t = max |g^_t - g~_t|
 *
 * y, target, g_hat, g_tilde [B][H][T][d_out] io; res_sq, res_max [B][H][T]
 * gate dtype.  The residuals are taken with g~ in the gate dtype, before it
 * is rounded to io.  Sweeping g^ <- g~ (scan, then this call) is the Picard
 * iteration of the causal map, whose unique fixed point is the serial
 * learner's costate trajectory.  Same descriptor (d_in, chunk, flags and
 * segments are not used) and rules as the scans; B*H*T == 0 is a no-op. */
gl_status_t gl_costate_quadratic(const gl_scan_desc_t* desc, const void* y, const void* target,
                                 const void* g_hat, void* g_tilde, void* res_sq, void* res_max,
                                 void* stream);

/* ---- The scan with its own read vector and write key.
 *
 *   y_t = (W0' + D_t) q_t,   D_{t+1} = alpha_t D_t - eta_t v_t k_t^T,  D_0 = 0
 *
 * per sequence-head, tokens in order; gl_scan_fwd is the case q = k = x,
 * v = g.  With q = u, k = g, v = x and W0' = W0^T it is the transpose read
 * (W0 + D_t)^T u_t that carries a hidden costate back through an adapted
 * layer ("Parallelize the Training, Keep the Learning Serial", cognaptus.com,
 * section "The synthetic test checks the mechanism, not model quality"); with
 * q = x, k = x_bar, v = g a write key of its own (section "Once the gradient
 * signals are known, the weight trajectory becomes parallelizable").
 * desc->d_in = dk (length of q and k), desc->d_out = dv (length of v and y);
 * chunk and segments are not used; GL_FLAG_GENERIC keeps every shape on the
 * token-serial vector kernel.  q, k [B][H][T][dk] io, v, y [B][H][T][dv] io,
 * eta, alpha [B][H][T] gate dtype, W0 [H][dv][dk] io, or [H][dk][dv] when
 * w0_transposed != 0.  Same rules as gl_scan_fwd; B*H*T == 0 is a no-op.
 * bf16 with dk = dv = 64 runs on the matrix cores (the chunked forward with a
 * read tile of its own); bf16 with dk = dv = 128 does so only through
 * gl_scan_qkv_fwd_ws with a workspace (here it takes the token-serial kernel);
 * every other case runs the token-serial kernel. */
gl_status_t gl_scan_qkv_fwd(const gl_scan_desc_t* desc, const void* q, const void* k,
                            const void* v, const void* eta, const void* alpha, const void* W0,
                            int w0_transposed, void* y, void* stream);

/* Workspace bytes gl_scan_qkv_fwd_ws uses: the state of the write-key scan
 * entering every group of eight 64-token chunks (bf16,
 * B*H*ceil(T/512)*dv*dk elements) for bf16 with dk = dv = 128 without
 * GL_FLAG_GENERIC; 0 otherwise. */
gl_status_t gl_scan_qkv_fwd_workspace_size(const gl_scan_desc_t* desc, size_t* ws_bytes);

/* gl_scan_qkv_fwd with a caller workspace (ws_bytes from
 * gl_scan_qkv_fwd_workspace_size; ws may be NULL when that is 0).  For bf16
 * with dk = dv = 128 it runs in two launches on the matrix cores: the
 * forward scan's state-only pass writes the state entering every group of
 * eight chunks into ws, then the groups' outputs are formed in parallel, each
 * group walking its chunks in order with the state in registers.  A smaller
 * workspace returns GL_ERROR_WORKSPACE_TOO_SMALL before any launch.  Results
 * as gl_scan_qkv_fwd. */
gl_status_t gl_scan_qkv_fwd_ws(const gl_scan_desc_t* desc, const void* q, const void* k,
                               const void* v, const void* eta, const void* alpha, const void* W0,
                               int w0_transposed, void* y, void* ws, size_t ws_bytes,
                               void* stream);

/* The reverse scan of gl_scan_qkv_fwd: for upstream dy [B][H][T][dv] io,
 * the gradients of L = sum_t <dy_t, y_t> w.r.t. q, k, v, eta, alpha and W0',
 *
 *   A_T = 0,  A_{t} = alpha_t A_{t+1} + dy_t q_t^T       (A_t = dL / dD_t)
 *   dq_t = (W0' + D_t)^T dy_t,       dk_t = -eta_t A_{t+1}^T v_t,
 *   dv_t = -eta_t A_{t+1} k_t,       deta_t = -v_t^T A_{t+1} k_t,
 *   dalpha_t = <A_{t+1}, D_t>,       dW0' = sum_b sum_t dy_t q_t^T
 *
 * (the same adjoint as gl_scan_bwd, whose dx is dq + dk when q = k = x).
 * dq, dk [B][H][T][dk] io; dv [B][H][T][dv] io; deta, dalpha [B][H][T] gate
 * dtype; dW0 [H][dv][dk] gate dtype, or [H][dk][dv] when w0_transposed != 0
 * (the layout W0 is passed in).  The chunk states of the forward are
 * recomputed inside the workspace `ws` of gl_scan_qkv_workspace_size bytes.
 * bf16 with dk = dv in {64, 128} (without GL_FLAG_GENERIC) runs
 * chunk-parallel on the matrix cores: the forward's chunk-start states
 * (bf16), then per group of 64-token chunks (sixteen; down to four when
 * the problem is small) the adjoint increment,
 * decay and dW0 share, the adjoint carry over groups (fp32), and the
 * gradients of every chunk with the adjoint walked right to left through
 * its group (at 128, with W0' not given transposed, a transposed copy of it
 * in the workspace first); every pointer must then be 16-byte aligned.  Every other case (and GL_FLAG_GENERIC) runs
 * portable chunked VALU kernels, any 1 <= dk, dv <= 128 (chunk 32, F64: 8).
 * Same rules as gl_scan_bwd; B*H*T == 0 writes the zero dW0 only. */
gl_status_t gl_scan_qkv_workspace_size(const gl_scan_desc_t* desc, size_t* ws_bytes);
gl_status_t gl_scan_qkv_bwd(const gl_scan_desc_t* desc, const void* q, const void* k,
                            const void* v, const void* eta, const void* alpha, const void* W0,
                            int w0_transposed, const void* dy, void* dq, void* dk, void* dv,
                            void* deta, void* dalpha, void* dW0, void* ws, size_t ws_bytes,
                            void* stream);

/* Static description of a status code. */
const char* gl_status_string(gl_status_t status);

/* Text of the last GL_ERROR_HIP / validation failure on the calling thread. */
const char* gl_last_error(void);

/* Name of the kernel family the library selects for desc ("generic-f64",
 * "mfma-bf16-d128", ...), or NULL if desc is unsupported. */
const char* gl_scan_path_name(const gl_scan_desc_t* desc);

#ifdef __cplusplus
}
#endif
#endif /* GL_SCAN_H */
