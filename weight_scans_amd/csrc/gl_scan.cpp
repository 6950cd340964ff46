// gl_scan.cpp -- host side of the C ABI (include/gl_scan.h): argument checks,
// kernel-family selection, workspace layout and launches.  Every check runs
// before the first launch; nothing here allocates device memory.
#include "gl_scan.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

void set_err(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

gl_status_t fail(gl_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Automatic segmenting: when one pass has fewer work-groups than the GPU has
// compute units (256 on MI355X), each sequence is cut into segments of at
// least kMinSegChunks chunks so that the pass fills the chip.
constexpr int64_t kSegTargetGroups = 256;
constexpr int kMinSegChunks = 16;
// Above this many backward segments the entering adjoints are composed by one
// combine launch rather than in every fused work-group's set-up.
constexpr int kBwdCombineAbove = 4;
// Chunks per segment of the adjoint-only pass, at least.
constexpr int kLamMinChunks = 8;

// Everything the launches need, derived from the descriptor alone so that the
// forward and the backward agree on the layout of `saved`.
struct Plan {
  int io = 0;
  bool mfma = false;        // bf16 matrix-core kernels
  bool mf = false;          // fp32 / fp64 matrix-core kernels
  bool out_f32 = false;     // y, dx, dg in fp32 (bf16 io)
  int chunk = 0, n_chunks = 0, ckpt_every = 1, n_ckpt = 0, n_tiles = 0;
  size_t comp = 8;          // bytes of the compute / gate / state type
  size_t saved_bytes = 0;   // chunk-boundary states
  size_t state_elem = 4;    // bytes per stored state element
  size_t part_bytes = 0;    // deta + dalpha partials
  size_t dw_bytes = 0;      // dW0 partials (per batch entry, per segment)
  int n_seg = 1, seg_chunks = 0;
  size_t seg_bytes = 0;     // per-segment states (fp32) + summed log2 alpha
  size_t seg_state_bytes = 0;
  int dw_groups = 1;        // dW0 partials per (b, h)
  // fused backward (matrix-core kernels, d = 64 and 128): its own segment count (a
  // work-group per segment and sequence-head), deta / dalpha written directly
  bool fused = false;
  int bwd_nseg = 1, bwd_seg_chunks = 0;
  // the adjoint-only pass: lam_r of its segments per fused segment
  int lam_r = 1, lam_n = 1, lam_seg_chunks = 0;
  size_t bwd_seg_bytes = 0, bwd_seg_state_bytes = 0;
  const char* name = "";
};

gl_status_t make_plan(const gl_scan_desc_t* d, Plan* p) {
  if (!d) return fail(GL_ERROR_INVALID_VALUE, "desc is NULL");
  if (d->B < 0 || d->H < 0 || d->T < 0)
    return fail(GL_ERROR_INVALID_VALUE, "negative B/H/T (%lld, %lld, %lld)", (long long)d->B,
                (long long)d->H, (long long)d->T);
  if (d->d_in < 1 || d->d_out < 1)
    return fail(GL_ERROR_INVALID_VALUE, "d_in and d_out must be >= 1");
  if (d->io_dtype < GL_DTYPE_F64 || d->io_dtype > GL_DTYPE_BF16)
    return fail(GL_ERROR_INVALID_VALUE, "unknown io_dtype %d", d->io_dtype);
  if ((d->flags & ~(GL_FLAG_GENERIC | GL_FLAG_OUT_F32)) != 0)
    return fail(GL_ERROR_INVALID_VALUE, "unknown flags");
  if ((d->flags & GL_FLAG_OUT_F32) && d->io_dtype == GL_DTYPE_F64)
    return fail(GL_ERROR_NOT_SUPPORTED, "GL_FLAG_OUT_F32 with fp64 io");
  if (d->segments > (1u << 20)) return fail(GL_ERROR_INVALID_VALUE, "segments above 2^20");
  if (d->chunk < 0) return fail(GL_ERROR_INVALID_VALUE, "negative chunk");
  if (d->d_in > gls::kGenericMaxD || d->d_out > gls::kGenericMaxD)
    return fail(GL_ERROR_NOT_SUPPORTED, "d_in/d_out above %d", gls::kGenericMaxD);
  if (d->B * d->H > 0x7fffffffLL)
    return fail(GL_ERROR_NOT_SUPPORTED, "B*H above 2^31-1");

  p->io = d->io_dtype;
  p->comp = (p->io == GL_DTYPE_F64) ? 8 : 4;
  p->out_f32 = (d->flags & GL_FLAG_OUT_F32) && p->io == GL_DTYPE_BF16;
  const bool mfma_shape = p->io == GL_DTYPE_BF16 && d->d_in == d->d_out &&
                          (d->d_in == 64 || d->d_in == 128) && !(d->flags & GL_FLAG_GENERIC);
  const size_t dd = static_cast<size_t>(d->d_in) * static_cast<size_t>(d->d_out);
  const size_t BH = static_cast<size_t>(d->B) * static_cast<size_t>(d->H);
  if (mfma_shape && (d->chunk == 0 || d->chunk == gls::kMfmaChunk)) {
    p->mfma = true;
    p->chunk = gls::kMfmaChunk;
    p->n_tiles = 1;  // the fused backward writes deta / dalpha itself (no tile partials)
    p->name = d->d_in == 64 ? "mfma-bf16-d64" : "mfma-bf16-d128";
    p->state_elem = 2;  // bf16 chunk-start states
  } else if (p->io != GL_DTYPE_BF16 && !(d->flags & GL_FLAG_GENERIC) &&
             (d->chunk == 0 || d->chunk == gls::kMfmaChunk) &&
             gls::mf_shape_ok(p->io, static_cast<int>(d->d_in), static_cast<int>(d->d_out))) {
    p->mf = true;
    p->chunk = gls::kMfmaChunk;
    p->n_tiles = 1;
    p->name = p->io == GL_DTYPE_F64 ? "mfma-f64" : "mfma-f32";
    p->state_elem = p->comp;
    if (d->segments > 1)
      return fail(GL_ERROR_NOT_SUPPORTED, "segments apply to the bf16 matrix-core kernels only");
  } else {
    if (d->chunk != 0 && !gls::generic_chunk_ok(p->io, d->chunk))
      return fail(GL_ERROR_NOT_SUPPORTED, "chunk %d not supported for this dtype/shape", d->chunk);
    p->mfma = false;
    p->chunk = d->chunk ? d->chunk : gls::generic_default_chunk(p->io);
    p->n_tiles = static_cast<int>((std::max(d->d_in, d->d_out) + gls::kGenericTile - 1) /
                                  gls::kGenericTile);
    p->name = (p->io == GL_DTYPE_F64) ? "generic-f64"
              : (p->io == GL_DTYPE_F32) ? "generic-f32"
              : p->out_f32 ? "generic-bf16-out-f32" : "generic-bf16";
    p->state_elem = p->comp;
    if (d->segments > 1)
      return fail(GL_ERROR_NOT_SUPPORTED, "segments apply to the matrix-core kernels only");
  }
  p->n_chunks = static_cast<int>((d->T + p->chunk - 1) / p->chunk);
  int nseg = 1;
  if (p->mfma && p->n_chunks > 0) {
    const int64_t groups = static_cast<int64_t>(BH) * (d->d_in / 32);
    if (d->segments > 0) {
      nseg = static_cast<int>(d->segments);
    } else if (groups > 0 && groups < kSegTargetGroups) {
      nseg = static_cast<int>(std::min<int64_t>((kSegTargetGroups + groups - 1) / groups,
                                                p->n_chunks / kMinSegChunks));
    }
    nseg = std::max(1, std::min(nseg, p->n_chunks));
  }
  p->seg_chunks = p->n_chunks > 0 ? (p->n_chunks + nseg - 1) / nseg : 0;
  p->n_seg = p->seg_chunks > 0 ? (p->n_chunks + p->seg_chunks - 1) / p->seg_chunks : 1;
  if (p->n_seg > 1) {
    p->seg_state_bytes = round_up(BH * p->n_seg * dd * sizeof(float));
    p->seg_bytes = p->seg_state_bytes + round_up(BH * p->n_seg * sizeof(float));
  }
  p->ckpt_every = 1;
  p->n_ckpt = p->n_chunks;
  p->saved_bytes = round_up(BH * p->n_ckpt * dd * p->state_elem);
  p->part_bytes = p->mf ? 0 : round_up(static_cast<size_t>(p->n_tiles) * BH * d->T * p->comp);
  p->fused = p->mfma;
  if (p->fused && p->n_chunks > 0) {
    int nb = 1;
    if (d->segments > 0) {
      nb = static_cast<int>(d->segments);
    } else if (BH > 0 && static_cast<int64_t>(BH) < kSegTargetGroups) {
      nb = static_cast<int>(std::min<int64_t>((kSegTargetGroups + BH - 1) / BH,
                                              p->n_chunks / kMinSegChunks));
    }
    nb = std::max(1, std::min(nb, p->n_chunks));
    p->bwd_seg_chunks = (p->n_chunks + nb - 1) / nb;
    p->bwd_nseg = (p->n_chunks + p->bwd_seg_chunks - 1) / p->bwd_seg_chunks;
    // With few fused segments the adjoint-only pass (one work-group per
    // segment and row tile, walking its chunks in order) would leave CUs
    // idle; it runs on segments lam_r times finer instead, as long as every
    // fused work-group still composes at most kBwdCombineAbove of them.
    p->lam_r = 1;
    if (p->bwd_nseg > 1 && p->bwd_nseg <= kBwdCombineAbove) {
      int r = std::min(kBwdCombineAbove / (p->bwd_nseg - 1), p->bwd_seg_chunks / kLamMinChunks);
      while (r > 1 && p->bwd_seg_chunks % r) --r;
      p->lam_r = std::max(1, r);
    }
    p->lam_seg_chunks = p->bwd_seg_chunks / p->lam_r;
    p->lam_n = (p->n_chunks + p->lam_seg_chunks - 1) / p->lam_seg_chunks;
    if (p->bwd_nseg > 1) {
      p->bwd_seg_state_bytes = round_up(BH * p->lam_n * dd * sizeof(float));
      p->bwd_seg_bytes = p->bwd_seg_state_bytes + round_up(BH * p->lam_n * sizeof(float));
    }
  }
  if (p->fused) p->part_bytes = 0;
  p->dw_groups = p->fused ? p->bwd_nseg : p->n_seg;
  if (p->mf) {
    // per-chunk decays (fwd); adjoint leaving every chunk + decays (bwd); a
    // dW0 share per chunk
    if (static_cast<int64_t>(BH) * std::max(p->n_chunks, 1) > 0x7fffffffLL)
      return fail(GL_ERROR_NOT_SUPPORTED, "B*H*chunks above 2^31-1");
    p->seg_bytes = round_up(BH * p->n_chunks * p->comp);
    p->bwd_seg_state_bytes = round_up(BH * p->n_chunks * dd * p->comp);
    p->bwd_seg_bytes = p->bwd_seg_state_bytes + p->seg_bytes;
    p->dw_groups = std::max(p->n_chunks, 1);
  }
  p->dw_bytes = round_up(BH * dd * p->comp * p->dw_groups);
  return GL_SUCCESS;
}

// fwd workspace: segment buffers; the fp32 / fp64 matrix-core kernels also
// keep the chunk-boundary states there when the call has no `saved` buffer
size_t fwd_ws(const Plan& p, bool have_saved) {
  return p.seg_bytes + (p.mf && !have_saved ? p.saved_bytes : 0);
}

// bwd workspace: deta / dalpha partials, dW0 partials, segment buffers (also
// used by the state recompute, which runs first), recomputed states
size_t bwd_ws(const Plan& p, bool have_saved) {
  return 2 * p.part_bytes + p.dw_bytes + std::max(p.seg_bytes, p.bwd_seg_bytes) +
         (have_saved ? 0 : p.saved_bytes);
}

bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; }

gl_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return GL_SUCCESS;
  set_err("%s: %s", where, hipGetErrorString(e));
  return GL_ERROR_HIP;
}

gls::FwdArgs fwd_args(const gl_scan_desc_t* d, const Plan& p, const void* x, const void* g,
                      const void* eta, const void* alpha, const void* W0, void* y,
                      void* states) {
  gls::FwdArgs a;
  a.x = x; a.g = g; a.eta = eta; a.alpha = alpha; a.W0 = W0; a.y = y; a.states = states;
  a.B = d->B; a.H = d->H; a.T = d->T;
  a.d_in = static_cast<int>(d->d_in); a.d_out = static_cast<int>(d->d_out);
  a.chunk = p.chunk; a.n_chunks = p.n_chunks; a.ckpt_every = p.ckpt_every; a.n_ckpt = p.n_ckpt;
  a.seg_chunks = p.seg_chunks; a.n_seg = p.n_seg;
  a.out_f32 = p.out_f32;
  return a;
}

// The forward scan.  With segments (a buffer of p.seg_bytes at seg_ws): a
// state-only pass per segment from a zero start, the exclusive affine scan
// over segments, then the full pass per segment from its incoming state.
hipError_t launch_fwd(const Plan& p, const gls::FwdArgs& a, void* seg_ws, hipStream_t s) {
  if (p.mf) {
    gls::FwdArgs am = a;
    am.mf_gam = seg_ws;
    return gls::launch_mf_fwd(p.io, am, s);
  }
  if (!p.mfma) return gls::launch_generic_fwd(p.io, a, s);
  if (p.n_seg <= 1) return gls::launch_mfma_fwd(a, s);
  float* seg = static_cast<float*>(seg_ws);
  float* lg = reinterpret_cast<float*>(static_cast<char*>(seg_ws) + p.seg_state_bytes);
  gls::FwdArgs a1 = a;
  a1.y = nullptr;
  a1.states = nullptr;
  a1.seg_out = seg;
  a1.seg_lg = lg;
  hipError_t e = gls::launch_mfma_fwd(a1, s);
  if (e != hipSuccess) return e;
  e = gls::launch_seg_combine(seg, lg, a.B * a.H, p.n_seg, a.d_in * a.d_out, false, s);
  if (e != hipSuccess) return e;
  gls::FwdArgs a3 = a;
  a3.seg_in = seg;
  return gls::launch_mfma_fwd(a3, s);
}

// Checks shared by the deployment calls (the descriptor fields they use).
gl_status_t check_dec(const gl_scan_desc_t* d, bool need_T) {
  if (!d) return fail(GL_ERROR_INVALID_VALUE, "desc is NULL");
  if (d->B < 0 || d->H < 0 || (need_T && d->T < 0))
    return fail(GL_ERROR_INVALID_VALUE, "negative B/H/T");
  if (d->d_in < 1 || d->d_out < 1)
    return fail(GL_ERROR_INVALID_VALUE, "d_in and d_out must be >= 1");
  if (d->io_dtype < GL_DTYPE_F64 || d->io_dtype > GL_DTYPE_BF16)
    return fail(GL_ERROR_INVALID_VALUE, "unknown io_dtype %d", d->io_dtype);
  if (d->d_in > gls::kGenericMaxD || d->d_out > gls::kGenericMaxD)
    return fail(GL_ERROR_NOT_SUPPORTED, "d_in/d_out above %d", gls::kGenericMaxD);
  if (d->B * d->H > 0x7fffffffLL) return fail(GL_ERROR_NOT_SUPPORTED, "B*H above 2^31-1");
  return GL_SUCCESS;
}

gl_status_t check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* q : ps) {
    if (!q) return fail(GL_ERROR_INVALID_VALUE, "NULL input or output pointer");
    if (misaligned(q)) return fail(GL_ERROR_MISALIGNED, "pointer %p not 16-byte aligned", q);
  }
  return GL_SUCCESS;
}

gls::DecArgs dec_args(const gl_scan_desc_t* d) {
  gls::DecArgs a{};
  a.B = d->B; a.H = d->H; a.T = d->T;
  a.d_in = static_cast<int>(d->d_in); a.d_out = static_cast<int>(d->d_out);
  return a;
}

}  // namespace

extern "C" {

gl_status_t gl_scan_saved_size(const gl_scan_desc_t* desc, size_t* saved_bytes) {
  Plan p;
  gl_status_t st = make_plan(desc, &p);
  if (st != GL_SUCCESS) return st;
  if (!saved_bytes) return fail(GL_ERROR_INVALID_VALUE, "saved_bytes is NULL");
  *saved_bytes = p.saved_bytes;
  return GL_SUCCESS;
}

gl_status_t gl_scan_workspace_size(const gl_scan_desc_t* desc, int have_saved,
                                   size_t* fwd_ws_bytes, size_t* bwd_ws_bytes) {
  Plan p;
  gl_status_t st = make_plan(desc, &p);
  if (st != GL_SUCCESS) return st;
  if (fwd_ws_bytes) *fwd_ws_bytes = fwd_ws(p, have_saved != 0);
  if (bwd_ws_bytes) *bwd_ws_bytes = bwd_ws(p, have_saved != 0);
  return GL_SUCCESS;
}

gl_status_t gl_scan_fwd(const gl_scan_desc_t* desc, const void* x, const void* g,
                        const void* eta, const void* alpha, const void* W0, void* y,
                        void* saved, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  gl_status_t st = make_plan(desc, &p);
  if (st != GL_SUCCESS) return st;
  if (desc->B * desc->H * desc->T == 0) return GL_SUCCESS;
  if (!x || !g || !eta || !alpha || !W0 || !y)
    return fail(GL_ERROR_INVALID_VALUE, "NULL input or output pointer");
  for (const void* q : {x, g, eta, alpha, W0, static_cast<const void*>(y),
                        static_cast<const void*>(saved)})
    if (q && misaligned(q)) return fail(GL_ERROR_MISALIGNED, "pointer %p not 16-byte aligned", q);
  const size_t need = fwd_ws(p, saved != nullptr);
  if (need > 0) {
    if (!ws) return fail(GL_ERROR_INVALID_VALUE, "workspace is NULL");
    if (misaligned(ws)) return fail(GL_ERROR_MISALIGNED, "workspace not 16-byte aligned");
    if (ws_bytes < need)
      return fail(GL_ERROR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", ws_bytes, need);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* states = saved;
  if (p.mf && !saved) states = static_cast<char*>(ws) + p.seg_bytes;
  return hip_status(launch_fwd(p, fwd_args(desc, p, x, g, eta, alpha, W0, y, states), ws, s),
                    "forward launch");
}

gl_status_t gl_scan_bwd(const gl_scan_desc_t* desc, const void* x, const void* g,
                        const void* eta, const void* alpha, const void* W0, const void* dy,
                        const void* saved, void* dx, void* dg, void* deta, void* dalpha,
                        void* dW0, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  gl_status_t st = make_plan(desc, &p);
  if (st != GL_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t dd = static_cast<size_t>(desc->d_in) * static_cast<size_t>(desc->d_out);
  if (desc->B * desc->H * desc->T == 0) {
    // empty batch / sequence: dW0 is the (zero) empty sum
    if (desc->H == 0) return GL_SUCCESS;
    if (!dW0) return fail(GL_ERROR_INVALID_VALUE, "dW0 is NULL");
    if (misaligned(dW0)) return fail(GL_ERROR_MISALIGNED, "dW0 not 16-byte aligned");
    return hip_status(gls::launch_clear(dW0, desc->H * dd * p.comp, s), "dW0 clear");
  }
  if (!x || !g || !eta || !alpha || !W0 || !dy || !dx || !dg || !deta || !dalpha || !dW0)
    return fail(GL_ERROR_INVALID_VALUE, "NULL input or output pointer");
  if (!ws) return fail(GL_ERROR_INVALID_VALUE, "workspace is NULL");
  for (const void* q : {x, g, eta, alpha, W0, dy, saved, static_cast<const void*>(dx),
                        static_cast<const void*>(dg), static_cast<const void*>(deta),
                        static_cast<const void*>(dalpha), static_cast<const void*>(dW0),
                        static_cast<const void*>(ws)})
    if (q && misaligned(q)) return fail(GL_ERROR_MISALIGNED, "pointer %p not 16-byte aligned", q);
  const size_t need = bwd_ws(p, saved != nullptr);
  if (ws_bytes < need)
    return fail(GL_ERROR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", ws_bytes, need);

  char* w = static_cast<char*>(ws);
  void* part_eta = w;
  void* part_alpha = w + p.part_bytes;
  void* part_dW0 = w + 2 * p.part_bytes;
  char* seg_ws = w + 2 * p.part_bytes + p.dw_bytes;
  char* rec = seg_ws + std::max(p.seg_bytes, p.bwd_seg_bytes);
  const void* states = saved;
  if (!states) {
    st = hip_status(
        launch_fwd(p, fwd_args(desc, p, x, g, eta, alpha, W0, nullptr, rec), seg_ws, s),
        "state recompute launch");
    if (st != GL_SUCCESS) return st;
    states = rec;
  }

  gls::BwdArgs b;
  b.x = x; b.g = g; b.eta = eta; b.alpha = alpha; b.W0 = W0; b.dy = dy; b.states = states;
  b.dx = dx; b.dg = dg; b.part_eta = part_eta; b.part_alpha = part_alpha; b.part_dW0 = part_dW0;
  b.B = desc->B; b.H = desc->H; b.T = desc->T;
  b.d_in = static_cast<int>(desc->d_in); b.d_out = static_cast<int>(desc->d_out);
  b.chunk = p.chunk; b.n_chunks = p.n_chunks; b.ckpt_every = p.ckpt_every; b.n_ckpt = p.n_ckpt;
  b.n_tiles = p.n_tiles;
  b.seg_chunks = p.seg_chunks; b.n_seg = p.n_seg;
  b.out_f32 = p.out_f32;
  if (p.mf) {
    b.deta_out = deta;
    b.dalpha_out = dalpha;
    b.mf_lam = seg_ws;
    b.mf_gam = seg_ws + p.bwd_seg_state_bytes;
    st = hip_status(gls::launch_mf_bwd(p.io, b, s), "backward launch");
  } else if (!p.mfma) {
    st = hip_status(gls::launch_generic_bwd(p.io, b, s), "backward launch");
  } else {
    // one work-group per (segment, sequence-head) walks its chunks from the
    // right; with segments, an adjoint-only pass gives each segment's own
    // adjoint, from which every work-group composes the one entering it
    gls::BwdArgs bf = b;
    bf.seg_chunks = p.bwd_seg_chunks;
    bf.n_seg = p.bwd_nseg;
    bf.dalpha_out = dalpha;
    bf.deta_out = deta;
    if (p.bwd_nseg > 1) {
      float* seg = reinterpret_cast<float*>(seg_ws);
      float* lg = reinterpret_cast<float*>(seg_ws + p.bwd_seg_state_bytes);
      gls::BwdArgs bs = bf;
      bs.seg_out = seg;
      bs.seg_lg = lg;
      bs.seg_chunks = p.lam_seg_chunks;
      bs.n_seg = p.lam_n;
      bs.seg_first = p.lam_r;  // the segments inside fused segment 0 are never needed
      st = hip_status(gls::launch_mfma_bwd_lam(bs, s), "backward segment pass");
      bf.seg_lam = seg;
      bf.lam_r = p.lam_r;
      bf.lam_n = p.lam_n;
      if (p.bwd_nseg > kBwdCombineAbove) {
        // the adjoint entering every segment, composed from the right in one
        // launch (in its set-up a work-group would wait for one load per
        // segment to its right, one after another)
        if (st == GL_SUCCESS)
          st = hip_status(gls::launch_seg_combine(seg, lg, b.B * b.H, p.bwd_nseg,
                                                  b.d_in * b.d_out, true, s),
                          "backward segment combine");
        bf.seg_lg_in = nullptr;
      } else {
        bf.seg_lg_in = lg;  // few segments: composed by the fused kernel itself
      }
    }
    if (st == GL_SUCCESS)
      st = hip_status(b.d_in == 64 ? gls::launch_mfma_bwd_f64(bf, s) : gls::launch_mfma_bwd_f128(bf, s),
                      "fused backward");
  }
  if (st != GL_SUCCESS) return st;

  gls::FinArgs f;
  f.part_eta = part_eta; f.part_alpha = part_alpha; f.part_dW0 = part_dW0;
  f.deta = deta; f.dalpha = dalpha; f.dW0 = dW0;
  f.B = desc->B; f.H = desc->H; f.T = desc->T;
  f.d_in = b.d_in; f.d_out = b.d_out; f.n_tiles = p.n_tiles; f.n_seg = p.dw_groups;
  f.alpha_done = p.fused || p.mf;
  f.eta_done = p.fused || p.mf;
  return hip_status(gls::launch_finalize(p.io, f, s), "finalize launch");
}

gl_status_t gl_scan_bwd_static(const gl_scan_desc_t* desc, const void* x, const void* g,
                               const void* eta, const void* alpha, const void* W0,
                               const void* dy, const void* saved, void* dx, void* dg,
                               void* deta, void* dalpha, void* dW0, void* stream) {
  Plan p;
  gl_status_t st = make_plan(desc, &p);
  if (st != GL_SUCCESS) return st;
  if (desc->B * desc->H * desc->T == 0)  // only the zero dW0: no scratch
    return gl_scan_bwd(desc, x, g, eta, alpha, W0, dy, saved, dx, dg, deta, dalpha, dW0,
                       nullptr, 0, stream);
  const size_t need = bwd_ws(p, saved != nullptr);
  if (need > gls::kStaticScratchBytes)
    return fail(GL_ERROR_WORKSPACE_TOO_SMALL,
                "this backward needs %zu bytes of scratch; the static scratch holds %zu "
                "(pass the forward's saved states, or use gl_scan_bwd with a workspace)",
                need, gls::kStaticScratchBytes);
  void* ws = nullptr;
  st = hip_status(gls::static_scratch(&ws), "static scratch address");
  if (st != GL_SUCCESS) return st;
  return gl_scan_bwd(desc, x, g, eta, alpha, W0, dy, saved, dx, dg, deta, dalpha, dW0, ws,
                     gls::kStaticScratchBytes, stream);
}

gl_status_t gl_decode_readout(const gl_scan_desc_t* desc, const void* x, const void* W0,
                              const void* state, void* y, void* stream) {
  gl_status_t st = check_dec(desc, false);
  if (st != GL_SUCCESS || desc->B * desc->H == 0) return st;
  st = check_ptrs({x, W0, state, y});
  if (st != GL_SUCCESS) return st;
  gls::DecArgs a = dec_args(desc);
  a.x = x; a.W0 = W0; a.state = const_cast<void*>(state); a.y = y;
  return hip_status(gls::launch_decode_readout(desc->io_dtype, a, static_cast<hipStream_t>(stream)),
                    "decode readout launch");
}

gl_status_t gl_decode_update(const gl_scan_desc_t* desc, const void* x, const void* g,
                             const void* eta, const void* alpha, void* state, void* stream) {
  gl_status_t st = check_dec(desc, false);
  if (st != GL_SUCCESS || desc->B * desc->H == 0) return st;
  st = check_ptrs({x, g, eta, alpha, state});
  if (st != GL_SUCCESS) return st;
  gls::DecArgs a = dec_args(desc);
  a.x = x; a.g = g; a.eta = eta; a.alpha = alpha; a.state = state;
  return hip_status(gls::launch_decode_update(desc->io_dtype, a, static_cast<hipStream_t>(stream)),
                    "decode update launch");
}

gl_status_t gl_decode_step(const gl_scan_desc_t* desc, const void* x_prev, const void* g_prev,
                           const void* eta_prev, const void* alpha_prev, const void* x,
                           const void* W0, void* state, void* y, void* stream) {
  gl_status_t st = check_dec(desc, false);
  if (st != GL_SUCCESS || desc->B * desc->H == 0) return st;
  st = check_ptrs({x_prev, g_prev, eta_prev, alpha_prev, x, W0, state, y});
  if (st != GL_SUCCESS) return st;
  gls::DecArgs a = dec_args(desc);
  a.x_prev = x_prev; a.g = g_prev; a.eta = eta_prev; a.alpha = alpha_prev;
  a.x = x; a.W0 = W0; a.state = state; a.y = y;
  return hip_status(gls::launch_decode_step(desc->io_dtype, a, static_cast<hipStream_t>(stream)),
                    "decode step launch");
}

gl_status_t gl_scan_final_state(const gl_scan_desc_t* desc, const void* x, const void* g,
                                const void* eta, const void* alpha, void* state,
                                void* stream) {
  gl_status_t st = check_dec(desc, true);
  if (st != GL_SUCCESS || desc->B * desc->H == 0) return st;
  st = desc->T > 0 ? check_ptrs({x, g, eta, alpha, state}) : check_ptrs({state});
  if (st != GL_SUCCESS) return st;
  const bool mfma = desc->io_dtype == GL_DTYPE_BF16 && desc->d_in == desc->d_out &&
                    (desc->d_in == 64 || desc->d_in == 128) && desc->T > 0 &&
                    !(desc->flags & GL_FLAG_GENERIC);
  if (mfma) {
    // the forward kernel's state-only instance over one segment: D_T from a
    // zero start, on the matrix cores (the scan's own arithmetic)
    gls::FwdArgs f;
    f.x = x; f.g = g; f.eta = eta; f.alpha = alpha;
    f.W0 = x;  // not read by the state-only instance
    f.y = nullptr;
    f.states = nullptr;
    f.B = desc->B; f.H = desc->H; f.T = desc->T;
    f.d_in = static_cast<int>(desc->d_in); f.d_out = static_cast<int>(desc->d_out);
    f.chunk = gls::kMfmaChunk;
    f.n_chunks = static_cast<int>((desc->T + gls::kMfmaChunk - 1) / gls::kMfmaChunk);
    f.ckpt_every = 1; f.n_ckpt = f.n_chunks;
    f.seg_chunks = f.n_chunks; f.n_seg = 1;
    f.seg_out = static_cast<float*>(state);
    return hip_status(gls::launch_mfma_final_state(f, static_cast<hipStream_t>(stream)),
                      "final state launch");
  }
  gls::DecArgs a = dec_args(desc);
  a.x = x; a.g = g; a.eta = eta; a.alpha = alpha; a.state = state;
  return hip_status(gls::launch_final_state(desc->io_dtype, a, static_cast<hipStream_t>(stream)),
                    "final state launch");
}

gl_status_t gl_costate_quadratic(const gl_scan_desc_t* desc, const void* y, const void* target,
                                 const void* g_hat, void* g_tilde, void* res_sq, void* res_max,
                                 void* stream) {
  gl_status_t st = check_dec(desc, true);
  if (st != GL_SUCCESS || desc->B * desc->H * desc->T == 0) return st;
  st = check_ptrs({y, target, g_hat, g_tilde, res_sq, res_max});
  if (st != GL_SUCCESS) return st;
  gls::CostArgs a;
  a.y = y; a.target = target; a.g_hat = g_hat; a.g_tilde = g_tilde;
  a.res_sq = res_sq; a.res_max = res_max;
  a.rows = desc->B * desc->H * desc->T;
  a.d_out = static_cast<int>(desc->d_out);
  return hip_status(gls::launch_costate(desc->io_dtype, a, static_cast<hipStream_t>(stream)),
                    "costate launch");
}

gl_status_t gl_scan_qkv_fwd(const gl_scan_desc_t* desc, const void* q, const void* k,
                            const void* v, const void* eta, const void* alpha, const void* W0,
                            int w0_transposed, void* y, void* stream) {
  return gl_scan_qkv_fwd_ws(desc, q, k, v, eta, alpha, W0, w0_transposed, y, nullptr, 0, stream);
}

namespace {
bool qkv_two_pass(const gl_scan_desc_t* d) {
  return !(d->flags & GL_FLAG_GENERIC) &&
         gls::mfma_qkv_two_pass(d->io_dtype, static_cast<int>(d->d_in), static_cast<int>(d->d_out));
}
}  // namespace

gl_status_t gl_scan_qkv_fwd_workspace_size(const gl_scan_desc_t* desc, size_t* ws_bytes) {
  gl_status_t st = check_dec(desc, true);
  if (st != GL_SUCCESS) return st;
  if (!ws_bytes) return fail(GL_ERROR_INVALID_VALUE, "ws_bytes is NULL");
  *ws_bytes = qkv_two_pass(desc) ? round_up(gls::mfma_qkv_states_bytes(desc->B * desc->H, desc->T)) : 0;
  return GL_SUCCESS;
}

gl_status_t gl_scan_qkv_fwd_ws(const gl_scan_desc_t* desc, const void* q, const void* k,
                               const void* v, const void* eta, const void* alpha, const void* W0,
                               int w0_transposed, void* y, void* ws, size_t ws_bytes,
                               void* stream) {
  gl_status_t st = check_dec(desc, true);
  if (st != GL_SUCCESS || desc->B * desc->H * desc->T == 0) return st;
  st = check_ptrs({q, k, v, eta, alpha, W0, y});
  if (st != GL_SUCCESS) return st;
  if (qkv_two_pass(desc) && ws) {
    const size_t need = round_up(gls::mfma_qkv_states_bytes(desc->B * desc->H, desc->T));
    if (ws_bytes < need)
      return fail(GL_ERROR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", ws_bytes, need);
    for (const void* p : {q, k, v, eta, alpha, W0, static_cast<const void*>(y),
                          static_cast<const void*>(ws)})
      if (misaligned(p)) return fail(GL_ERROR_MISALIGNED, "pointer %p not 16-byte aligned", p);
    gls::FwdArgs f;
    f.x = k; f.g = v; f.q = q; f.eta = eta; f.alpha = alpha; f.W0 = W0; f.y = y;
    f.states = ws;
    f.B = desc->B; f.H = desc->H; f.T = desc->T;
    f.d_in = 128; f.d_out = 128;
    f.chunk = gls::kMfmaChunk;
    f.n_chunks = static_cast<int>((desc->T + gls::kMfmaChunk - 1) / gls::kMfmaChunk);
    f.ckpt_every = 1; f.n_ckpt = f.n_chunks;
    f.seg_chunks = f.n_chunks; f.n_seg = 1;
    f.w0_t = w0_transposed != 0;
    if (desc->B * desc->H * static_cast<int64_t>(f.n_chunks) > 0x7fffffffLL)
      return fail(GL_ERROR_NOT_SUPPORTED, "B*H*chunks above 2^31-1");
    return hip_status(gls::launch_mfma_qkv_two_pass(f, static_cast<hipStream_t>(stream)),
                      "qkv scan launch");
  }
  if (desc->io_dtype == GL_DTYPE_BF16 && desc->d_in == 64 && desc->d_out == 64 &&
      !(desc->flags & GL_FLAG_GENERIC)) {
    // the forward matrix-core kernel with a read tile of its own: x is the
    // write key, g the value (one segment; every pointer 16-byte aligned)
    for (const void* p : {q, k, v, eta, alpha, W0, static_cast<const void*>(y)})
      if (misaligned(p)) return fail(GL_ERROR_MISALIGNED, "pointer %p not 16-byte aligned", p);
    gls::FwdArgs f;
    f.x = k; f.g = v; f.q = q; f.eta = eta; f.alpha = alpha; f.W0 = W0; f.y = y;
    f.states = nullptr;
    f.B = desc->B; f.H = desc->H; f.T = desc->T;
    f.d_in = 64; f.d_out = 64;
    f.chunk = gls::kMfmaChunk;
    f.n_chunks = static_cast<int>((desc->T + gls::kMfmaChunk - 1) / gls::kMfmaChunk);
    f.ckpt_every = 1; f.n_ckpt = f.n_chunks;
    f.seg_chunks = f.n_chunks; f.n_seg = 1;
    f.w0_t = w0_transposed != 0;
    return hip_status(gls::launch_mfma_qkv_fwd(f, static_cast<hipStream_t>(stream)),
                      "qkv scan launch");
  }
  gls::QkvArgs a;
  a.q = q; a.k = k; a.v = v; a.eta = eta; a.alpha = alpha; a.W0 = W0; a.y = y;
  a.B = desc->B; a.H = desc->H; a.T = desc->T;
  a.dk = static_cast<int>(desc->d_in); a.dv = static_cast<int>(desc->d_out);
  a.w0_transposed = w0_transposed != 0;
  return hip_status(gls::launch_qkv_fwd(desc->io_dtype, a, static_cast<hipStream_t>(stream)),
                    "qkv scan launch");
}

// The reverse scan with a read vector and write key of their own: the forward
// chunk states recomputed by the generic forward (states only) into the
// workspace, the generic reverse scan, then the fixed-order sums.  Layout of
// the workspace: states [B*H][n_chunks][dv][dk], deta / dalpha tile partials
// [n_tiles][B*H*T] each, dW0 partials [B*H][dv][dk] (compute type).
namespace {
struct QkvPlan {
  int chunk = 0, n_chunks = 0, n_tiles = 0;
  size_t comp = 8, states = 0, part = 0, dw = 0, total = 0;
  // bf16, dk = dv = 64 on the matrix cores: bf16 chunk-start states; per
  // group of chunks the fp32 adjoint leaving it (lam), its decay (gam) and
  // a dW0' share (dw); part is unused
  bool mfma = false;
  int n_grp = 0, grp_chunks = 0;
  size_t lam = 0, gam = 0, w0t = 0;  // w0t: W0' transposed (d = 128, bf16)
};
gl_status_t qkv_plan(const gl_scan_desc_t* d, QkvPlan* p) {
  gl_status_t st = check_dec(d, true);
  if (st != GL_SUCCESS) return st;
  const size_t dd = static_cast<size_t>(d->d_in) * static_cast<size_t>(d->d_out);
  const size_t BH = static_cast<size_t>(d->B) * static_cast<size_t>(d->H);
  p->comp = d->io_dtype == GL_DTYPE_F64 ? 8 : 4;
  if (!(d->flags & GL_FLAG_GENERIC) &&
      gls::mfma_qkv_bwd_ok(d->io_dtype, static_cast<int>(d->d_in), static_cast<int>(d->d_out))) {
    p->mfma = true;
    p->chunk = gls::kMfmaChunk;
    p->n_chunks = static_cast<int>((d->T + p->chunk - 1) / p->chunk);
    if (static_cast<int64_t>(BH) * p->n_chunks > 0x7fffffffLL)
      return fail(GL_ERROR_NOT_SUPPORTED, "B*H*chunks above 2^31-1");
    const size_t cells = BH * static_cast<size_t>(p->n_chunks);
    p->grp_chunks = gls::mfma_qkv_bwd_group_chunks(static_cast<int64_t>(BH), p->n_chunks,
                                                   static_cast<int>(d->d_in));
    p->n_grp = gls::mfma_qkv_bwd_groups(p->n_chunks, p->grp_chunks);
    p->states = round_up(cells * dd * 2);
    const size_t groups = BH * static_cast<size_t>(p->n_grp);
    p->lam = round_up(groups * dd * sizeof(float));
    p->gam = round_up(groups * sizeof(float));
    p->dw = round_up(BH * static_cast<size_t>(p->n_grp) * dd * sizeof(float));
    p->w0t = d->d_in == 128 ? round_up(static_cast<size_t>(d->H) * dd * 2) : 0;
    p->total = p->states + p->lam + p->gam + p->dw + p->w0t;
    return GL_SUCCESS;
  }
  p->chunk = d->io_dtype == GL_DTYPE_F64 ? 8 : 32;  // LDS of the generic kernels with a read tile
  p->n_chunks = static_cast<int>((d->T + p->chunk - 1) / p->chunk);
  p->n_tiles = static_cast<int>((std::max(d->d_in, d->d_out) + gls::kGenericTile - 1) /
                                gls::kGenericTile);
  p->states = round_up(BH * p->n_chunks * dd * p->comp);
  p->part = round_up(static_cast<size_t>(p->n_tiles) * BH * d->T * p->comp);
  p->dw = round_up(BH * dd * p->comp);
  p->total = p->states + 2 * p->part + p->dw;
  return GL_SUCCESS;
}
}  // namespace

gl_status_t gl_scan_qkv_workspace_size(const gl_scan_desc_t* desc, size_t* ws_bytes) {
  QkvPlan p;
  gl_status_t st = qkv_plan(desc, &p);
  if (st != GL_SUCCESS) return st;
  if (!ws_bytes) return fail(GL_ERROR_INVALID_VALUE, "ws_bytes is NULL");
  *ws_bytes = p.total;
  return GL_SUCCESS;
}

gl_status_t gl_scan_qkv_bwd(const gl_scan_desc_t* desc, const void* q, const void* k,
                            const void* v, const void* eta, const void* alpha, const void* W0,
                            int w0_transposed, const void* dy, void* dq, void* dk, void* dv,
                            void* deta, void* dalpha, void* dW0, void* ws, size_t ws_bytes,
                            void* stream) {
  QkvPlan p;
  gl_status_t st = qkv_plan(desc, &p);
  if (st != GL_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t dd = static_cast<size_t>(desc->d_in) * static_cast<size_t>(desc->d_out);
  if (desc->B * desc->H * desc->T == 0) {
    if (desc->H == 0) return GL_SUCCESS;
    st = check_ptrs({dW0});
    if (st != GL_SUCCESS) return st;
    return hip_status(gls::launch_clear(dW0, desc->H * dd * p.comp, s), "dW0 clear");
  }
  st = check_ptrs({q, k, v, eta, alpha, W0, dy, dq, dk, dv, deta, dalpha, dW0, ws});
  if (st != GL_SUCCESS) return st;
  if (ws_bytes < p.total)
    return fail(GL_ERROR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", ws_bytes, p.total);
  char* w = static_cast<char*>(ws);
  void* states = w;
  if (p.mfma) {
    gls::BwdArgs b;
    b.x = k; b.q = q; b.g = v; b.eta = eta; b.alpha = alpha; b.W0 = W0; b.dy = dy;
    b.states = states;
    b.dx = dk; b.dq = dq; b.dg = dv;
    b.mf_lam = w + p.states;
    b.mf_gam = w + p.states + p.lam;
    b.part_dW0 = w + p.states + p.lam + p.gam;
    b.W0t = p.w0t ? w + p.states + p.lam + p.gam + p.dw : nullptr;
    b.grp_chunks = p.grp_chunks;
    b.deta_out = deta; b.dalpha_out = dalpha;
    b.B = desc->B; b.H = desc->H; b.T = desc->T;
    b.d_in = static_cast<int>(desc->d_in); b.d_out = b.d_in;
    b.chunk = p.chunk; b.n_chunks = p.n_chunks; b.ckpt_every = 1; b.n_ckpt = p.n_chunks;
    b.n_tiles = 1;
    b.seg_chunks = p.n_chunks; b.n_seg = 1;
    b.w0_t = w0_transposed != 0;
    st = hip_status(gls::launch_mfma_qkv_bwd(b, s), "qkv backward launch");
    if (st != GL_SUCCESS) return st;
    gls::FinArgs fa;
    fa.part_eta = nullptr; fa.part_alpha = nullptr; fa.part_dW0 = b.part_dW0;
    fa.deta = deta; fa.dalpha = dalpha; fa.dW0 = dW0;
    fa.B = desc->B; fa.H = desc->H; fa.T = desc->T;
    fa.d_in = b.d_in; fa.d_out = b.d_in; fa.n_tiles = 1; fa.n_seg = p.n_grp;
    fa.alpha_done = true;
    fa.eta_done = true;
    return hip_status(gls::launch_finalize(desc->io_dtype, fa, s), "qkv finalize launch");
  }
  void* part_eta = w + p.states;
  void* part_alpha = w + p.states + p.part;
  void* part_dW0 = w + p.states + 2 * p.part;

  gls::FwdArgs f;
  f.x = k; f.q = q; f.g = v; f.eta = eta; f.alpha = alpha; f.W0 = W0;
  f.y = nullptr; f.states = states;
  f.B = desc->B; f.H = desc->H; f.T = desc->T;
  f.d_in = static_cast<int>(desc->d_in); f.d_out = static_cast<int>(desc->d_out);
  f.chunk = p.chunk; f.n_chunks = p.n_chunks; f.ckpt_every = 1; f.n_ckpt = p.n_chunks;
  f.seg_chunks = p.n_chunks; f.n_seg = 1;
  f.w0_t = w0_transposed != 0;
  st = hip_status(gls::launch_generic_fwd(desc->io_dtype, f, s), "qkv state recompute");
  if (st != GL_SUCCESS) return st;

  gls::BwdArgs b;
  b.x = k; b.q = q; b.g = v; b.eta = eta; b.alpha = alpha; b.W0 = W0; b.dy = dy;
  b.states = states;
  b.dx = dk; b.dq = dq; b.dg = dv;
  b.part_eta = part_eta; b.part_alpha = part_alpha; b.part_dW0 = part_dW0;
  b.B = desc->B; b.H = desc->H; b.T = desc->T;
  b.d_in = f.d_in; b.d_out = f.d_out;
  b.chunk = p.chunk; b.n_chunks = p.n_chunks; b.ckpt_every = 1; b.n_ckpt = p.n_chunks;
  b.n_tiles = p.n_tiles;
  b.seg_chunks = p.n_chunks; b.n_seg = 1;
  b.w0_t = w0_transposed != 0;
  st = hip_status(gls::launch_generic_bwd(desc->io_dtype, b, s), "qkv backward launch");
  if (st != GL_SUCCESS) return st;

  gls::FinArgs fa;
  fa.part_eta = part_eta; fa.part_alpha = part_alpha; fa.part_dW0 = part_dW0;
  fa.deta = deta; fa.dalpha = dalpha; fa.dW0 = dW0;
  fa.B = desc->B; fa.H = desc->H; fa.T = desc->T;
  fa.d_in = f.d_in; fa.d_out = f.d_out; fa.n_tiles = p.n_tiles; fa.n_seg = 1;
  return hip_status(gls::launch_finalize(desc->io_dtype, fa, s), "qkv finalize launch");
}

const char* gl_status_string(gl_status_t status) {
  switch (status) {
    case GL_SUCCESS: return "success";
    case GL_ERROR_INVALID_VALUE: return "invalid value";
    case GL_ERROR_NOT_SUPPORTED: return "not supported";
    case GL_ERROR_MISALIGNED: return "pointer not 16-byte aligned";
    case GL_ERROR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case GL_ERROR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* gl_last_error(void) { return g_err; }

const char* gl_scan_path_name(const gl_scan_desc_t* desc) {
  Plan p;
  if (make_plan(desc, &p) != GL_SUCCESS) return nullptr;
  return p.name;
}

}  // extern "C"
