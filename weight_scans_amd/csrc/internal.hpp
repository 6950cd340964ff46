// internal.hpp -- argument blocks and launchers shared by the host API and the
// kernel translation units of libglscan.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace gls {

enum IoType { IO_F64 = 0, IO_F32 = 1, IO_BF16 = 2 };

// Forward scan.  One work-group owns one (b, h) and a tile of rows of the
// adaptation D (rows are independent chains: y reduces over columns only).
struct FwdArgs {
  const void* x;      // [B][H][T][d_in]   io
  const void* g;      // [B][H][T][d_out]  io
  const void* eta;    // [B][H][T]         gate
  const void* alpha;  // [B][H][T]         gate
  const void* W0;     // [H][d_out][d_in]  io
  void* y;            // [B][H][T][d_out]  io, may be null (states only)
  void* states;       // [B*H][n_ckpt][d_out][d_in] compute type, may be null
  int64_t B, H, T;
  int d_in, d_out;
  int chunk;          // tokens per chunk
  int n_chunks;       // ceil(T / chunk)
  int ckpt_every;     // a state is stored before every ckpt_every-th chunk
  int n_ckpt;         // ceil(n_chunks / ckpt_every)
  // Segments (matrix-core kernels): each sequence is cut into n_seg runs of
  // seg_chunks chunks (the last may be shorter), scanned by separate
  // work-groups.  seg_in: [B*H][n_seg][d_out][d_in] fp32 state entering each
  // segment (NULL = zero); seg_out / seg_lg: the segment's final state from a
  // zero start and its summed log2 alpha (state-only pass; NULL = not wanted).
  int seg_chunks = 0, n_seg = 1;
  const float* seg_in = nullptr;
  float* seg_out = nullptr;
  float* seg_lg = nullptr;
  // A read vector of its own (generic kernels): y_t = (W0' + D_t) q_t while the
  // update keeps x as the write key; NULL = read with x.  w0_t: W0' is stored
  // transposed ([H][d_in][d_out]).  out_f32: y is fp32 (bf16 io only).
  const void* q = nullptr;
  bool w0_t = false;
  bool out_f32 = false;
  // fp32 / fp64 matrix-core scans: [B*H][n_chunks] per-chunk decay (compute type)
  void* mf_gam = nullptr;
  // bf16 matrix-core kernels: `states` keeps the chunk-start state of every
  // st_every-th chunk only ([B*H][ceil(n_chunks / st_every)][d_out][d_in])
  int st_every = 1;
};

// Reverse scan.  Work-group (k, b*H+h) owns column tile k of D and Lambda
// (for dx) and row tile k of Lambda (for dg); per-token scalars and dW0 are
// emitted as partials and summed by the finalize kernel in a fixed order.
struct BwdArgs {
  const void* x;
  const void* g;
  const void* eta;
  const void* alpha;
  const void* W0;
  const void* dy;
  const void* states;  // chunk-boundary states written by the forward kernel
  void* dx;
  void* dg;
  void* part_eta;      // [n_tiles][B*H*T]  compute type
  void* part_alpha;    // [n_tiles][B*H*T]  compute type
  void* part_dW0;      // [B*H][d_out][d_in] compute type
  int64_t B, H, T;
  int d_in, d_out;
  int chunk, n_chunks, ckpt_every, n_ckpt;
  int n_tiles;
  // Segments, mirrored: seg_lam [B*H][n_seg][d_out][d_in] fp32 adjoint
  // entering each segment from its right end (NULL = zero); seg_out / seg_lg:
  // the adjoint at the segment's left end from a zero start, and the summed
  // log2 alpha (adjoint-only pass).  part_dW0 holds [n_seg][B*H][d_out][d_in].
  int seg_chunks = 0, n_seg = 1;
  const float* seg_lam = nullptr;
  // Fused backward: if seg_lg_in is set, seg_lam holds each segment's own
  // adjoint (from a zero start, as the adjoint-only pass leaves it) and
  // seg_lg_in its summed log2 alpha; the kernel composes the entering adjoint.
  const float* seg_lg_in = nullptr;
  float* seg_out = nullptr;
  float* seg_lg = nullptr;
  // The adjoint-only pass may cut the sequence finer than the fused pass:
  // lam_r of its segments (lam_seg_chunks chunks each) per fused segment,
  // lam_n of them in all; seg_lam / seg_lg_in / seg_out / seg_lg are then
  // indexed by those segments ([B*H][lam_n]).  seg_first: the first segment
  // the adjoint-only pass computes (the ones to its left are never needed).
  int lam_r = 1, lam_n = 0;
  int seg_first = 1;
  // Fused backward: deta and dalpha written directly ([B,H,T]).
  void* deta_out = nullptr;
  void* dalpha_out = nullptr;
  // A read vector of its own (generic kernels; see FwdArgs): x is then the
  // write key only, dx receives its gradient and dq that of q.
  const void* q = nullptr;
  void* dq = nullptr;
  bool w0_t = false;
  bool out_f32 = false;   // dx, dg (and dq) in fp32 (bf16 io only)
  // The write-key reverse scan on the matrix cores at d = 128: room for W0'
  // transposed ([H][dk][dv] bf16) when it is not given so
  const void* W0t = nullptr;
  int grp_chunks = 8;  // chunks per group of that scan's reverse pass
  // fp32 / fp64 matrix-core scans: the adjoint leaving every chunk
  // [B*H][n_chunks][d_out][d_in] and the per-chunk decay [B*H][n_chunks]
  // (compute type); part_dW0 then holds [n_chunks][B*H][d_out][d_in]
  void* mf_lam = nullptr;
  void* mf_gam = nullptr;
};

// Deployment (one token at a time): the cached adaptation `state`
// [B*H][d_out][d_in] in the compute type.
struct DecArgs {
  const void* x;      // readout / update: [B*H][d_in];  final state: [B*H][T][d_in]
  const void* g;      // update: [B*H][d_out];           final state: [B*H][T][d_out]
  const void* eta;    // update: [B*H];                  final state: [B*H][T]
  const void* alpha;  // (as eta)
  const void* W0;     // readout: [H][d_out][d_in]
  void* state;
  void* y;            // readout: [B*H][d_out]
  const void* x_prev = nullptr;  // step: the previous token's x [B*H][d_in]
  int64_t B, H, T;
  int d_in, d_out;
};

// Costate reconstruction under the quadratic token loss: rows = B*H*T token
// rows of d_out elements.
struct CostArgs {
  const void* y;       // [rows][d_out] io
  const void* target;  // [rows][d_out] io
  const void* g_hat;   // [rows][d_out] io
  void* g_tilde;       // [rows][d_out] io
  void* res_sq;        // [rows] compute type
  void* res_max;       // [rows] compute type
  int64_t rows;
  int d_out;
};

// The scan with its own read vector and write key (q != k): D is dv x dk.
struct QkvArgs {
  const void* q;      // [B*H][T][dk] io
  const void* k;      // [B*H][T][dk] io
  const void* v;      // [B*H][T][dv] io
  const void* eta;    // [B*H][T] gate type
  const void* alpha;  // [B*H][T] gate type
  const void* W0;     // [H][dv][dk] io, or [H][dk][dv] with w0_transposed
  void* y;            // [B*H][T][dv] io
  int64_t B, H, T;
  int dk, dv;
  bool w0_transposed;
};

struct FinArgs {
  const void* part_eta;
  const void* part_alpha;
  const void* part_dW0;
  void* deta;
  void* dalpha;
  void* dW0;
  int64_t B, H, T;
  int d_in, d_out;
  int n_tiles;
  int n_seg = 1;             // dW0 partials per (b, h)
  bool alpha_done = false;   // dalpha already written (fused backward)
  bool eta_done = false;     // deta already written (fused backward)
  int lanes = 1;             // lanes summing one dW0 element group (set by the launcher)
};

// Generic (VALU) kernels: any 1 <= d_in, d_out <= 128, all io types.
constexpr int kGenericMaxD = 128;
constexpr int kGenericTile = 16;  // rows per forward tile, cols/rows per bwd tile
bool generic_chunk_ok(int io, int chunk);
int generic_default_chunk(int io);
hipError_t launch_generic_fwd(int io, const FwdArgs& a, hipStream_t s);
hipError_t launch_generic_bwd(int io, const BwdArgs& a, hipStream_t s);
hipError_t launch_finalize(int io, const FinArgs& a, hipStream_t s);
// The no-allocation backward: the device address, on the current device, of
// a static scratch buffer of kStaticScratchBytes (taken once per device).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(void** ptr);
// Zero fill of `bytes` (a multiple of 4) at the 4-byte aligned device pointer p.
hipError_t launch_clear(void* p, size_t bytes, hipStream_t s);
hipError_t launch_decode_readout(int io, const DecArgs& a, hipStream_t s);
hipError_t launch_decode_update(int io, const DecArgs& a, hipStream_t s);
hipError_t launch_decode_step(int io, const DecArgs& a, hipStream_t s);
hipError_t launch_final_state(int io, const DecArgs& a, hipStream_t s);
hipError_t launch_costate(int io, const CostArgs& a, hipStream_t s);
hipError_t launch_qkv_fwd(int io, const QkvArgs& a, hipStream_t s);
hipError_t launch_mfma_final_state(const FwdArgs& a, hipStream_t s);

// Matrix-core kernels in fp32 / fp64 (io = compute type), chunk 64: any
// d_in, d_out <= 64 (fp32) or <= 32 (fp64).  The backward writes deta, dalpha
// directly (deta_out, dalpha_out) and one dW0 partial per sequence-head.
bool mf_shape_ok(int io, int d_in, int d_out);
hipError_t launch_mf_fwd(int io, const FwdArgs& a, hipStream_t s);
hipError_t launch_mf_bwd(int io, const BwdArgs& a, hipStream_t s);

// Matrix-core kernels: bf16 io, d_in == d_out in {64, 128}, chunk 64.
constexpr int kMfmaChunk = 64;
hipError_t launch_mfma_fwd(const FwdArgs& a, hipStream_t s);
hipError_t launch_mfma_qkv_fwd(const FwdArgs& a, hipStream_t s);  // read tile of its own, d = 64
// the write-key scan at d_k = d_v = 128 (bf16): states pass, then chunk outputs
bool mfma_qkv_two_pass(int io, int dk, int dv);
size_t mfma_qkv_states_bytes(int64_t BH, int64_t T);
hipError_t launch_mfma_qkv_two_pass(const FwdArgs& a, hipStream_t s);
// the reverse scan of the write-key scan at d_k = d_v in {64, 128} (bf16):
// states, group increments, carry over groups, chunk gradients (x = k,
// g = v; dx <- dk, dg <- dv; states / mf_lam / mf_gam / part_dW0 / W0t in
// the workspace)
bool mfma_qkv_bwd_ok(int io, int dk, int dv);
int mfma_qkv_bwd_groups(int n_chunks, int grp_chunks);  // groups (dW0' shares) per sequence-head
int mfma_qkv_bwd_group_chunks(int64_t BH, int n_chunks, int d);  // chunks per group
hipError_t launch_mfma_qkv_bwd(const BwdArgs& a, hipStream_t s);
hipError_t launch_mfma_bwd_lam(const BwdArgs& a, hipStream_t s);  // adjoint-only segment pass
hipError_t launch_mfma_bwd_f64(const BwdArgs& a, hipStream_t s);   // fused reverse scan, d = 64
hipError_t launch_mfma_bwd_f128(const BwdArgs& a, hipStream_t s);  // fused reverse scan, d = 128
// Exclusive affine scan over the segments of every (b, h): buf[s] <- the state
// entering segment s (in segment order, or from the right end if reverse).
hipError_t launch_seg_combine(float* buf, const float* lg, int64_t BH, int n_seg, int dd,
                              bool reverse, hipStream_t s);

}  // namespace gls
