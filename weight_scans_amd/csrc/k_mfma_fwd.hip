// k_mfma_fwd.hip -- matrix-core forward scan for bf16 io, d_in = d_out = D
// in {64, 128} (gfx950, wave64, v_mfma_f32_16x16x32_bf16).
//
// One work-group = one sequence-head (b, h) x one tile of kTN = 32 rows of
// the adaptation D_t (rows are independent chains because y reduces over
// columns only).  The tile's fp32 state lives in MFMA accumulators for the
// whole sequence.  Per chunk of kC = 64 tokens (l = chunk-local inclusive
// cumsum of log2 alpha, lq_i = l_{i-1}, e(.) = 2^(.)):
//   A_ij  = (x_i . x_j) e(lq_i - l_j) (-eta_j)        j < i  (else 0)
//   y_i   = W0 x_i + e(lq_i) D_in x_i + sum_j A_ij g_j
//   D_out = e(l_last) D_in + sum_j e(l_last - l_j)(-eta_j) g_j x_j^T
// i.e. earlier rank-one updates damped by the later gates, composed as an
// affine scan across chunks ("Parallelize the Training, Keep the Learning
// Serial", cognaptus.com, section "Once the gradient signals are known, the
// weight trajectory becomes parallelizable").  Every exponent is <= 0.
//
// Pipeline (one work-group barrier per chunk): chunk tiles are copied
// HBM -> LDS by direct buffer loads into a ring of kRing slots; while chunk c
// is finished (y and the state update), the scores of chunk c + 1 are formed
// and the gates of chunk c + 2 derived, and the loads of chunks
// c + 3 and c + 4 are in flight.  Sixteen waves (four per SIMD) in two roles:
// y waves 0-3 own two 16 x 16 blocks of y (token blocks 2 (w/2) and
// 2 (w/2) + 1, row block w%2), y waves 4-7 one strip each of the next
// chunk's score blocks, and y wave 4 also derives the gates; state waves
// 8-15 own D/64 16 x 16 blocks of the fp32 state, issue every load (and wait
// for them), store the chunk-start states and scale the g tile.  (The state
// waves' step is the longest: the gates moved off them shortened it a
// little, the g scaling or score blocks moved onto them lengthened it.)  In
// the state-only instance the idle y waves 2 and 3 derive the gates, one
// half each.  Each role runs its own copy
// of the chunk loop, so registers are allocated per role.  All LDS tiles are
// XOR-swizzled (mfma.hpp) so that fragment reads are free of bank conflicts.
//
// `states` (optional) receives D_in of every chunk in bf16:
// [B*H][n_chunks][D (row r)][D (col c)] -- read by the matrix-core backward.
//
// Segments: work-group (segment s, head, tile) scans only the chunks of s,
// starting from the state given in seg_in (zero if absent).  The state-only
// instance (no y, no states) instead reports the segment's final state from
// a zero start and its summed log2 alpha (with one segment, the hand-over
// state D_T for decoding); an exclusive affine scan over the
// segments (k_seg.hip) turns these into each segment's starting state.  This
// is the associative composition of the scan across chunks
// ("Parallelize the Training, Keep the Learning Serial", cognaptus.com,
// section "Once the gradient signals are known, the weight trajectory becomes
// parallelizable") applied one level up.
#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kC = 64;         // tokens per chunk
constexpr int kTN = 32;        // rows of the adaptation per work-group
constexpr int kNW = 16;        // waves per work-group: 8 y waves, 8 state (loader) waves
constexpr int kNT = 64 * kNW;  // threads
constexpr int kRing = 5;       // chunk slots: 3 in use, 2 in flight
// the gates: with y, y wave kPrepWaveY alone (the one with the lightest
// score strip: the state waves carry the loads and the state update, the
// longest chain of a step); without y (the state-only instance, where the y
// waves are otherwise idle), y waves kPrepWave and kPrepWave + 1, one half
// each
constexpr int kPrepWave = 2;
constexpr int kPrepWaveY = 4;

// Per-token factors of a chunk derived from the gates (i = token, b = 16-token
// block of i, m_b = l_{16 b - 1} with m_0 = 0):
//   eq_i = e(lq_i),  R_i = e(lq_i - m_b),  C_{b', i} = e(m_b' - l_i)(-eta_i)  (b' = 1..3)
// so that for i in block b' > block of j:  e(lq_i - l_j)(-eta_j) = R_i C_{b', j},
// with both factors <= 1 in magnitude (l is non-increasing).
struct GateRows {
  float eta[kC], R[kC], C1[kC], C2[kC];  // eta: as loaded; the rest derived
  float alpha[kC], C3[kC], eq[kC], pad[kC];
};

template <int D, bool QK = false>
struct alignas(16) Slot {
  __bf16 X[kC * D];                      // x (the write key) of the chunk, swizzled [token][D]
  __bf16 G[kC * kTN];                    // g of the row tile, swizzled [token][kTN]
  union {
    float q[2][4 * kC];                  // loaded: eta = q[0][0..63], alpha = q[1][0..63]
    GateRows f;                          // after the gate pass (same bytes)
  };
  float lq[kC], li[kC], nb[kC], bk[kC];  // l_{i-1}, l_i, -eta_i, e(l_last - l_i)(-eta_i)
  float gam[4];                          // gam[0] = e(l_last)
  __bf16 Q[QK ? kC * D : 8];             // a read vector of its own, swizzled [token][D]
};

// Per-lane byte offsets of the chunk loads (loop invariant).  Wave w loads
// x units of instructions w + 8 s, and a quarter of the g tile (w < 4) or a
// gate row (w = 4, 6: eta; 5, 7: alpha -- two waves write the same bytes).
template <int D>
struct DmaOff {
  uint32_t x[D / 64];
  uint32_t gq;
};
template <int D>
__device__ __forceinline__ DmaOff<D> dma_off(int wave, int lane) {
  constexpr int U = D / 8;  // 16-byte units per row of x
  DmaOff<D> o;
#pragma unroll
  for (int s = 0; s < D / 64; ++s) {
    const int p = (wave + 8 * s) * 64 + lane;
    const int row = p / U, kl = (p % U) ^ swz<D>(row);
    o.x[s] = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  }
  if (wave < 4) {
    const int p = wave * 64 + lane;
    const int row = p >> 2, kl = (p & 3) ^ swz<kTN>(row);
    o.gq = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  } else {
    o.gq = static_cast<uint32_t>(lane * 4);
  }
  return o;
}

// Vector-memory instructions one wave issues per chunk load.
template <int D, bool QK = false>
constexpr int kLoadOps = (QK ? 2 : 1) * (D / 64) + 1;

// Queue the loads of chunk k into `sl`.  Rows past the sequence end, and
// chunks from c_end on, are zero-filled by the buffer bounds (every wave
// always issues the same number of loads).
template <int D, bool QK>
__device__ __forceinline__ void issue_chunk(Slot<D, QK>& sl, const DmaOff<D>& o, const uint16_t* x,
                                            const uint16_t* q, const uint16_t* g, const float* eta,
                                            const float* alpha, int64_t T, int k, int c_end,
                                            int r0, int wave) {
  const bool in = k < c_end;
  const int64_t t0 = in ? static_cast<int64_t>(k) * kC : 0;
  const int cv = in ? static_cast<int>(std::min<int64_t>(kC, T - t0)) : 0;
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + t0 * D, cv * D * 2);
#pragma unroll
  for (int s = 0; s < D / 64; ++s) dma16(rx, o.x[s], sl.X + (wave + 8 * s) * 512);
  if constexpr (QK) {
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q + t0 * D, cv * D * 2);
#pragma unroll
    for (int s = 0; s < D / 64; ++s) dma16(rq, o.x[s], sl.Q + (wave + 8 * s) * 512);
  }
  // the same instruction in every wave (no branch): scalar-selected source
  // and destination offset within the slot
  const bool gw = wave < 4;
  const __amdgpu_buffer_rsrc_t r4 =
      gw ? buffer_rsrc(g + t0 * D + r0, cv > 0 ? (cv * D - r0) * 2 : 0)
         : buffer_rsrc(((wave & 1) == 0 ? eta : alpha) + t0, cv * 4);
  const int lds_off = gw ? static_cast<int>(offsetof(Slot<D>, G)) + wave * 1024
                         : static_cast<int>(offsetof(Slot<D>, q)) + (wave & 1) * 1024;
  using SlotQ = Slot<D, true>;
  static_assert(offsetof(Slot<D>, G) == offsetof(SlotQ, G) &&
                    offsetof(Slot<D>, q) == offsetof(SlotQ, q),
                "the read tile follows the common part of a slot");
  // a gate row is 64 floats: one 4-byte load per lane
  if (gw)
    dma16(r4, o.gq, reinterpret_cast<char*>(&sl) + lds_off);
  else
    dma4(r4, o.gq, reinterpret_cast<char*>(&sl) + lds_off);
}

// Gates of a chunk, lane = token: PART 0 the per-token decays and Gamma
// (returns l_last), PART 1 the rank-one factors of the off-diagonal score
// blocks, PART 2 both (one wave).  Two waves can each take one part, each
// deriving the log2 cumsum itself.
template <int D, int PART, bool QK>
__device__ __forceinline__ float prep_gates(Slot<D, QK>& sl, int cv, int lane) {
  const ChunkGates gt = chunk_gates(lane < cv ? sl.f.alpha[lane] : 1.f, lane);
  if constexpr (PART == 2) {
    const float et = lane < cv ? sl.f.eta[lane] : 0.f;
    const float m1 = readlane_f(gt.l, 15), m2 = readlane_f(gt.l, 31), m3 = readlane_f(gt.l, 47);
    const int b = lane >> 4;
    const float mb = b == 0 ? 0.f : b == 1 ? m1 : b == 2 ? m2 : m3;
    sl.lq[lane] = gt.lq;
    sl.li[lane] = gt.l;
    sl.nb[lane] = -et;
    sl.bk[lane] = -et * fexp2(gt.llast - gt.l);
    sl.f.eq[lane] = fexp2(gt.lq);
    sl.f.R[lane] = fexp2(gt.lq - mb);
    sl.f.C1[lane] = -et * fexp2(fminf(m1 - gt.l, 0.f));
    sl.f.C2[lane] = -et * fexp2(fminf(m2 - gt.l, 0.f));
    sl.f.C3[lane] = -et * fexp2(fminf(m3 - gt.l, 0.f));
    if (lane == 0) sl.gam[0] = fexp2(gt.llast);
    return gt.llast;
  } else if constexpr (PART == 0) {
    const float et = lane < cv ? sl.f.eta[lane] : 0.f;
    sl.lq[lane] = gt.lq;
    sl.li[lane] = gt.l;
    sl.nb[lane] = -et;
    sl.bk[lane] = -et * fexp2(gt.llast - gt.l);
    sl.f.eq[lane] = fexp2(gt.lq);
    if (lane == 0) sl.gam[0] = fexp2(gt.llast);
    return gt.llast;
  } else {
    const float et = lane < cv ? sl.f.eta[lane] : 0.f;
    const float m1 = readlane_f(gt.l, 15), m2 = readlane_f(gt.l, 31), m3 = readlane_f(gt.l, 47);
    const int b = lane >> 4;
    const float mb = b == 0 ? 0.f : b == 1 ? m1 : b == 2 ? m2 : m3;
    sl.f.R[lane] = fexp2(gt.lq - mb);
    sl.f.C1[lane] = -et * fexp2(fminf(m1 - gt.l, 0.f));
    sl.f.C2[lane] = -et * fexp2(fminf(m2 - gt.l, 0.f));
    sl.f.C3[lane] = -et * fexp2(fminf(m3 - gt.l, 0.f));
    return 0.f;
  }
}

// Decayed score block (ib, jb), jb <= ib, of a chunk from its raw products
// xx = (x_i . x_j) (q_i . k_j with a read tile), written transposed:
// AT[j][i] = A_ij.  Blocks above the diagonal are never written (they stay
// zero).
template <int D, bool QK>
__device__ __forceinline__ void score_out(const Slot<D, QK>& sl, __bf16* AT, const LaneOff<kC>& oA,
                                          int ib, int jb, const f32x4& xx, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const int j = jb * 16 + l16, i0 = ib * 16 + 4 * g4;
  f32x4 v;
  if (ib == jb) {  // diagonal block: decay per element, causal mask
    const float lj = sl.li[j], nj = sl.nb[j];
    const f32x4 lqi = *reinterpret_cast<const f32x4*>(&sl.lq[i0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float e = xx[q] * fexp2(lqi[q] - lj) * nj;
      v[q] = (j < i0 + q) ? e : 0.f;
    }
  } else {  // every j < i: rank-one decay
    const float cj = (ib == 1 ? sl.f.C1 : ib == 2 ? sl.f.C2 : sl.f.C3)[j];
    const f32x4 ri = *reinterpret_cast<const f32x4*>(&sl.f.R[i0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = xx[q] * (ri[q] * cj);
  }
  uint2 pk;
  pk.x = pack2(v[0], v[1]);
  pk.y = pack2(v[2], v[3]);
  put4<kC>(AT, oA, jb * 16, ib * 16, pk);
}

// Strip s (0..3) of the causal triangle of 16 x 16 score blocks: the row
// block's fragments are read once and serve every block of the strip.
//   s = 0: row block 3, column blocks 0-1;  s = 1: row block 3, blocks 2-3;
//   s = 2: row block 2, blocks 0-2;  s = 3: row block 1, blocks 0-1, and
//   row block 0, block 0.
template <int D, bool QK>
__device__ __forceinline__ void score_strip(const Slot<D, QK>& sl, __bf16* AT, const LaneOff<D>& oX,
                                            const LaneOff<kC>& oA, int s, int lane) {
  const auto strip = [&](int ib, int jb0, int nj) {
    bf16x8 af[D / 32];
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) af[kb] = frag_s<D>(QK ? sl.Q : sl.X, oX, ib * 16, kb * 32);
    for (int jb = jb0; jb < jb0 + nj; ++jb) {
      __builtin_amdgcn_sched_barrier(0);  // one block's fragments live at a time
      f32x4 xx = zero4();
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) xx = mfma16x16x32(af[kb], frag_s<D>(sl.X, oX, jb * 16, kb * 32), xx);
      score_out<D>(sl, AT, oA, ib, jb, xx, lane);
    }
  };
  if (s == 0) {
    strip(3, 0, 2);
  } else if (s == 1) {
    strip(3, 2, 2);
  } else if (s == 2) {
    strip(2, 0, 3);
  } else {
    strip(1, 0, 2);
    strip(0, 0, 1);
  }
}

// One thread's share of the decay-scaled g tile of a chunk:
// GS[j][r] = bf16(g_j[r] e(l_last - l_j)(-eta_j)) for 4 consecutive r.
template <int D, bool QK>
__device__ __forceinline__ void scale_g(const Slot<D, QK>& sl, __bf16* GS, uint32_t off, int row) {
  const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(sl.G) + off);
  const float s = sl.bk[row];
  uint2 r;
  r.x = pack2(bf16_val(v.x & 0xffffu) * s, bf16_val(v.x >> 16) * s);
  r.y = pack2(bf16_val(v.y & 0xffffu) * s, bf16_val(v.y >> 16) * s);
  *reinterpret_cast<uint2*>(reinterpret_cast<char*>(GS) + off) = r;
}

// The same with the remainder of each product, v - bf16(v) (exact in fp32),
// rounded to bf16 into GL: the pair carries the product to about 2^-17.
template <int D, bool QK>
__device__ __forceinline__ void scale_g_split(const Slot<D, QK>& sl, __bf16* GS, __bf16* GL,
                                              uint32_t off, int row) {
  const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(sl.G) + off);
  const float s = sl.bk[row];
  const float p0 = bf16_val(v.x & 0xffffu) * s, p1 = bf16_val(v.x >> 16) * s;
  const float p2 = bf16_val(v.y & 0xffffu) * s, p3 = bf16_val(v.y >> 16) * s;
  uint2 h, l;
  h.x = pack2(p0, p1);
  h.y = pack2(p2, p3);
  l.x = pack2(p0 - bf16_val(h.x & 0xffffu), p1 - bf16_val(h.x >> 16));
  l.y = pack2(p2 - bf16_val(h.y & 0xffffu), p3 - bf16_val(h.y >> 16));
  *reinterpret_cast<uint2*>(reinterpret_cast<char*>(GS) + off) = h;
  *reinterpret_cast<uint2*>(reinterpret_cast<char*>(GL) + off) = l;
}

// The remainder tiles of the split decay-scaled g, by chunk parity; empty
// where the split is not used.
template <bool ON>
struct RemTiles {
  __bf16 t[2][kC * kTN];
};
template <>
struct RemTiles<false> {};

template <int D, bool HAS_Y, bool HAS_ST, bool F32 = false, bool QK = false, bool SPLIT = false>
__global__ __launch_bounds__(kNT) void fwd_mfma(FwdArgs a) {
  static_assert(D == 64 || D == 128, "D");
  static_assert(!QK || (D == 64 && HAS_Y && !HAS_ST), "a read tile of its own: d = 64, y only");
  using SL = Slot<D, QK>;
  constexpr int NTILE = D / kTN;
  constexpr int NS = D / 64;  // 16x16 state blocks per state wave
  constexpr int P = kLoadOps<D, QK>;
  constexpr int S = HAS_ST ? 1 : 0;  // stores per state wave per chunk
  // Each ring slot is a separate LDS object, and every reference to one is
  // static (the chunk loop is unrolled by kRing), so the compiler can tell a
  // slot being read from the slots still being filled and adds no waits.
  __shared__ SL ring0, ring1, ring2, ring3, ring4;
  __shared__ __bf16 AT_s[2][kC * kC];  // AT[j][i] = A_ij, swizzled, by chunk parity
  __shared__ __bf16 S_s[2][kTN * D];   // D_in of the tile, bf16, swizzled [row][col], by parity
  __shared__ __bf16 GS_s[2][kC * kTN]; // decay-scaled g tile, swizzled, by chunk parity
  // The hand-over instance carries the decay-scaled g as a bf16 pair (value
  // and remainder): its state is a result of its own, not only an operand of
  // the next readout.
  constexpr bool HILO = SPLIT;
  static_assert(!SPLIT || (!HAS_Y && !HAS_ST), "the split is for the state-only instance");
  __shared__ RemTiles<HILO> GL;  // (empty in the other instances)
  static_assert(kRing == 5, "ring objects");
  SL* const rs[kRing] = {&ring0, &ring1, &ring2, &ring3, &ring4};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int role = wave >> 3, w8 = wave & 7;  // 0: y waves, 1: state (and loader) waves
  const int g4 = lane >> 4, l16 = lane & 15;
  const int tb = w8 >> 1, rbw = w8 & 1;  // y block / state row block of this wave
  // 8 consecutive sequence-heads and all their row tiles share one XCD
  // (work-groups are dealt to the 8 XCDs round-robin), so the x chunk that
  // every tile reads is fetched from HBM once into that XCD's L2.
  // (segment is the slowest index, so the XCD of a head does not change)
  const int per_seg = static_cast<int>((a.B * a.H + 7) / 8) * 8 * NTILE;
  const int seg = blockIdx.x / per_seg, bid = blockIdx.x % per_seg;
  const int grp = bid / (8 * NTILE), within = bid % (8 * NTILE);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  const int tile = within >> 3;
  if (bh >= a.B * a.H) return;
  const int r0 = tile * kTN;
  const int h = static_cast<int>(bh % a.H);
  const int64_t T = a.T;
  const int n = a.n_chunks;
  const int c_beg = seg * a.seg_chunks;
  const int c_end = std::min(n, c_beg + a.seg_chunks);
  const int nloc = c_end - c_beg;
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * D;
  const uint16_t* qv = QK ? static_cast<const uint16_t*>(a.q) + bh * T * D : nullptr;
  const uint16_t* g = static_cast<const uint16_t*>(a.g) + bh * T * D;
  const float* eta = static_cast<const float*>(a.eta) + bh * T;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * D * D;
  constexpr int YE = F32 ? 4 : 2;  // bytes per element of y
  char* y = HAS_Y ? static_cast<char*>(a.y) + bh * T * D * YE : nullptr;
  // states: one per a.st_every chunks (the chunk-start state of chunks c with
  // c % st_every == 0), ceil(n / st_every) per sequence-head
  const int st_every = a.st_every;
  const int n_st = (n + st_every - 1) / st_every;
  uint16_t* st = HAS_ST ? static_cast<uint16_t*>(a.states) + bh * static_cast<int64_t>(n_st) * D * D
                        : nullptr;

  // y waves: W0 rows of this wave's row block as MFMA A fragments, in
  // registers throughout
  bf16x8 wf[D / 32];
  if (HAS_Y && role == 0) {
    const int wr = r0 + rbw * 16 + l16;
    if (QK && a.w0_t) {  // W0' given transposed, [D (k)][D (r)]: gathered once
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          wf[kb][e] = __builtin_bit_cast(__bf16, W0[static_cast<int64_t>(kb * 32 + 8 * g4 + e) * D + wr]);
    } else {
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
        wf[kb] = *reinterpret_cast<const bf16x8*>(W0 + static_cast<int64_t>(wr) * D + kb * 32 + 8 * g4);
    }
  }
  // state waves: starting state of the tile, zero or the segment's incoming
  // state (fp32 accumulators, and its bf16 copy for the first readout)
  f32x4 sacc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) sacc[s] = zero4();
  if (role == 1 && a.seg_in) {
    const float* si = a.seg_in + (bh * a.n_seg + seg) * D * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int cb = tb + 4 * s;
      sacc[s] = *reinterpret_cast<const f32x4*>(si + (r0 + rbw * 16 + l16) * D + cb * 16 + 4 * g4);
    }
  }
  if (HAS_Y)
    for (int idx = tid; idx < 2 * kC * kC / 8; idx += kNT)
      reinterpret_cast<uint4*>(&AT_s[0][0])[idx] = make_uint4(0, 0, 0, 0);
  wait_vm<0>();

  // valid tokens of chunk c (none outside this segment)
  const auto cv_of = [&](int c) {
    return c < c_end ? static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC))
                     : 0;
  };
  const LaneOff<D> oX = lane_off<D>(lane);
  const LaneOff<kTN> oG = lane_off<kTN>(lane);
  const LaneOff<kC> oA = lane_off<kC>(lane);
  const DmaOff<D> od = dma_off<D>(w8, lane);
  // per-lane byte offsets of the stores (loop invariant; the buffer base
  // moves per chunk and its byte count drops rows past the sequence end)
  // (y waves 0-3: the first of their two token blocks, 2 (w8 / 2))
  const uint32_t oy =
      static_cast<uint32_t>(((2 * (w8 >> 1) * 16 + l16) * D + r0 + rbw * 16 + 4 * g4) * 2);
  const __amdgpu_buffer_rsrc_t r_none = buffer_rsrc(a.x, 0);
  // a state-wave thread's 4 elements of the scaled g tile: row t/8, columns 4 (t%8)..
  const int gt_id = tid & 511;
  const int gs_row = gt_id >> 3;
  const uint32_t gs_off = static_cast<uint32_t>(sidx<kTN>(gs_row, 4 * (gt_id & 7)) * 2);
  // chunk-start state: state-wave thread t stores D / 16 consecutive elements
  // (row t / 16, columns (D / 16)(t % 16) ..) of the tile's bf16 copy in LDS,
  // so every store instruction writes whole rows
  constexpr int kStEl = D / 16;
  const int st_row = gt_id >> 4, st_col = kStEl * (gt_id & 15);
  const uint32_t st_l = static_cast<uint32_t>(sidx<D>(st_row, st_col) * 2);
  const uint32_t st_g = static_cast<uint32_t>(((r0 + st_row) * D + st_col) * 2);
  if (role == 1) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      uint2 pk;
      pk.x = pack2(sacc[s][0], sacc[s][1]);
      pk.y = pack2(sacc[s][2], sacc[s][3]);
      put4<D>(S_s[0], oX, rbw * 16, (tb + 4 * s) * 16, pk);
    }
    // Initial loads, each followed by S state stores into a zero-byte buffer
    // (they are dropped) so that the vector-memory instruction stream has
    // the same shape as in the loop: chunk load, S stores, chunk load, ...
    // Then the wait at the top of every iteration is the same constant.
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k) {
      issue_chunk<D>(*rs[k], od, x, qv, g, eta, alpha, T, c_beg + k, c_end, r0, w8);
#pragma unroll
      for (int s = 0; s < S; ++s) store8(r_none, 64 * k, make_uint2(0, 0));  // not merged
    }
    // chunks 0 and 1 done: after chunk 1 come two more chunk loads and three store groups
    wait_vm<2 * P + 3 * S>();
  }
  lds_barrier();
  float lsum = 0.f;  // sum of l_last over the segment's chunks (prep wave)
  if (HAS_Y && role == 0 && w8 == kPrepWaveY) {
    lsum += prep_gates<D, 2>(*rs[0], cv_of(c_beg), lane);
    lsum += prep_gates<D, 2>(*rs[1], cv_of(c_beg + 1), lane);
  }
  if (!HAS_Y && role == 0 && w8 == kPrepWave) {
    lsum += prep_gates<D, 0>(*rs[0], cv_of(c_beg), lane);
    lsum += prep_gates<D, 0>(*rs[1], cv_of(c_beg + 1), lane);
  }
  if (!HAS_Y && role == 0 && w8 == kPrepWave + 1) {
    prep_gates<D, 1>(*rs[0], cv_of(c_beg), lane);
    prep_gates<D, 1>(*rs[1], cv_of(c_beg + 1), lane);
  }
  lds_barrier();
  if (role == 1) {
    if constexpr (HILO)
      scale_g_split<D>(*rs[0], GS_s[0], GL.t[0], gs_off, gs_row);
    else
      scale_g<D>(*rs[0], GS_s[0], gs_off, gs_row);
  }
  if (HAS_Y && role == 0 && w8 >= 4) score_strip<D>(*rs[0], AT_s[0], oX, oA, w8 - 4, lane);

  // one chunk; K = (c - c_beg) % kRing is a compile-time constant
  const auto step = [&](auto RC, auto KC, int c) {
    constexpr int R = decltype(RC)::value;
    constexpr int K = decltype(KC)::value;
    SL& cur = *rs[K];
    SL& nx1 = *rs[(K + 1) % kRing];
    SL& nx2 = *rs[(K + 2) % kRing];
    SL& dst = *rs[(K + kRing - 1) % kRing];
    const int vl = c - c_beg;  // position in the segment: double-buffer parity
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = cv_of(c);
    // state (loader) waves: chunk c + 2 loaded -- issued after it are its own
    // store group and one more (chunk load + stores); past the end it is a
    // zero fill
    if constexpr (R == 1) wait_vm<P + 2 * S>();
    lds_barrier();  // scores and gates of c + 1, D_in of c visible
    if constexpr (R == 1) {
      issue_chunk<D>(dst, od, x, qv, g, eta, alpha, T, c + kRing - 1, c_end, r0, w8);
      if (HAS_ST) {
        // chunk-start state (natural layout, bf16): the copy in LDS that the
        // y waves read in this step, whole rows per store instruction
        // every chunk issues its store (the waits count a fixed number of
        // memory operations per step); a chunk whose state is not kept
        // stores into an empty buffer, which drops it
        const bool keep = c % st_every == 0;
        const __amdgpu_buffer_rsrc_t r_st =
            buffer_rsrc(st + static_cast<int64_t>(keep ? c / st_every : 0) * D * D,
                        keep ? D * D * 2 : 0);
        const char* sp = reinterpret_cast<const char*>(S_s[vl & 1]) + st_l;
        if constexpr (D == 128)
          store16(r_st, st_g, *reinterpret_cast<const uint4*>(sp));
        else
          store8(r_st, st_g, *reinterpret_cast<const uint2*>(sp));
      }
      if constexpr (HILO)
        scale_g_split<D>(nx1, GS_s[(vl + 1) & 1], GL.t[(vl + 1) & 1], gs_off, gs_row);
      else
        scale_g<D>(nx1, GS_s[(vl + 1) & 1], gs_off, gs_row);
      // state update, transposed: D^T[c][r] = Gamma D^T + sum_j x_j[c] (bk_j g_j[r]),
      // into the other state buffer (the current one may still be read)
      const __bf16* GS = GS_s[vl & 1];
      bf16x8 gs[2], gl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        gs[kb] = frag_ts<kTN>(GS, oG, kb * 32, rbw * 16);
        if constexpr (HILO) gl[kb] = frag_ts<kTN>(GL.t[vl & 1], oG, kb * 32, rbw * 16);
      }
      const float gam = cur.gam[0];
      __bf16* S_out = S_s[(vl + 1) & 1];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int cb = tb + 4 * s;
        sacc[s] = sacc[s] * gam;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 xf = frag_ts<D>(cur.X, oX, kb * 32, cb * 16);
          sacc[s] = mfma16x16x32(xf, gs[kb], sacc[s]);
          if constexpr (HILO) sacc[s] = mfma16x16x32(xf, gl[kb], sacc[s]);
        }
        uint2 pk;
        pk.x = pack2(sacc[s][0], sacc[s][1]);
        pk.y = pack2(sacc[s][2], sacc[s][3]);
        put4<D>(S_out, oX, rbw * 16, cb * 16, pk);
      }
    } else {
      if (HAS_Y && w8 >= 4) score_strip<D>(nx1, AT_s[(vl + 1) & 1], oX, oA, w8 - 4, lane);
      // gates of chunk c + 2 (loaded: the state waves waited for it before
      // the barrier)
      if (HAS_Y && w8 == kPrepWaveY) lsum += prep_gates<D, 2>(nx2, cv_of(c + 2), lane);
      // gates of chunk c + 2 (loaded: the state waves waited for it before
      // the barrier), two halves on two waves
      if (!HAS_Y) {
        if (w8 == kPrepWave) lsum += prep_gates<D, 0>(nx2, cv_of(c + 2), lane);
        if (w8 == kPrepWave + 1) prep_gates<D, 1>(nx2, cv_of(c + 2), lane);
        return;
      }
      // y waves 0-3: y^T[r][i] for row block rbw and the token blocks 2 p,
      // 2 p + 1 (p = w8 / 2), sharing the row block's fragments of G^T and
      // D_in; each lane stores 4 consecutive rows of one token straight from
      // the accumulators.  (For token blocks 0 and 1 the second K block of
      // A^T is zero.)  Waves 4-7 form the scores of the next chunk.
      if (w8 >= 4) return;
      const int pb = 2 * (w8 >> 1);
      const __bf16* S_in = S_s[vl & 1];
      const __bf16* AT = AT_s[vl & 1];
      f32x4 ya[2] = {zero4(), zero4()}, yb[2] = {zero4(), zero4()};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 gf = frag_ts<kTN>(cur.G, oG, kb * 32, rbw * 16);
#pragma unroll
        for (int t = 0; t < 2; ++t) ya[t] = mfma16x16x32(gf, frag_ts<kC>(AT, oA, kb * 32, (pb + t) * 16), ya[t]);
      }
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        __builtin_amdgcn_sched_barrier(0);  // one K step of fragments live at a time
        const bf16x8 sf = frag_s<D>(S_in, oX, rbw * 16, kb * 32);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 xf = frag_s<D>(QK ? cur.Q : cur.X, oX, (pb + t) * 16, kb * 32);
          ya[t] = mfma16x16x32(wf[kb], xf, ya[t]);
          yb[t] = mfma16x16x32(sf, xf, yb[t]);
        }
      }
      const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(y + t0 * D * YE, cv * D * YE);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float eqi = cur.f.eq[(pb + t) * 16 + l16];
        const uint32_t oyt = oy + static_cast<uint32_t>(t * 16 * D * 2);
        if constexpr (F32) {
          typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
          const f32x4 yo = ya[t] + eqi * yb[t];
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, yo), ry, 2 * oyt, 0, 0);
        } else {
          uint2 pk;
          pk.x = pack2(ya[t][0] + eqi * yb[t][0], ya[t][1] + eqi * yb[t][1]);
          pk.y = pack2(ya[t][2] + eqi * yb[t][2], ya[t][3] + eqi * yb[t][3]);
          store8(ry, oyt, pk);
        }
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  // each role walks in its own copy of the loop (same barriers), so that
  // registers are allocated per role; the loader role first (with this
  // order the compiler's wait analysis keeps the loaders' loads in flight
  // out of the other role's loop)
  const auto walk = [&](auto RC) {
    for (int v = 0; v < nloc; v += kRing) {
      step(RC, I0{}, c_beg + v);
      if (v + 1 >= nloc) break;
      step(RC, I1{}, c_beg + v + 1);
      if (v + 2 >= nloc) break;
      step(RC, I2{}, c_beg + v + 2);
      if (v + 3 >= nloc) break;
      step(RC, I3{}, c_beg + v + 3);
      if (v + 4 >= nloc) break;
      step(RC, I4{}, c_beg + v + 4);
    }
  };
  if (role == 1)
    walk(I1{});
  else
    walk(I0{});
  wait_vm<0>();  // no load into LDS may outlive the work-group
  if (a.seg_out && role == 1) {
    // the segment's final state (zero start) and its summed log2 alpha
    float* so = a.seg_out + (bh * a.n_seg + seg) * D * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int cb = tb + 4 * s;
      *reinterpret_cast<f32x4*>(so + (r0 + rbw * 16 + l16) * D + cb * 16 + 4 * g4) = sacc[s];
    }
  }
  if (a.seg_out && a.seg_lg && role == 0 && tile == 0 && w8 == (HAS_Y ? kPrepWaveY : kPrepWave) &&
      lane == 0)
    a.seg_lg[bh * a.n_seg + seg] = lsum;
}

template <int D, bool HAS_Y, bool HAS_ST, bool F32 = false, bool QK = false, bool SPLIT = false>
hipError_t launch_v(const FwdArgs& a, hipStream_t s, bool every_segment = false) {
  const int64_t groups = (a.B * a.H + 7) / 8;
  // the state-only pass of the segmented scan skips the last segment (nothing
  // lies to its right that would use its final state)
  const int nseg = (!HAS_Y && !HAS_ST && !every_segment) ? a.n_seg - 1 : a.n_seg;
  if (nseg <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (D / kTN) * nseg));
  hipLaunchKernelGGL((fwd_mfma<D, HAS_Y, HAS_ST, F32, QK, SPLIT>), grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  if (a.y && a.out_f32)
    return a.states ? launch_v<D, true, true, true>(a, s) : launch_v<D, true, false, true>(a, s);
  if (a.y && a.states) return launch_v<D, true, true>(a, s);
  if (a.y) return launch_v<D, true, false>(a, s);
  if (a.states) return launch_v<D, false, true>(a, s);
  if (a.seg_out) return launch_v<D, false, false>(a, s);  // state-only segment pass
  return hipSuccess;
}

}  // namespace

hipError_t launch_mfma_fwd(const FwdArgs& a, hipStream_t s) {
  return a.d_in == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

// The scan with a read vector of its own (a.q; a.x is the write key, a.g the
// value), d = 64, y only, one segment.
hipError_t launch_mfma_qkv_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.d_in != 64 || a.d_out != 64 || !a.q || !a.y || a.states || a.n_seg != 1)
    return hipErrorInvalidValue;
  return launch_v<64, true, false, false, true>(a, s);
}

// The final state of every segment from a zero start (with one segment: the
// adaptation after the last token, D_T) into a.seg_out [B*H][n_seg][D][D].
hipError_t launch_mfma_final_state(const FwdArgs& a, hipStream_t s) {
  return a.d_in == 128 ? launch_v<128, false, false, false, false, true>(a, s, true)
                       : launch_v<64, false, false, false, false, true>(a, s, true);
}

}  // namespace gls
