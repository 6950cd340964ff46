// k_mfma_bwd_c.hip -- chunk-parallel part of the matrix-core reverse scan
// (bf16 io, d_in = d_out = 64; gfx950, v_mfma_f32_16x16x32_bf16).
//
// The adjoint Lam = dL/dD is the only quantity the reverse scan carries from
// chunk to chunk (the exact adjoint of the forward scan, GradLev abstract,
// omanscience.com).  Once a first pass has stored Lam_out -- Lam entering
// every chunk from its right end, bf16 [B*H][n_chunks][D][D], next to the
// forward's chunk states D_in -- every chunk's outputs depend on that chunk
// alone, so this pass runs chunks in parallel: one work-group per
// (sequence-head, run of chunks), all D rows and columns of a chunk.  With
// chunk-local l (inclusive cumsum of log2 alpha), lq_i = l_{i-1}, e(.) = 2^(.):
//   P_ui  = e(lq_u - l_i)(x_u . x_i)                          (u > i)
//   Be_ij = e(lq_i - l_j)(-eta_j)(dy_i . g_j)                 (j < i)
//   u_i   = e(l_last - l_i) Lam_out x_i + sum_{u>i} P_ui dy_u
//   dg_i  = -eta_i u_i,   deta_i = -g_i . u_i
//   dx_i  = W0^T dy_i + e(lq_i) D_in^T dy_i + (Be X)_i + (Be^T X)_i
//           - eta_i e(l_last - l_i) Lam_out^T g_i
//   dW0  += sum_u dy_u x_u^T
// and the four per-token dots of the dalpha identity
//   pp_i = x_i.(Lam_out^T g_i), rr_i = x_i.(D_in^T dy_i),
//   qq_i = x_i.(Be X)_i,        kk_i = x_i.(Be^T X)_i
// plus <Lam_out, D_in>, from which dalpha_chunks (below) forms dalpha.
//
// Pipeline: 16 waves (four per SIMD, to hide the latency of each wave's
// dependent MFMA / exp / LDS steps); two chunk slots filled by direct buffer
// loads (x, g, dy, D_in, Lam_out tiles; the gate rows of the chunk after),
// two barriers per chunk.  Phase 1: the 10 + 10 causal 16 x 16 blocks of P
// and Be (MFMA, decay and mask), the <Lam_out, D_in> partials.  Phase 2:
// wave w owns the 16 x 16 block (token block w/4, row block w%4) of u / dg,
// the block (token block w/4, column block w%4) of dx with its dots, and the
// block (column block w/4, row block w%4) of dW0; one wave derives the gates
// of the next chunk.
#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kD = 64;          // d_in = d_out
constexpr int kC = 64;          // tokens per chunk
constexpr int kNW = 16;         // waves per work-group
constexpr int kNT = 64 * kNW;   // threads
constexpr int kGateWave = 0;    // derives the gates of the next chunk
constexpr int kPerGroupTarget = 256;  // work-groups to aim for
constexpr int kDotsPerChunk = 4 * 4 * kC;  // [column block][kind][token]

struct alignas(16) SlotC {
  __bf16 X[kC * kD];    // x, swizzled [token][D]
  __bf16 G[kC * kD];    // g, swizzled [token][D]
  __bf16 DY[kC * kD];   // dy, swizzled [token][D]
  __bf16 S[kD * kD];    // D_in, swizzled [row][col]
  __bf16 L[kD * kD];    // Lam_out, swizzled [row][col]
  float q[2][kC];       // eta, alpha of the next chunk
  __bf16 pad[512];      // target of the loads of waves with nothing to load
};

struct alignas(16) GatesC {
  float lq[kC], li[kC], nb[kC], eq[kC], e2[kC];
  float gam[4];
};

// Per-lane byte offset of instruction wi (of 8) of a [64][64] tile load.
__device__ __forceinline__ uint32_t dma_off_c(int wi, int lane) {
  const int p = wi * 64 + lane;
  const int row = p >> 3, kl = (p & 7) ^ swz<kD>(row);
  return static_cast<uint32_t>(row * kD * 2 + 16 * kl);
}

// Tiles of chunk k and the gate rows of chunk kq (negative: zero fill).
// Waves 0-7 load instruction w of the x, g and dy tiles, waves 8-15
// instruction w - 8 of the D_in and Lam_out tiles (and a zero-size load into
// the pad): the same three instructions in every wave, with scalar-selected
// sources and destinations.
__device__ __forceinline__ void issue_chunk_c(SlotC& sl, uint32_t ot, uint32_t oq,
                                              const uint16_t* x, const uint16_t* g,
                                              const uint16_t* dy, const uint16_t* st,
                                              const uint16_t* lo, const float* eta,
                                              const float* alpha, int64_t T, int k, int kq,
                                              int wave) {
  const bool in = k >= 0;
  const int64_t t0 = in ? static_cast<int64_t>(k) * kC : 0;
  const int cv = in ? static_cast<int>(std::min<int64_t>(kC, T - t0)) : 0;
  const int64_t s0 = (in ? static_cast<int64_t>(k) : 0) * kD * kD;
  const int sb = in ? kD * kD * 2 : 0;
  const bool io = wave < 8;
  const int wi = wave & 7;
  char* base = reinterpret_cast<char*>(&sl);
  const int o1 = io ? static_cast<int>(offsetof(SlotC, X)) : static_cast<int>(offsetof(SlotC, S));
  const int o2 = io ? static_cast<int>(offsetof(SlotC, G)) : static_cast<int>(offsetof(SlotC, L));
  const int o3 = io ? static_cast<int>(offsetof(SlotC, DY)) + wi * 1024
                    : static_cast<int>(offsetof(SlotC, pad));
  dma16(io ? buffer_rsrc(x + t0 * kD, cv * kD * 2) : buffer_rsrc(st + s0, sb), ot,
        base + o1 + wi * 1024);
  dma16(io ? buffer_rsrc(g + t0 * kD, cv * kD * 2) : buffer_rsrc(lo + s0, sb), ot,
        base + o2 + wi * 1024);
  dma16(io ? buffer_rsrc(dy + t0 * kD, cv * kD * 2) : buffer_rsrc(x, 0), ot, base + o3);
  const bool inq = kq >= 0;
  const int64_t tq = inq ? static_cast<int64_t>(kq) * kC : 0;
  const int cq = inq ? static_cast<int>(std::min<int64_t>(kC, T - tq)) : 0;
  dma4(buffer_rsrc(((wave & 1) == 0 ? eta : alpha) + tq, cq * 4), oq, sl.q[wave & 1]);
}
__device__ __forceinline__ void gates_c(const float (*q)[kC], GatesC& gs, int cv, int lane) {
  const float et = lane < cv ? q[0][lane] : 0.f;
  const ChunkGates gt = chunk_gates(lane < cv ? q[1][lane] : 1.f, lane);
  gs.lq[lane] = gt.lq;
  gs.li[lane] = gt.l;
  gs.nb[lane] = -et;
  gs.eq[lane] = fexp2(gt.lq);
  gs.e2[lane] = fexp2(gt.llast - gt.l);
  if (lane == 0) gs.gam[0] = fexp2(gt.llast);
}

// One causal 16 x 16 block b (0..9) of P^T or Be^T.  Both are
//   OUT[col][row] = (T1_row . T2_col) e(lq_row - l_col) f_col   (col < row)
// with, for P^T (rows u, cols i): T1 = T2 = x, f = 1 (PT[i][u] = P_ui); for
// Be^T (rows i, cols j): T1 = dy, T2 = g, f = -eta (BeT[j][i] = Be_ij).
// Blocks above the diagonal are never written (they stay zero).
__device__ __forceinline__ void causal_block(const __bf16* T1, const __bf16* T2, __bf16* OUT,
                                             bool with_eta, const GatesC& gs,
                                             const LaneOff<kD>& oX, const LaneOff<kC>& oA, int b,
                                             int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const int rb = tri_i(b), cb = tri_j(b);
  f32x4 d = zero4();
#pragma unroll
  for (int kb = 0; kb < kD / 32; ++kb)
    d = mfma16x16x32(frag_s<kD>(T1, oX, rb * 16, kb * 32), frag_s<kD>(T2, oX, cb * 16, kb * 32), d);
  const int col = cb * 16 + l16, r0 = rb * 16 + 4 * g4;
  const float lc = gs.li[col], fc = with_eta ? gs.nb[col] : 1.f;
  const f32x4 lqr = *reinterpret_cast<const f32x4*>(&gs.lq[r0]);
  f32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float e = d[q] * fexp2(lqr[q] - lc) * fc;
    v[q] = (col < r0 + q) ? e : 0.f;
  }
  uint2 pk;
  pk.x = pack2(v[0], v[1]);
  pk.y = pack2(v[2], v[3]);
  put4<kC>(OUT, oA, cb * 16, rb * 16, pk);
}

__device__ __forceinline__ f32x4 unpack4c(const uint2& p) {
  f32x4 v;
  v[0] = bf16_val(p.x & 0xffffu);
  v[1] = bf16_val(p.x >> 16);
  v[2] = bf16_val(p.y & 0xffffu);
  v[3] = bf16_val(p.y >> 16);
  return v;
}

__device__ __forceinline__ float dot4(const f32x4& a, const f32x4& b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// Chunks per work-group: enough work-groups to fill the GPU, at least one
// chunk each.
__host__ __device__ inline int chunks_per_group(int64_t BH, int n_chunks) {
  const int64_t per_bh = std::max<int64_t>(1, (kPerGroupTarget + BH - 1) / std::max<int64_t>(BH, 1));
  const int64_t g = std::min<int64_t>(per_bh, n_chunks);
  return static_cast<int>((n_chunks + g - 1) / g);
}

__global__ __launch_bounds__(kNT) void bwd_c64(BwdArgs a) {
  __shared__ SlotC ring0, ring1;
  __shared__ __bf16 PT_s[kC * kC];   // P^T, swizzled; W0 staging at the start
  __shared__ __bf16 BeT_s[kC * kC];  // Be^T, swizzled
  __shared__ GatesC gs0, gs1;
  SlotC* const rs[2] = {&ring0, &ring1};
  GatesC* const gsb[2] = {&gs0, &gs1};

  const int64_t BH = a.B * a.H, T = a.T, BHT = BH * T;
  const int n = a.n_chunks;
  const int per = chunks_per_group(BH, n);
  const int ngrp = (n + per - 1) / per;
  const int64_t bh = blockIdx.x / ngrp;
  const int grp = static_cast<int>(blockIdx.x % ngrp);
  if (bh >= BH) return;
  const int c_beg = grp * per;
  const int c_end = std::min(n, c_beg + per);
  const int nloc = c_end - c_beg;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int ib = wave >> 2, jb = wave & 3;  // token (dW0: column) block; row / column block
  const int h = static_cast<int>(bh % a.H);
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * kD;
  const uint16_t* g = static_cast<const uint16_t*>(a.g) + bh * T * kD;
  const uint16_t* dy = static_cast<const uint16_t*>(a.dy) + bh * T * kD;
  const float* eta = static_cast<const float*>(a.eta) + bh * T;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * kD * kD;
  const uint16_t* st = static_cast<const uint16_t*>(a.states) + bh * static_cast<int64_t>(n) * kD * kD;
  const uint16_t* lo = static_cast<const uint16_t*>(a.lam_out) + bh * static_cast<int64_t>(n) * kD * kD;
  uint16_t* dx = static_cast<uint16_t*>(a.dx) + bh * T * kD;
  uint16_t* dg = static_cast<uint16_t*>(a.dg) + bh * T * kD;
  float* pe = static_cast<float*>(a.part_eta) + jb * BHT + bh * T;
  float* pdots = a.part_dots + bh * static_cast<int64_t>(n) * kDotsPerChunk;
  float* pc0 = a.part_c0 + bh * static_cast<int64_t>(n) * kNW;

  const LaneOff<kD> oX = lane_off<kD>(lane);
  const LaneOff<kC> oA = lane_off<kC>(lane);

  // W0^T fragments of this wave's column block (staged through PT_s), then
  // the never-written triangles of PT_s / BeT_s cleared
  for (int idx = tid; idx < kD * kD / 8; idx += kNT) {
    const int r = idx >> 3, cc = 8 * (idx & 7);
    *reinterpret_cast<uint4*>(&PT_s[sidx<kD>(r, cc)]) =
        *reinterpret_cast<const uint4*>(W0 + static_cast<int64_t>(r) * kD + cc);
  }
  __syncthreads();
  bf16x8 w0f[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) w0f[kb] = frag_ts<kD>(PT_s, oX, kb * 32, jb * 16);
  __syncthreads();
  for (int idx = tid; idx < kC * kC / 8; idx += kNT) {
    reinterpret_cast<uint4*>(PT_s)[idx] = make_uint4(0, 0, 0, 0);
    reinterpret_cast<uint4*>(BeT_s)[idx] = make_uint4(0, 0, 0, 0);
  }

  const auto cv_of = [&](int c) {
    return (c < c_beg || c >= c_end)
               ? 0
               : static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };
  const auto in_grp = [&](int c) { return c < c_end ? c : -1; };
  const uint32_t ot = dma_off_c(wave & 7, lane);
  const uint32_t oq = static_cast<uint32_t>(lane * 4);
  const __amdgpu_buffer_rsrc_t r_none = buffer_rsrc(a.x, 0);
  // c0 partials: this thread's 4 elements of D_in and Lam_out (same layout)
  const uint32_t oc0 = static_cast<uint32_t>(sidx<kD>(tid >> 4, 4 * (tid & 15)) * 2);
  // dots: lane (g4, l16) stores kind kind_of(g4) of token ib*16 + l16
  const int kind = g4 == 0 ? 0 : g4 == 1 ? 2 : g4 == 2 ? 1 : 3;
  const uint32_t odots = static_cast<uint32_t>(((jb * 4 + kind) * kC + ib * 16 + l16) * 4);
  const uint32_t oeta = g4 == 0 ? static_cast<uint32_t>((ib * 16 + l16) * 4) : 0xfffffff0u;
  const uint32_t odx = static_cast<uint32_t>(((ib * 16 + l16) * kD + jb * 16 + 4 * g4) * 2);
  constexpr int S = 5;  // stores per wave per chunk: c0, dg, deta, dx, dots

  f32x4 dw = zero4();

  // first chunk (and the gate rows of the second) into slot 0, its own gate
  // rows into slot 1; S dropped stores (stream shape as in the loop)
  issue_chunk_c(*rs[0], ot, oq, x, g, dy, st, lo, eta, alpha, T, c_beg, in_grp(c_beg + 1), wave);
  dma4(buffer_rsrc(((wave & 1) == 0 ? eta : alpha) + static_cast<int64_t>(c_beg) * kC,
                   cv_of(c_beg) * 4),
       oq, rs[1]->q[wave & 1]);
#pragma unroll
  for (int k = 0; k < S; ++k) store4(r_none, oq + 64 * k, 0.f);  // spaced: not merged
  wait_vm<S>();
  lds_barrier();
  if (wave == kGateWave) gates_c(rs[1]->q, *gsb[0], cv_of(c_beg), lane);

  const auto step = [&](auto KC, int v) {
    constexpr int K = decltype(KC)::value;
    SlotC& cur = *rs[K];
    SlotC& dst = *rs[K ^ 1];
    const GatesC& gc = *gsb[K];  // v & 1 == K
    const int c = c_beg + v;
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = cv_of(c);
    wait_vm<S>();   // chunk c loaded: after it only the previous chunk's stores
    lds_barrier();  // and the previous chunk's reads of the other slot are done
    issue_chunk_c(dst, ot, oq, x, g, dy, st, lo, eta, alpha, T, in_grp(c + 1), in_grp(c + 2), wave);

    // ---- phase 1: P and Be blocks (blocks 0-9 of P, 10-19 of Be: wave w
    // takes w and w + 16), <Lam_out, D_in> partial
    const auto blk = [&](int b) {
      const bool be = b >= 10;
      causal_block(be ? cur.DY : cur.X, be ? cur.G : cur.X, be ? BeT_s : PT_s, be, gc, oX, oA,
                   be ? b - 10 : b, lane);
    };
    blk(wave);
    if (wave < 4) blk(wave + 16);
    {
      const uint2 sv = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(cur.S) + oc0);
      const uint2 lv = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(cur.L) + oc0);
      float p = dot4(unpack4c(sv), unpack4c(lv));
      p = wave_sum(p);
      store4(buffer_rsrc(pc0 + static_cast<int64_t>(c) * kNW + wave, 4), oq, p);
    }
    lds_barrier();  // P^T, Be^T visible

    // ---- phase 2
    const int i = ib * 16 + l16;
    const float e2i = gc.e2[i], nbi = gc.nb[i], eqi = gc.eq[i];
    {
      // u^T[r][i] for row block jb; dg; deta partial over its 16 rows
      f32x4 ain = zero4(), apd = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        ain = mfma16x16x32(frag_s<kD>(cur.L, oX, jb * 16, kb * 32),
                           frag_s<kD>(cur.X, oX, ib * 16, kb * 32), ain);
        apd = mfma16x16x32(frag_ts<kD>(cur.DY, oX, kb * 32, jb * 16),
                           frag_s<kC>(PT_s, oA, ib * 16, kb * 32), apd);
      }
      const f32x4 u = ain * e2i + apd;
      uint2 pk;
      pk.x = pack2(u[0] * nbi, u[1] * nbi);
      pk.y = pack2(u[2] * nbi, u[3] * nbi);
      store8(buffer_rsrc(dg + t0 * kD, cv * kD * 2), odx, pk);
      float p = dot4(unpack4c(get4<kD>(cur.G, oX, ib * 16, jb * 16)), u);
      p = sum_rows(p);
      store4(buffer_rsrc(pe + t0, cv * 4), oeta, -p);
    }
    {
      // dx^T[k][i] for column block jb, and the four dots over its columns
      f32x4 aws = zero4(), as_ = zero4(), al = zero4(), aq = zero4(), ak = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 df = frag_s<kD>(cur.DY, oX, ib * 16, kb * 32);
        aws = mfma16x16x32(w0f[kb], df, aws);
        as_ = mfma16x16x32(frag_ts<kD>(cur.S, oX, kb * 32, jb * 16), df, as_);
        al = mfma16x16x32(frag_ts<kD>(cur.L, oX, kb * 32, jb * 16),
                          frag_s<kD>(cur.G, oX, ib * 16, kb * 32), al);
        const bf16x8 xf = frag_ts<kD>(cur.X, oX, kb * 32, jb * 16);
        aq = mfma16x16x32(xf, frag_ts<kC>(BeT_s, oA, kb * 32, ib * 16), aq);
        ak = mfma16x16x32(xf, frag_s<kC>(BeT_s, oA, ib * 16, kb * 32), ak);
      }
      const f32x4 v = aws + as_ * eqi + aq + ak + al * (nbi * e2i);
      uint2 pk;
      pk.x = pack2(v[0], v[1]);
      pk.y = pack2(v[2], v[3]);
      store8(buffer_rsrc(dx + t0 * kD, cv * kD * 2), odx, pk);
      const f32x4 xv = unpack4c(get4<kD>(cur.X, oX, ib * 16, jb * 16));
      float pp = dot4(xv, al), rr = dot4(xv, as_), qq = dot4(xv, aq), kk = dot4(xv, ak);
      // four sums over the 16-lane rows at once: afterwards row g4 of the
      // wave holds pp (0), qq (1), rr (2), kk (3) of token i
      permlane32_swap(pp, rr);
      permlane32_swap(qq, kk);
      float s1 = pp + rr, s2 = qq + kk;
      permlane16_swap(s1, s2);
      store4(buffer_rsrc(pdots + static_cast<int64_t>(c) * kDotsPerChunk, kDotsPerChunk * 4), odots,
             s1 + s2);
    }
    // dW0^T[k][r] for column block ib, row block jb
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      dw = mfma16x16x32(frag_ts<kD>(cur.X, oX, kb * 32, ib * 16),
                        frag_ts<kD>(cur.DY, oX, kb * 32, jb * 16), dw);
    // gates of the next chunk (its gate rows came with this chunk's tiles)
    if (wave == kGateWave) gates_c(cur.q, *gsb[K ^ 1], cv_of(c + 1), lane);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  for (int v = 0; v < nloc; v += 2) {
    step(I0{}, v);
    if (v + 1 >= nloc) break;
    step(I1{}, v + 1);
  }
  wait_vm<0>();  // no load into LDS may outlive the work-group
  float* pw = static_cast<float*>(a.part_dW0) + (grp * BH + bh) * kD * kD;
  *reinterpret_cast<f32x4*>(pw + (jb * 16 + l16) * kD + ib * 16 + 4 * g4) = dw;
}

// dalpha of one chunk per wave from the dots and <Lam_out, D_in> partials:
//   dalpha_i = e(l_last - l_i + lq_i) c0 + e(l_last - l_i) sum_{j<i} e(lq_i - l_j)(-eta_j) pp_j
//              + e(lq_i) sum_{u>i} e(lq_u - l_i) rr_u
//              + (sum_{u>i} qq_u - sum_{j>=i} kk_j) / alpha_i
// (the sums are affine-pair and plain scans over the lanes; the suffix sums
// run on the reversed lane order).
constexpr int kDaThreads = 256;
__global__ __launch_bounds__(kDaThreads) void dalpha_chunks(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * (kDaThreads / 64) + (threadIdx.x >> 6);
  const int64_t BH = a.B * a.H, T = a.T;
  const int n = a.n_chunks;
  if (item >= BH * n) return;
  const int64_t bh = item / n;
  const int c = static_cast<int>(item % n);
  const int64_t t0 = static_cast<int64_t>(c) * kC;
  const int cv = static_cast<int>(std::min<int64_t>(kC, T - t0));
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T + t0;
  const float* eta = static_cast<const float*>(a.eta) + bh * T + t0;
  const float* pd = a.part_dots + item * kDotsPerChunk;
  const float* pc = a.part_c0 + item * kNW;
  const int ir = kC - 1 - lane;
  const float al = lane < cv ? alpha[lane] : 1.f;
  const float al_r = ir < cv ? alpha[ir] : 1.f;
  const float nb = lane < cv ? -eta[lane] : 0.f;
  const auto dsum = [&](int kind, int t) {
    return (pd[kind * kC + t] + pd[(4 + kind) * kC + t]) +
           (pd[(8 + kind) * kC + t] + pd[(12 + kind) * kC + t]);
  };
  const float pp = dsum(0, lane), kk = dsum(3, lane);
  const float rr_r = dsum(1, ir), z_r = dsum(2, ir) - dsum(3, ir);
  float c0 = 0.f;
#pragma unroll
  for (int w = 0; w < kNW; ++w) c0 += pc[w];
  const ChunkGates gt = chunk_gates(al, lane);
  float a2 = al, b2 = nb * pp;
  wave_scan_affine(a2, b2);
  const float s2 = wave_shift_up(b2, 0.f);
  const float lq_r = wave_reverse(gt.lq, lane);
  float a3 = al_r, b3 = rr_r;
  wave_scan_affine(a3, b3);
  const float s3_r = wave_shift_up(b3, 0.f);
  const float zs_r = wave_shift_up(wave_scan_add(z_r), 0.f);
  const float t34 = wave_reverse(fexp2(lq_r) * s3_r + zs_r * __builtin_amdgcn_rcpf(al_r), lane);
  const float v = fexp2(gt.llast - gt.l + gt.lq) * c0 + fexp2(gt.llast - gt.l) * s2 + t34 -
                  kk * __builtin_amdgcn_rcpf(al);
  if (lane < cv) static_cast<float*>(a.dalpha_out)[bh * T + t0 + lane] = v;
}

}  // namespace

ChunkParLayout mfma_bwd_c64_layout() { return {4, kDotsPerChunk, kNW}; }

int mfma_bwd_c64_groups(int64_t BH, int n_chunks) {
  return (n_chunks + chunks_per_group(BH, n_chunks) - 1) / chunks_per_group(BH, n_chunks);
}

hipError_t launch_mfma_bwd_c64(const BwdArgs& a, hipStream_t s) {
  const int64_t BH = a.B * a.H;
  const int ngrp = mfma_bwd_c64_groups(BH, a.n_chunks);
  hipLaunchKernelGGL(bwd_c64, dim3(static_cast<unsigned>(BH * ngrp)), dim3(kNT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = BH * a.n_chunks;
  const int64_t per_block = kDaThreads / 64;
  hipLaunchKernelGGL(dalpha_chunks, dim3(static_cast<unsigned>((items + per_block - 1) / per_block)),
                     dim3(kDaThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace gls
