// k_mfma_fwd.hip -- matrix-core forward scan for bf16 io, d_in = d_out = D
// in {64, 128} (gfx950, wave64, v_mfma_f32_16x16x32_bf16).
//
// One work-group = one sequence-head (b, h) x one tile of kTN = 32 rows of
// the adaptation D_t (rows are independent chains because y reduces over
// columns only).  The tile's fp32 state lives in MFMA accumulators for the
// whole sequence; chunks of kC = 64 tokens are streamed through LDS with a
// one-chunk register prefetch.  Per chunk (l = chunk-local inclusive cumsum
// of log2 alpha, lq_i = l_{i-1}, e(.) = 2^(.)):
//   A_ij  = (x_i . x_j) e(lq_i - l_j) (-eta_j)        j < i  (else 0)
//   y_i   = W0 x_i + e(lq_i) D_in x_i + sum_j A_ij g_j
//   D_out = e(l_last) D_in + sum_j e(l_last - l_j)(-eta_j) g_j x_j^T
// i.e. the discounted sum of rank-one updates of "Parallelize the Training,
// Keep the Learning Serial" (cognaptus.com, section "Once the gradient signals
// are known, the weight trajectory becomes parallelizable") composed as an
// affine scan across chunks.  Every exponent is <= 0.
//
// Layout choices: every LDS tile is token-major (as in HBM); products that
// contract over tokens read their operands with transposing LDS reads, and
// y and D are produced transposed (lane = 4 consecutive rows of one token /
// column), so every LDS and global write is 8 or 16 bytes wide.
//
// `states` (optional) receives D_in of every chunk in bf16:
// [B*H][n_chunks][D (row r)][D (col c)] -- read by the matrix-core backward.
#include <algorithm>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kC = 64;    // tokens per chunk
constexpr int kTN = 32;   // rows of the adaptation per work-group
constexpr int kNT = 256;  // threads (4 waves)

// Chunk inputs (double-buffered: chunk c + 1 is staged while chunk c is used).
template <int D>
struct alignas(16) FwdChunk {
  static constexpr int XP = D + 8;    // row stride of [token][D] tiles (elements)
  static constexpr int NP = kTN + 8;  // row stride of [token][kTN] tiles
  __bf16 X[kC][XP];                   // x of the chunk
  __bf16 G[kC][NP];                   // g of the row tile
  __bf16 Gs[kC][NP];                  // e(l_last - l_j)(-eta_j) g_j
  float lq[kC], li[kC], eq[kC], neta[kC];
  float gam;
};

template <int D>
struct alignas(16) FwdSmem {
  static constexpr int XP = D + 8;
  static constexpr int NP = kTN + 8;
  static constexpr int CP = kC + 8;   // row stride of [token][token] tiles
  FwdChunk<D> ch[2];
  __bf16 AT[kC][CP];                  // AT[j][i] = A_ij
  __bf16 S[2][kTN][XP];               // D_in of the tile, bf16 [row][col] (double-buffered)
  __bf16 W[kTN][XP];                  // W0 of the tile [row][col]
};

template <int D>
struct Prefetch {
  static constexpr int RPT = kC * D / (8 * kNT);  // x rows per thread (4 or 2)
  uint4 x[RPT];
  uint4 g;
  float eta, alpha;  // token tid % 64
};

template <int D>
__device__ __forceinline__ void load_chunk(Prefetch<D>& p, const uint16_t* x, const uint16_t* g,
                                           const float* eta, const float* alpha, int64_t t0,
                                           int cv, int r0, int tid) {
  constexpr int CG = D / 8;
  const int cg = tid % CG, rg = tid / CG;
#pragma unroll
  for (int s = 0; s < Prefetch<D>::RPT; ++s)
    p.x[s] = load_row16(x + t0 * D + 8 * cg, D, rg * Prefetch<D>::RPT + s, cv);
  p.g = load_row16(g + t0 * D + r0 + 8 * (tid & 3), D, tid >> 2, cv);
  const int jt = tid & (kC - 1), jc = jt < cv ? jt : cv - 1;
  p.eta = eta[t0 + jc];
  p.alpha = alpha[t0 + jc];
}

__device__ __forceinline__ uint4 scale_bf16x8(const uint4& v, float s) {
  uint4 r;
  r.x = pack2(bf16_val(v.x & 0xffffu) * s, bf16_val(v.x >> 16) * s);
  r.y = pack2(bf16_val(v.y & 0xffffu) * s, bf16_val(v.y >> 16) * s);
  r.z = pack2(bf16_val(v.z & 0xffffu) * s, bf16_val(v.z >> 16) * s);
  r.w = pack2(bf16_val(v.w & 0xffffu) * s, bf16_val(v.w >> 16) * s);
  return r;
}

template <int D>
__global__ __launch_bounds__(kNT) void fwd_mfma(FwdArgs a) {
  static_assert(D == 64 || D == 128, "D");
  constexpr int NTILE = D / kTN;
  constexpr int XP = FwdSmem<D>::XP, NP = FwdSmem<D>::NP, CP = FwdSmem<D>::CP;
  constexpr int RPT = Prefetch<D>::RPT, CG = D / 8;
  constexpr int NS = (2 * (D / 16)) / 4;  // state blocks per wave
  __shared__ FwdSmem<D> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int grp = blockIdx.x / (8 * NTILE), within = blockIdx.x % (8 * NTILE);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  const int tile = within >> 3;
  if (bh >= a.B * a.H) return;
  const int r0 = tile * kTN;
  const int h = static_cast<int>(bh % a.H);
  const int64_t T = a.T;
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * D;
  const uint16_t* g = static_cast<const uint16_t*>(a.g) + bh * T * D;
  const float* eta = static_cast<const float*>(a.eta) + bh * T;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * D * D;
  uint16_t* y = a.y ? static_cast<uint16_t*>(a.y) + bh * T * D : nullptr;
  uint16_t* st = a.states ? static_cast<uint16_t*>(a.states) + bh * a.n_chunks * D * D : nullptr;
  const int cg = tid % CG, rg = tid / CG, jg = tid >> 2, c8 = 8 * (tid & 3);

  for (int idx = tid; idx < kTN * (D / 8); idx += kNT) {
    const int r = idx / (D / 8), cc = 8 * (idx % (D / 8));
    *reinterpret_cast<uint4*>(&sm.W[r][cc]) =
        *reinterpret_cast<const uint4*>(W0 + static_cast<int64_t>(r0 + r) * D + cc);
    *reinterpret_cast<uint4*>(&sm.S[0][r][cc]) = make_uint4(0, 0, 0, 0);
  }
  for (int idx = tid; idx < kC * CP; idx += kNT) (&sm.AT[0][0])[idx] = static_cast<__bf16>(0.f);

  f32x4 sacc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) sacc[s] = zero4();

  const auto cv_of = [&](int c) {
    return static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };
  // Stage a loaded chunk (and its gates) into LDS buffer `buf`.
  const auto stage = [&](const Prefetch<D>& pf, FwdChunk<D>& buf, int cv) {
    const float et = lane < cv ? pf.eta : 0.f;
    const ChunkGates gt = chunk_gates(lane < cv ? pf.alpha : 1.f, lane);
    const float bk = -et * fexp2(gt.llast - gt.l);
    if (wave == 0) {
      buf.lq[lane] = gt.lq;
      buf.li[lane] = gt.l;
      buf.eq[lane] = fexp2(gt.lq);
      buf.neta[lane] = -et;
      if (lane == 0) buf.gam = fexp2(gt.llast);
    }
#pragma unroll
    for (int s = 0; s < RPT; ++s)
      *reinterpret_cast<uint4*>(&buf.X[rg * RPT + s][8 * cg]) = keep_row(pf.x[s], rg * RPT + s, cv);
    const uint4 gv = keep_row(pf.g, jg, cv);
    *reinterpret_cast<uint4*>(&buf.G[jg][c8]) = gv;
    *reinterpret_cast<uint4*>(&buf.Gs[jg][c8]) = scale_bf16x8(gv, __shfl(bk, jg, 64));
  };

  {
    Prefetch<D> pf;
    load_chunk<D>(pf, x, g, eta, alpha, 0, cv_of(0), r0, tid);
    stage(pf, sm.ch[0], cv_of(0));
  }
  lds_barrier();

  for (int c = 0; c < a.n_chunks; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = cv_of(c);
    FwdChunk<D>& cur = sm.ch[c & 1];
    // loads of the next chunk are issued now and consumed at the end of this
    // iteration, hidden behind this chunk's arithmetic
    const bool more = c + 1 < a.n_chunks;
    Prefetch<D> pf;
    if (more) load_chunk<D>(pf, x, g, eta, alpha, t0 + kC, cv_of(c + 1), r0, tid);

    if (y) {
      // causal decayed scores, written transposed: AT[j][i]
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        const int b = wave + 4 * s;
        if (b < 10) {
          const int ib = tri_i(b), jb = tri_j(b);
          f32x4 xx = zero4();
#pragma unroll
          for (int kb = 0; kb < D / 32; ++kb)
            xx = mfma16x16x32(frag(&cur.X[0][0], XP, ib * 16, kb * 32, lane),
                              frag(&cur.X[0][0], XP, jb * 16, kb * 32, lane), xx);
          const int j = jb * 16 + l16, i0 = ib * 16 + 4 * g4;
          const float lj = cur.li[j], nj = cur.neta[j];
          const f32x4 lqi = *reinterpret_cast<const f32x4*>(&cur.lq[i0]);
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float e = xx[q] * fexp2(lqi[q] - lj) * nj;
            v[q] = (j < i0 + q) ? e : 0.f;
          }
          uint2 pk;
          pk.x = pack2(v[0], v[1]);
          pk.y = pack2(v[2], v[3]);
          *reinterpret_cast<uint2*>(&sm.AT[j][i0]) = pk;
        }
      }
    }
    if (st) {
      // chunk-start state of this tile (rows r0.., natural layout, bf16)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int b = wave + 4 * s, cb = b >> 1, rb = b & 1;
        uint2 v;
        v.x = pack2(sacc[s][0], sacc[s][1]);
        v.y = pack2(sacc[s][2], sacc[s][3]);
        *reinterpret_cast<uint2*>(st + (static_cast<int64_t>(c) * D + r0 + rb * 16 + l16) * D +
                                  cb * 16 + 4 * g4) = v;
      }
    }
    lds_barrier();  // scores visible

    const __bf16* S_in = &sm.S[c & 1][0][0];
    if (y) {
      // y^T[r][i] for i in this wave's token block, both row blocks; each lane
      // stores 4 consecutive rows of one token straight from the accumulators
      const int w = wave;
      f32x4 ya[2] = {zero4(), zero4()}, yb[2] = {zero4(), zero4()};
      for (int kb = 0; kb < (w + 2) / 2; ++kb) {
        const bf16x8 af = frag_t(&sm.AT[0][0], CP, kb * 32, w * 16, lane);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          ya[rb] = mfma16x16x32(frag_t(&cur.G[0][0], NP, kb * 32, rb * 16, lane), af, ya[rb]);
      }
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8 xf = frag(&cur.X[0][0], XP, w * 16, kb * 32, lane);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          ya[rb] = mfma16x16x32(frag(&sm.W[0][0], XP, rb * 16, kb * 32, lane), xf, ya[rb]);
          yb[rb] = mfma16x16x32(frag(S_in, XP, rb * 16, kb * 32, lane), xf, yb[rb]);
        }
      }
      const int i = w * 16 + l16;
      const float eqi = cur.eq[i];
      if (i < cv) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          uint2 pk;
          pk.x = pack2(ya[rb][0] + eqi * yb[rb][0], ya[rb][1] + eqi * yb[rb][1]);
          pk.y = pack2(ya[rb][2] + eqi * yb[rb][2], ya[rb][3] + eqi * yb[rb][3]);
          *reinterpret_cast<uint2*>(y + (t0 + i) * D + r0 + rb * 16 + 4 * g4) = pk;
        }
      }
    }

    // state update, transposed: D^T[c][r] = Gamma D^T + sum_j x_j[c] (bk_j g_j[r]),
    // written to the other state buffer (the current one may still be read)
    __bf16 (*S_out)[XP] = sm.S[(c + 1) & 1];
    const float gam = cur.gam;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int b = wave + 4 * s, cb = b >> 1, rb = b & 1;
      sacc[s] = sacc[s] * gam;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[s] = mfma16x16x32(frag_t(&cur.X[0][0], XP, kb * 32, cb * 16, lane),
                               frag_t(&cur.Gs[0][0], NP, kb * 32, rb * 16, lane), sacc[s]);
      uint2 pk;
      pk.x = pack2(sacc[s][0], sacc[s][1]);
      pk.y = pack2(sacc[s][2], sacc[s][3]);
      *reinterpret_cast<uint2*>(&S_out[rb * 16 + l16][cb * 16 + 4 * g4]) = pk;
    }
    if (more) stage(pf, sm.ch[(c + 1) & 1], cv_of(c + 1));
    lds_barrier();  // new state and next chunk visible
  }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const int64_t groups = (a.B * a.H + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (D / kTN)));
  hipLaunchKernelGGL(fwd_mfma<D>, grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_fwd(const FwdArgs& a, hipStream_t s) {
  return a.d_in == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace gls
