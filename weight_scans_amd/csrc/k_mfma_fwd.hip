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

template <int D>
struct FwdSmem {
  static constexpr int XP = D + 8;    // row stride of [token][D] tiles (elements)
  static constexpr int NP = kTN + 8;  // row stride of [token][kTN] tiles
  static constexpr int CP = kC + 8;   // row stride of [token][token] tiles
  __bf16 X[kC][XP];                   // x of the chunk
  __bf16 G[kC][NP];                   // g of the row tile
  __bf16 Gs[kC][NP];                  // e(l_last - l_j)(-eta_j) g_j
  __bf16 AT[kC][CP];                  // AT[j][i] = A_ij
  __bf16 S[kTN][XP];                  // D_in of the tile, bf16 [row][col]
  __bf16 W[kTN][XP];                  // W0 of the tile [row][col]
  __bf16 Y[kC][NP];                   // y staging [token][row]
  float lq[kC], li[kC], eq[kC], neta[kC];
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
  r.x = bf16_bits(bf16_val(v.x & 0xffffu) * s) | (bf16_bits(bf16_val(v.x >> 16) * s) << 16);
  r.y = bf16_bits(bf16_val(v.y & 0xffffu) * s) | (bf16_bits(bf16_val(v.y >> 16) * s) << 16);
  r.z = bf16_bits(bf16_val(v.z & 0xffffu) * s) | (bf16_bits(bf16_val(v.z >> 16) * s) << 16);
  r.w = bf16_bits(bf16_val(v.w & 0xffffu) * s) | (bf16_bits(bf16_val(v.w >> 16) * s) << 16);
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
    *reinterpret_cast<uint4*>(&sm.S[r][cc]) = make_uint4(0, 0, 0, 0);
  }
  for (int idx = tid; idx < kC * CP; idx += kNT) (&sm.AT[0][0])[idx] = static_cast<__bf16>(0.f);

  f32x4 sacc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) sacc[s] = zero4();

  Prefetch<D> pf;
  load_chunk<D>(pf, x, g, eta, alpha, 0, static_cast<int>(std::min<int64_t>(kC, T)), r0, tid);

  for (int c = 0; c < a.n_chunks; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = static_cast<int>(std::min<int64_t>(kC, T - t0));

    // ---- gates (every wave, lane = token) and staging of the chunk
    const float et = lane < cv ? pf.eta : 0.f;
    const ChunkGates gt = chunk_gates(lane < cv ? pf.alpha : 1.f, lane);
    const float bk = -et * fexp2(gt.llast - gt.l);
    const float gam = fexp2(gt.llast);
    if (wave == 0) {
      sm.lq[lane] = gt.lq;
      sm.li[lane] = gt.l;
      sm.eq[lane] = fexp2(gt.lq);
      sm.neta[lane] = -et;
    }
#pragma unroll
    for (int s = 0; s < RPT; ++s)
      *reinterpret_cast<uint4*>(&sm.X[rg * RPT + s][8 * cg]) = keep_row(pf.x[s], rg * RPT + s, cv);
    {
      const uint4 gv = keep_row(pf.g, jg, cv);
      *reinterpret_cast<uint4*>(&sm.G[jg][c8]) = gv;
      *reinterpret_cast<uint4*>(&sm.Gs[jg][c8]) = scale_bf16x8(gv, __shfl(bk, jg, 64));
    }
    lds_barrier();  // B1: chunk tiles and gates visible
    {
      // prefetch the next chunk (the last chunk is re-read and ignored)
      const int cn = std::min(c + 1, a.n_chunks - 1);
      const int64_t t1 = static_cast<int64_t>(cn) * kC;
      load_chunk<D>(pf, x, g, eta, alpha, t1, static_cast<int>(std::min<int64_t>(kC, T - t1)),
                    r0, tid);
    }

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
            xx = mfma16x16x32(frag(&sm.X[0][0], XP, ib * 16, kb * 32, lane),
                              frag(&sm.X[0][0], XP, jb * 16, kb * 32, lane), xx);
          const int j = jb * 16 + l16, i0 = ib * 16 + 4 * g4;
          const float lj = sm.li[j], nj = sm.neta[j];
          const f32x4 lqi = *reinterpret_cast<const f32x4*>(&sm.lq[i0]);
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float e = xx[q] * fexp2(lqi[q] - lj) * nj;
            v[q] = (j < i0 + q) ? e : 0.f;
          }
          uint2 pk;
          pk.x = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
          pk.y = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
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
        v.x = bf16_bits(sacc[s][0]) | (bf16_bits(sacc[s][1]) << 16);
        v.y = bf16_bits(sacc[s][2]) | (bf16_bits(sacc[s][3]) << 16);
        *reinterpret_cast<uint2*>(st + (static_cast<int64_t>(c) * D + r0 + rb * 16 + l16) * D +
                                  cb * 16 + 4 * g4) = v;
      }
    }
    lds_barrier();  // B2: scores visible

    if (y) {
      // y^T[r][i] for i in this wave's token block, both row blocks
      const int w = wave;
      f32x4 ya[2] = {zero4(), zero4()}, yb[2] = {zero4(), zero4()};
      for (int kb = 0; kb < (w + 2) / 2; ++kb) {
        const bf16x8 af = frag_t(&sm.AT[0][0], CP, kb * 32, w * 16, lane);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          ya[rb] = mfma16x16x32(frag_t(&sm.G[0][0], NP, kb * 32, rb * 16, lane), af, ya[rb]);
      }
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8 xf = frag(&sm.X[0][0], XP, w * 16, kb * 32, lane);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          ya[rb] = mfma16x16x32(frag(&sm.W[0][0], XP, rb * 16, kb * 32, lane), xf, ya[rb]);
          yb[rb] = mfma16x16x32(frag(&sm.S[0][0], XP, rb * 16, kb * 32, lane), xf, yb[rb]);
        }
      }
      const int i = w * 16 + l16;
      const float eqi = sm.eq[i];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        uint2 pk;
        pk.x = bf16_bits(ya[rb][0] + eqi * yb[rb][0]) | (bf16_bits(ya[rb][1] + eqi * yb[rb][1]) << 16);
        pk.y = bf16_bits(ya[rb][2] + eqi * yb[rb][2]) | (bf16_bits(ya[rb][3] + eqi * yb[rb][3]) << 16);
        *reinterpret_cast<uint2*>(&sm.Y[i][rb * 16 + 4 * g4]) = pk;
      }
    }
    lds_barrier();  // B3: y staged; reads of S, AT, G done

    if (y && jg < cv)
      *reinterpret_cast<uint4*>(y + (t0 + jg) * D + r0 + c8) =
          *reinterpret_cast<const uint4*>(&sm.Y[jg][c8]);
    // state update, transposed: D^T[c][r] = Gamma D^T + sum_j x_j[c] (bk_j g_j[r])
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int b = wave + 4 * s, cb = b >> 1, rb = b & 1;
      sacc[s] = sacc[s] * gam;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[s] = mfma16x16x32(frag_t(&sm.X[0][0], XP, kb * 32, cb * 16, lane),
                               frag_t(&sm.Gs[0][0], NP, kb * 32, rb * 16, lane), sacc[s]);
      uint2 pk;
      pk.x = bf16_bits(sacc[s][0]) | (bf16_bits(sacc[s][1]) << 16);
      pk.y = bf16_bits(sacc[s][2]) | (bf16_bits(sacc[s][3]) << 16);
      *reinterpret_cast<uint2*>(&sm.S[rb * 16 + l16][cb * 16 + 4 * g4]) = pk;
    }
    lds_barrier();  // B4: new state visible; chunk tiles free
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
