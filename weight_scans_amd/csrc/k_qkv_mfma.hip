// k_qkv_mfma.hip -- the scan with a read vector and a write key of their own
// on the matrix cores for bf16 io at d_k = d_v = 128 (gfx950,
// v_mfma_f32_16x16x32_bf16):
//   y_t = (W0' + D_t) q_t,   D_{t+1} = alpha_t D_t - eta_t v_t k_t^T
// (the write key of "Parallelize the Training, Keep the Learning Serial",
// cognaptus.com, section "Once the gradient signals are known, the weight
// trajectory becomes parallelizable"; with q = u, k = g, v = x and W0' = W0^T
// it is the transpose read of the two-layer mechanism test).
//
// At this width a chunk slot with its own q tile does not fit the forward
// kernel's ring, so the scan runs in two launches: the forward kernel's
// state-only instance with x = k, g = v writes the chunk-start states D_in
// (bf16, [B*H][n_chunks][d_v][d_k]) into the caller's workspace, and this
// kernel forms every chunk's outputs from them, one work-group per
// (sequence-head, chunk):
//   A_ij = (q_i . k_j) e(lq_i - l_j)(-eta_j)                      (j < i)
//   y_i  = W0' q_i + e(lq_i) D_in q_i + sum_j A_ij v_j
// (l = chunk-local inclusive cumsum of log2 alpha, lq_i = l_{i-1}, e(.) = 2^(.)).
// Eight waves: wave w owns rows 16 w .. of y^T over all 64 tokens (its W0'
// and D_in rows as register fragments) and score blocks w and w + 8 of the
// causal triangle.  q, k and v of the chunk sit in LDS (swizzled), the
// decayed scores transposed beside them.
#include <algorithm>
#include <cstdint>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kD = 128;        // d_k = d_v
constexpr int kC = 64;         // tokens per chunk
constexpr int kNW = 8;         // waves
constexpr int kNT = 64 * kNW;  // threads

struct alignas(16) QkvLds {
  __bf16 Q[kC * kD], K[kC * kD], V[kC * kD];  // swizzled [token][128]
  __bf16 AT[kC * kC];                          // AT[j][i] = A_ij, swizzled
  float lq[kC], li[kC], nb[kC], eq[kC];        // l_{i-1}, l_i, -eta_i, e(lq_i)
  float R[kC], C[3][kC];                       // rank-one factors of the off-diagonal blocks
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kNT) void qkv_chunk(FwdArgs a) {
  __shared__ QkvLds L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int n = a.n_chunks;
  const int64_t bh = blockIdx.x / n;
  const int c = static_cast<int>(blockIdx.x % n);
  const int h = static_cast<int>(bh % a.H);
  const int64_t T = a.T, t0 = static_cast<int64_t>(c) * kC;
  const int cv = static_cast<int>(std::min<int64_t>(kC, T - t0));
  const uint16_t* q = static_cast<const uint16_t*>(a.q) + (bh * T + t0) * kD;
  const uint16_t* k = static_cast<const uint16_t*>(a.x) + (bh * T + t0) * kD;
  const uint16_t* v = static_cast<const uint16_t*>(a.g) + (bh * T + t0) * kD;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * kD * kD;
  const uint16_t* S = static_cast<const uint16_t*>(a.states) + (bh * n + c) * kD * kD;

  // ---- loads: the chunk's q, k, v (two 16-byte units per thread each, rows
  // past the sequence end zero-filled by the buffer bounds), this wave's W0'
  // and D_in rows as A fragments, and the gate rows (wave 0)
  const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q, cv * kD * 2);
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(k, cv * kD * 2);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(v, cv * kD * 2);
  u32x4 uq[2], uk[2], uv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t off = static_cast<uint32_t>((tid + kNT * j) * 16);
    uq[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    uk[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    uv[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
  }
  const int wr = wave * 16 + l16;  // this lane's row of y^T (row of W0', D_in)
  bf16x8 wf[kD / 32], sf[kD / 32];
#pragma unroll
  for (int kb = 0; kb < kD / 32; ++kb)
    sf[kb] = *reinterpret_cast<const bf16x8*>(S + static_cast<int64_t>(wr) * kD + kb * 32 + 8 * g4);
  if (a.w0_t) {  // W0' given transposed, [d_k][d_v]: gathered
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        wf[kb][e] = __builtin_bit_cast(__bf16, W0[static_cast<int64_t>(kb * 32 + 8 * g4 + e) * kD + wr]);
  } else {
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb)
      wf[kb] = *reinterpret_cast<const bf16x8*>(W0 + static_cast<int64_t>(wr) * kD + kb * 32 + 8 * g4);
  }
  float al = 1.f, et = 0.f;
  if (wave == 0 && lane < cv) {
    al = static_cast<const float*>(a.alpha)[bh * T + t0 + lane];
    et = static_cast<const float*>(a.eta)[bh * T + t0 + lane];
  }
  // the six score blocks above the diagonal stay zero
  for (int idx = tid; idx < 6 * 256; idx += kNT) {
    const int u = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
    const int ib = static_cast<int>((0x211000u >> (4 * u)) & 0xf);
    const int jb = static_cast<int>((0x332321u >> (4 * u)) & 0xf);
    L.AT[sidx<kC>(jb * 16 + r, ib * 16 + cc)] = __bf16(0.f);
  }
  if (wave == 0) {
    // gates (lane = token; padding tokens alpha = 1, eta = 0); m_b = l at the
    // end of 16-token block b - 1 splits e(lq_i - l_j) = R_i C_{b, j} for j
    // in an earlier block than i, both factors <= 1
    const ChunkGates gt = chunk_gates(al, lane);
    const float m1 = readlane_f(gt.l, 15), m2 = readlane_f(gt.l, 31), m3 = readlane_f(gt.l, 47);
    const int b = lane >> 4;
    const float mb = b == 0 ? 0.f : b == 1 ? m1 : b == 2 ? m2 : m3;
    L.lq[lane] = gt.lq;
    L.li[lane] = gt.l;
    L.nb[lane] = -et;
    L.eq[lane] = fexp2(gt.lq);
    L.R[lane] = fexp2(gt.lq - mb);
    L.C[0][lane] = -et * fexp2(fminf(m1 - gt.l, 0.f));
    L.C[1][lane] = -et * fexp2(fminf(m2 - gt.l, 0.f));
    L.C[2][lane] = -et * fexp2(fminf(m3 - gt.l, 0.f));
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = tid + kNT * j, row = u >> 4, cg = u & 15;
    const uint32_t lo = static_cast<uint32_t>(sidx<kD>(row, 8 * cg) * 2);
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(L.Q) + lo) = uq[j];
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(L.K) + lo) = uk[j];
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(L.V) + lo) = uv[j];
  }
  __syncthreads();

  // ---- decayed scores, causal blocks w and w + 8 of the ten, transposed into AT
  const LaneOff<kD> oD = lane_off<kD>(lane);
  const LaneOff<kC> oA = lane_off<kC>(lane);
  for (int b = wave; b < 10; b += kNW) {
    const int ib = tri_i(b), jb = tri_j(b);
    f32x4 xx = zero4();
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb)
      xx = mfma16x16x32(frag_s<kD>(L.Q, oD, ib * 16, kb * 32), frag_s<kD>(L.K, oD, jb * 16, kb * 32),
                        xx);
    const int jj = jb * 16 + l16, i0 = ib * 16 + 4 * g4;
    f32x4 sc;
    if (ib == jb) {  // diagonal block: decay per element, causal mask
      const float lj = L.li[jj], nj = L.nb[jj];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const float e = xx[qq] * fexp2(L.lq[i0 + qq] - lj) * nj;
        sc[qq] = jj < i0 + qq ? e : 0.f;
      }
    } else {  // every j < i: rank-one decay
      const float cj = L.C[ib - 1][jj];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) sc[qq] = xx[qq] * (L.R[i0 + qq] * cj);
    }
    uint2 pk;
    pk.x = pack2(sc[0], sc[1]);
    pk.y = pack2(sc[2], sc[3]);
    put4<kC>(L.AT, oA, jb * 16, ib * 16, pk);
  }
  __syncthreads();

  // ---- y^T[r][i] for rows 16 w .. and every token block: W0' q + e(lq) D_in q
  // (two accumulators) + V^T A^T; each lane stores 4 consecutive rows of one token
  bf16x8 vt[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) vt[kb] = frag_ts<kD>(L.V, oD, kb * 32, wave * 16);
  const __amdgpu_buffer_rsrc_t ry =
      buffer_rsrc(static_cast<uint16_t*>(a.y) + (bh * T + t0) * kD, cv * kD * 2);
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    f32x4 ya = zero4(), yb = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ya = mfma16x16x32(vt[kb], frag_ts<kC>(L.AT, oA, kb * 32, tb * 16), ya);
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb) {
      const bf16x8 qf = frag_s<kD>(L.Q, oD, tb * 16, kb * 32);
      ya = mfma16x16x32(wf[kb], qf, ya);
      yb = mfma16x16x32(sf[kb], qf, yb);
    }
    const float eqi = L.eq[tb * 16 + l16];
    uint2 pk;
    pk.x = pack2(ya[0] + eqi * yb[0], ya[1] + eqi * yb[1]);
    pk.y = pack2(ya[2] + eqi * yb[2], ya[3] + eqi * yb[3]);
    store8(ry, static_cast<uint32_t>(((tb * 16 + l16) * kD + wave * 16 + 4 * g4) * 2), pk);
  }
}

}  // namespace

bool mfma_qkv_two_pass(int io, int dk, int dv) { return io == IO_BF16 && dk == kD && dv == kD; }

size_t mfma_qkv_states_bytes(int64_t BH, int64_t T) {
  const int64_t n = (T + kC - 1) / kC;
  return static_cast<size_t>(BH * n) * kD * kD * 2;
}

// a: x = k (write key), g = v, q the read vector, states = the workspace
// that receives the chunk-start states; one segment.
hipError_t launch_mfma_qkv_two_pass(const FwdArgs& a, hipStream_t s) {
  if (a.d_in != kD || a.d_out != kD || !a.q || !a.y || !a.states || a.n_seg != 1)
    return hipErrorInvalidValue;
  FwdArgs st = a;  // the forward kernel's state-only instance (states of x = k, g = v)
  st.y = nullptr;
  st.q = nullptr;
  hipError_t e = launch_mfma_fwd(st, s);
  if (e != hipSuccess) return e;
  const int64_t groups = a.B * a.H * a.n_chunks;
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(qkv_chunk, dim3(static_cast<unsigned>(groups)), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace gls
