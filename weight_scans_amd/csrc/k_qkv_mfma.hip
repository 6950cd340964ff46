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
// state-only instance with x = k, g = v writes the chunk-start state of every
// eighth chunk (the start of each group of eight; bf16,
// [B*H][ceil(n_chunks / 8)][d_v][d_k]) into the caller's workspace, and this
// kernel walks every group's chunks in order, one work-group per
// (sequence-head, group), carrying D in fp32 registers:
//   A_ij = (q_i . k_j) e(lq_i - l_j)(-eta_j)                      (j < i)
//   y_i  = W0' q_i + e(lq_i) D_in q_i + sum_j A_ij v_j
//   D_out = e(l_last) D_in + sum_j e(l_last - l_j)(-eta_j) v_j k_j^T
// (l = chunk-local inclusive cumsum of log2 alpha, lq_i = l_{i-1}, e(.) = 2^(.)).
// Eight waves: wave w owns rows 16 w .. of D and of y^T over all 64 tokens
// (its W0' rows as register fragments for the whole walk) and score blocks w
// and w + 8 of the causal triangle.  q, k and v of the chunk sit in LDS
// (swizzled), the decayed scores transposed beside them.
//
// The products over k (W0' q and D_in q) take the 32 k of each step in a
// permuted order: lane group g holds k = 4 g .. 4 g + 3 and 16 + 4 g .. 16 +
// 4 g + 3 of the step rather than 8 g .. 8 g + 7.  That is the order in which
// the state update's matrix-core result leaves D in each lane, so the bf16
// D_in fragments are packed from the fp32 registers directly; the q
// fragments are read in the same order (two 8-byte reads), which leaves each
// product's sum unchanged.
#include <algorithm>
#include <cstdint>

#include "bwd_fused.hpp"
#include "dev_common.hpp"

namespace gls {
namespace {

constexpr int kD = 128;        // d_k = d_v
constexpr int kC = 64;         // tokens per chunk
constexpr int kNW = 8;         // waves
constexpr int kNT = 64 * kNW;  // threads

constexpr int kGroup = 8;       // chunks per work-group (one kept state each)

struct alignas(16) QkvLds {
  float lq[kC], li[kC], nb[kC], eq[kC];        // l_{i-1}, l_i, -eta_i, e(lq_i)
  float R[kC], C[3][kC];                       // rank-one factors of the off-diagonal blocks
  float wu[kC];                                // e(l_last - l_j)(-eta_j): the state update
  float gam;                                   // e(l_last)
  float pad[3];
  __bf16 AT[kC * kC];                          // AT[j][i] = A_ij, swizzled
  __bf16 Q[kC * kD], K[kC * kD], V[kC * kD];   // swizzled [token][128]
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 8 bf16 from two 4-element halves
__device__ __forceinline__ bf16x8 join8(const uint2& lo, const uint2& hi) {
  const u32x4 u = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, u);
}

__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(4, 4))) void qkv_group(FwdArgs a,
                                                                                      int n_grp) {
  __shared__ QkvLds L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int n = a.n_chunks;
  const int64_t bh = blockIdx.x / n_grp;
  const int grp = static_cast<int>(blockIdx.x % n_grp);
  const int c_beg = grp * kGroup, c_end = std::min(n, c_beg + kGroup);
  const int h = static_cast<int>(bh % a.H);
  const int64_t T = a.T;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * kD * kD;
  const int wr = wave * 16 + l16;  // this lane's row of D and y^T (row of W0')

  // this wave's W0' rows as A fragments, k in the permuted order of each
  // 32-wide step (lane group g4: 4 g4 .. + 3 and 16 + 4 g4 .. + 3)
  bf16x8 wf[kD / 32];
  if (a.w0_t) {  // W0' given transposed, [d_k][d_v]: gathered once
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = kb * 32 + 4 * g4 + (e & 3) + 16 * (e >> 2);
        wf[kb][e] = __builtin_bit_cast(__bf16, W0[static_cast<int64_t>(kk) * kD + wr]);
      }
  } else {
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb) {
      const uint16_t* wp = W0 + static_cast<int64_t>(wr) * kD + kb * 32 + 4 * g4;
      wf[kb] = join8(*reinterpret_cast<const uint2*>(wp), *reinterpret_cast<const uint2*>(wp + 16));
    }
  }
  // the state entering the group (bf16 in the workspace) in fp32 registers:
  // ds[cb][q] = D[wr][16 cb + 4 g4 + q]
  f32x4 ds[kD / 16];
  {
    const uint16_t* S = static_cast<const uint16_t*>(a.states) + (bh * n_grp + grp) * kD * kD +
                        static_cast<int64_t>(wr) * kD + 4 * g4;
#pragma unroll
    for (int cb = 0; cb < kD / 16; ++cb) ds[cb] = unpack4f(*reinterpret_cast<const uint2*>(S + 16 * cb));
  }
  // the six score blocks above the diagonal stay zero for the whole walk
  for (int idx = tid; idx < 6 * 256; idx += kNT) {
    const int u = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
    const int ib = static_cast<int>((0x211000u >> (4 * u)) & 0xf);
    const int jb = static_cast<int>((0x332321u >> (4 * u)) & 0xf);
    L.AT[sidx<kC>(jb * 16 + r, ib * 16 + cc)] = __bf16(0.f);
  }
  const LaneOff<kD> oD = lane_off<kD>(lane);
  const LaneOff<kC> oA = lane_off<kC>(lane);

  for (int c = c_beg; c < c_end; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = static_cast<int>(std::min<int64_t>(kC, T - t0));
    // ---- loads: the chunk's q, k, v (two 16-byte units per thread each,
    // rows past the sequence end zero-filled by the buffer bounds) and the
    // gate rows (every wave; wave 0 uses them)
    const int64_t tok = (bh * T + t0) * kD;
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(static_cast<const uint16_t*>(a.q) + tok, cv * kD * 2);
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(static_cast<const uint16_t*>(a.x) + tok, cv * kD * 2);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(static_cast<const uint16_t*>(a.g) + tok, cv * kD * 2);
    u32x4 uq[2], uk[2], uv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t off = static_cast<uint32_t>((tid + kNT * j) * 16);
      uq[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      uk[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      uv[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
    const uint32_t go = static_cast<uint32_t>(lane * 4);
    const float et = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        buffer_rsrc(static_cast<const float*>(a.eta) + bh * T + t0, cv * 4), go, 0, 0));
    const float al_l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        buffer_rsrc(static_cast<const float*>(a.alpha) + bh * T + t0, cv * 4), go, 0, 0));
    __syncthreads();  // the previous chunk is done with every LDS array
    if (wave == 0) {
      // gates (lane = token; padding tokens alpha = 1, eta = 0); m_b = l at
      // the end of 16-token block b - 1 splits e(lq_i - l_j) = R_i C_{b, j}
      // for j in an earlier block than i, both factors <= 1
      const ChunkGates gt = chunk_gates(lane < cv ? al_l : 1.f, lane);
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
      L.wu[lane] = -et * fexp2(gt.llast - gt.l);
      if (lane == 0) L.gam = fexp2(gt.llast);
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
    // (two accumulators, k permuted as above) + V^T A^T; each lane stores 4
    // consecutive rows of one token
    bf16x8 df[kD / 32];  // D_in rows as A fragments, from the fp32 registers
#pragma unroll
    for (int kb = 0; kb < kD / 32; ++kb) df[kb] = join8(pack4f(ds[2 * kb]), pack4f(ds[2 * kb + 1]));
    bf16x8 vt[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) vt[kb] = frag_ts<kD>(L.V, oD, kb * 32, wave * 16);
    const __amdgpu_buffer_rsrc_t ry =
        buffer_rsrc(static_cast<uint16_t*>(a.y) + (bh * T + t0) * kD, cv * kD * 2);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      __builtin_amdgcn_sched_barrier(0);
      f32x4 ya = zero4(), yb = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        ya = mfma16x16x32(vt[kb], frag_ts<kC>(L.AT, oA, kb * 32, tb * 16), ya);
#pragma unroll
      for (int kb = 0; kb < kD / 32; ++kb) {
        const bf16x8 qf = join8(get4<kD>(L.Q, oD, tb * 16, kb * 32), get4<kD>(L.Q, oD, tb * 16, kb * 32 + 16));
        ya = mfma16x16x32(wf[kb], qf, ya);
        yb = mfma16x16x32(df[kb], qf, yb);
      }
      const float eqi = L.eq[tb * 16 + l16];
      uint2 pk;
      pk.x = pack2(ya[0] + eqi * yb[0], ya[1] + eqi * yb[1]);
      pk.y = pack2(ya[2] + eqi * yb[2], ya[3] + eqi * yb[3]);
      store8(ry, static_cast<uint32_t>(((tb * 16 + l16) * kD + wave * 16 + 4 * g4) * 2), pk);
    }
    // ---- D_out = e(l_last) D_in + (k^T diag(wu) v)^T for rows 16 w ..
    // (operands swapped: the product comes out in ds's layout)
    __builtin_amdgcn_sched_barrier(0);
    {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&L.wu[8 * g4]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&L.wu[8 * g4 + 4]);
      const f32x4 w2 = *reinterpret_cast<const f32x4*>(&L.wu[32 + 8 * g4]);
      const f32x4 w3 = *reinterpret_cast<const f32x4*>(&L.wu[32 + 8 * g4 + 4]);
      const bf16x8 vw[2] = {scale8(vt[0], w0, w1), scale8(vt[1], w2, w3)};
      const float gam = L.gam;
#pragma unroll
      for (int cb = 0; cb < kD / 16; ++cb) {
        f32x4 u = ds[cb] * gam;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) u = mfma16x16x32(frag_ts<kD>(L.K, oD, kb * 32, cb * 16), vw[kb], u);
        ds[cb] = u;
      }
    }
  }
}

}  // namespace

bool mfma_qkv_two_pass(int io, int dk, int dv) { return io == IO_BF16 && dk == kD && dv == kD; }

size_t mfma_qkv_states_bytes(int64_t BH, int64_t T) {
  const int64_t n = (T + kC - 1) / kC;
  return static_cast<size_t>(BH * ((n + kGroup - 1) / kGroup)) * kD * kD * 2;
}

// a: x = k (write key), g = v, q the read vector, states = the workspace
// that receives the group-start states; one segment.
hipError_t launch_mfma_qkv_two_pass(const FwdArgs& a, hipStream_t s) {
  if (a.d_in != kD || a.d_out != kD || !a.q || !a.y || !a.states || a.n_seg != 1)
    return hipErrorInvalidValue;
  FwdArgs st = a;  // the forward kernel's state-only instance (states of x = k, g = v)
  st.y = nullptr;
  st.q = nullptr;
  st.st_every = kGroup;
  hipError_t e = launch_mfma_fwd(st, s);
  if (e != hipSuccess) return e;
  const int n_grp = (a.n_chunks + kGroup - 1) / kGroup;
  const int64_t groups = a.B * a.H * n_grp;
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(qkv_group, dim3(static_cast<unsigned>(groups)), dim3(kNT), 0, s, a, n_grp);
  return hipGetLastError();
}

}  // namespace gls
