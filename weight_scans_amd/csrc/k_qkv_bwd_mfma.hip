// k_qkv_bwd_mfma.hip -- the reverse scan of the scan with a read vector and a
// write key of their own on the matrix cores, bf16 io, d_k = d_v = D in
// {64, 128} (gfx950, v_mfma_f32_16x16x32_bf16).
//
//   y_t = (W0' + D_t) q_t,   D_{t+1} = alpha_t D_t - eta_t v_t k_t^T
// and its exact adjoint for L = sum_t <dy_t, y_t> (the recurrence is affine
// in D, so its adjoint is the same recurrence run backwards: "Parallelize
// the Training, Keep the Learning Serial", cognaptus.com, section "Once the
// gradient signals are known, the weight trajectory becomes
// parallelizable"), with A_{t+1} = dL/dD_{t+1}:
//   dq_t = (W0' + D_t)^T dy_t,  dk_t = -eta_t A_{t+1}^T v_t,  dv_t = -eta_t A_{t+1} k_t,
//   deta_t = -v_t^T A_{t+1} k_t,  dalpha_t = <A_{t+1}, D_t>,  dW0' = sum dy_t q_t^T.
// Per chunk of 64 tokens (l = chunk-local inclusive cumsum of log2 alpha,
// lq_t = l_{t-1}, e(.) = 2^(.), D_in / A_out the carries at the chunk's ends):
//   D_t     = e(lq_t) D_in + sum_{j<t} e(lq_t - l_j)(-eta_j) v_j k_j^T
//   A_{t+1} = e(l_last - l_t) A_out + sum_{u>t} e(lq_u - l_t) dy_u q_u^T
// so that, with P_ut = e(lq_u - l_t)(q_u . k_t) and
// Be_tj = e(lq_t - l_j)(-eta_j)(dy_t . v_j) (zero unless the first index is the later token):
//   dq = W0'^T dy + e(lq) D_in^T dy + Be K
//   u  = e(l_last - l) A_out k + P^T dy,   dv = -eta u,   deta = -v . u
//   dk = Be^T Q - eta e(l_last - l) A_out^T v
// and dalpha from <A_out, D_in>, pp_j = v_j . (A_out k_j), rr_u = q_u . (D_in^T dy_u)
// and the row / column sums of Be o (Q K^T) (the same identity as the scan's).
//
// Chunks are taken in groups (a.grp_chunks of them, chosen by the host:
// sixteen, fewer when that would leave the GPU short of work-groups).  Five
// launches: the forward
// kernel's state-only instance (x = k, g = v) writes D_in of every chunk
// (bf16); qkv_bwd_inc forms every group's adjoint increment (the chunk
// formula over the group's tokens: sum_u e(L_{u-1}) dy_u q_u^T with L the
// group-local cumsum of log2 alpha), its decay and its dW0' share;
// qkv_grp_carry turns the increments into the adjoint leaving every group;
// qkv_bwd_chunk walks the chunks of its group from right to left carrying
// the adjoint in fp32 registers (A_in = e(l_last) A_out + sum_u e(lq_u)
// dy_u q_u^T) and forms every chunk's gradients from its tiles and the two
// carries; the finalize kernel sums the dW0' shares in a fixed order.  At
// D = 128 with W0' not given transposed, a small kernel first writes W0'
// transposed into the workspace (the gradient kernel reads its fragments
// from there).
#include <algorithm>
#include <cstdint>

#include "bwd_fused.hpp"

namespace gls {
namespace {

constexpr int kCk = 64;   // tokens per chunk

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte unit u (D / 8 per row) of a [rows][D] bf16 tile: its swizzled LDS
// offset in bytes.
template <int D>
__device__ __forceinline__ uint32_t unit_off(int u) {
  return static_cast<uint32_t>(sidx<D>(u / (D / 8), 8 * (u % (D / 8))) * 2);
}
template <int D>
__device__ __forceinline__ void put_unit(__bf16* tile, int u, const u32x4& v) {
  *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(tile) + unit_off<D>(u)) = v;
}

// ---- adjoint increment, decay and dW0' share of every group ----
// Work-group (bh, group), D / 16 waves (wave w: rows 16 w .. of the
// increment and of the dW0' share), walks the chunks of its group in order;
// the loads of the next two chunks are in flight while the current one is
// multiplied.
template <int D>
struct alignas(16) IncLds {
  __bf16 Q[kCk * D], DY[kCk * D];  // swizzled [token][D]
  float eq[kCk];                   // e(L_{u-1}) from the group's start
};

template <int D>
__global__ __launch_bounds__(4 * D) void qkv_bwd_inc(BwdArgs a, int n_grp) {
  constexpr int NT = 4 * D, NB = D / 16;
  __shared__ IncLds<D> L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int n = a.n_chunks;
  const int64_t bh = blockIdx.x / n_grp, BH = a.B * a.H;
  const int grp = static_cast<int>(blockIdx.x % n_grp);
  const int c_beg = grp * a.grp_chunks, c_end = std::min(n, c_beg + a.grp_chunks);
  const int64_t T = a.T, dd = static_cast<int64_t>(D) * D;
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + bh * T * D;
  const uint16_t* db = static_cast<const uint16_t*>(a.dy) + bh * T * D;
  // two chunks in flight: 8 D units per tile, two per thread, and the
  // lane's alpha (raw: the padding select is made where it is used, so that
  // no wait follows the loads)
  u32x4 uq[2][2], ud[2][2];
  float alr[2];
  // every step issues the same loads (past the group's end into empty
  // buffers), so the waits the compiler places are the same in every step
  const auto valid = [&](int c) {
    return c < c_end ? static_cast<int>(std::min<int64_t>(kCk, T - static_cast<int64_t>(c) * kCk))
                     : 0;
  };
  const auto fetch = [&](auto PC, int c) {
    constexpr int P = decltype(PC)::value;
    const int cv = valid(c);
    const int64_t t0 = cv > 0 ? static_cast<int64_t>(c) * kCk : 0;
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(qb + t0 * D, cv * D * 2);
    const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(db + t0 * D, cv * D * 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t off = static_cast<uint32_t>((tid + NT * j) * 16);
      uq[P][j] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      ud[P][j] = __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t ra =
        buffer_rsrc(static_cast<const float*>(a.alpha) + bh * T + t0, cv * 4);
    alr[P] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(ra, static_cast<uint32_t>(lane * 4), 0, 0));
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  fetch(I0{}, c_beg);
  fetch(I1{}, c_beg + 1);
  const LaneOff<D> o = lane_off<D>(lane);
  const int rb = wave;
  // accumulators in the transposed MFMA layout (operands swapped): lane
  // holds row r = rb 16 + l16, columns k = cb 16 + 4 g4 .. + 3
  f32x4 w[NB], v[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) w[cb] = v[cb] = zero4();
  float lg = 0.f;  // log2 of the decay from the group's start to chunk c (wave 0)
  const auto step = [&](auto PC, int c) {
    constexpr int P = decltype(PC)::value;
    __syncthreads();  // the previous chunk's fragment reads are done
    if (wave == 0) {
      const ChunkGates gt = chunk_gates(lane < valid(c) ? alr[P] : 1.f, lane);
      L.eq[lane] = fexp2(lg + gt.lq);
      lg += gt.llast;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      put_unit<D>(L.Q, tid + NT * j, uq[P][j]);
      put_unit<D>(L.DY, tid + NT * j, ud[P][j]);
    }
    fetch(PC, c + 2);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 df = frag_ts<D>(L.DY, o, kb * 32, rb * 16);
      const f32x4 e0 = *reinterpret_cast<const f32x4*>(&L.eq[kb * 32 + 8 * g4]);
      const f32x4 e1 = *reinterpret_cast<const f32x4*>(&L.eq[kb * 32 + 8 * g4 + 4]);
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const bf16x8 qf = frag_ts<D>(L.Q, o, kb * 32, cb * 16);
        w[cb] = mfma16x16x32(qf, df, w[cb]);
        v[cb] = mfma16x16x32(scale8(qf, e0, e1), df, v[cb]);
      }
    }
  };
  // (the loop's back edge always follows both steps, so the waits in it see
  // one pattern of loads)
  int c = c_beg;
  for (; c + 1 < c_end; c += 2) {
    step(I0{}, c);
    step(I1{}, c + 1);
  }
  if (c < c_end) step(I0{}, c);
  // the group's increment arrives at the group before it (fp32); its decay
  const int r = rb * 16 + l16;
  if (grp > 0) {
    float* pv = static_cast<float*>(a.mf_lam) + (bh * n_grp + grp - 1) * dd;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
      *reinterpret_cast<f32x4*>(pv + r * D + cb * 16 + 4 * g4) = v[cb];
  }
  if (tid == 0) static_cast<float*>(a.mf_gam)[bh * n_grp + grp] = fexp2(lg);
  float* pw = static_cast<float*>(a.part_dW0) + (static_cast<int64_t>(grp) * BH + bh) * dd;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int k = cb * 16 + 4 * g4;
    if (a.w0_t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) pw[(k + q) * D + r] = w[cb][q];
    } else {
      *reinterpret_cast<f32x4*>(pw + r * D + k) = w[cb];
    }
  }
}

// ---- the adjoint leaving every group, from the group increments (fp32):
// slot g holds the increment of group g + 1 on entry and the adjoint
// leaving group g on exit; zero for the last group, then
// A_out(g) = gam(g + 1) A_out(g + 1) + V(g + 1).
constexpr int kCarryT = 256;  // threads per work-group; four elements per thread
constexpr int kCarryG = 16;   // groups whose loads are issued together

__global__ __launch_bounds__(kCarryT) void qkv_grp_carry(float* buf, const float* gam, int ng,
                                                          int dd, int n_eb) {
  const int64_t bh = blockIdx.x / n_eb;
  const int e4 = static_cast<int>(blockIdx.x % n_eb) * kCarryT + threadIdx.x;  // < dd / 4
  float* p = buf + bh * ng * static_cast<int64_t>(dd) + 4 * e4;
  const float* gm = gam + bh * ng;
  f32x4 carry = zero4();
  for (int k0 = 0; k0 < ng; k0 += kCarryG) {
    f32x4 inc[kCarryG];
    float dec[kCarryG];
#pragma unroll
    for (int j = 0; j < kCarryG; ++j) {
      const int k = k0 + j, g = ng - 1 - k;
      const bool use = k >= 1 && k < ng;
      inc[j] = use ? *reinterpret_cast<const f32x4*>(p + static_cast<int64_t>(g) * dd) : zero4();
      dec[j] = use ? gm[g + 1] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kCarryG; ++j) {
      const int k = k0 + j;
      if (k < ng) {
        carry = dec[j] * carry + inc[j];
        *reinterpret_cast<f32x4*>(p + static_cast<int64_t>(ng - 1 - k) * dd) = carry;
      }
    }
  }
}

// ---- W0' transposed ([H][D][D], [r][k] -> [k][r]) for the d = 128
// gradient kernel, which reads W0' fragments from global memory
__global__ __launch_bounds__(256) void qkv_w0_transpose(const uint16_t* w, uint16_t* wt, int D,
                                                         int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t dd = static_cast<int64_t>(D) * D;
  const int64_t h = i / dd, e = i % dd;
  const int64_t k = e / D, r = e % D;  // output element [h][k][r]
  wt[i] = w[h * dd + r * D + k];
}

// ---- the gradients of every chunk ----
// Work-group (bh, group), D / 8 waves, walks the chunks of its group from
// right to left.  The adjoint A_out of the chunk at hand is kept in fp32
// registers (wave w: D / 32 of the 16 x 16 blocks of A, block b holding rows
// r = 16 (b / (D / 16)) + l16, columns 16 (b % (D / 16)) + 4 g4 .. + 3) and
// copied to LDS in bf16 for the products.  At D = 64 W0' is staged in LDS
// once; at D = 128 (no LDS room left) its fragments are read from global
// memory, from W0' stored [k][r].
template <int D>
struct alignas(16) GradLds {
  // the small per-chunk arrays first: their addresses stay within the 64 KB
  // reach of the LDS instructions' offset field
  RecF rc;
  QkF qk;
  float pp[D / 32][kCk], rr[D / 32][kCk], de[D / 32][kCk];  // shares over column groups
  float c0[D / 8];
  __bf16 PT[kCk * kCk], BT[kCk * kCk];       // PT[t][u] = P_ut, BT[j][t] = Be_tj
  __bf16 Q[kCk * D], K[kCk * D], V[kCk * D], DY[kCk * D];  // swizzled [token][D]
  __bf16 S[D * D], A[D * D];                 // D_in [r][k], A_out [r][k]
  __bf16 W[D == 64 ? D * D : 8];             // W0' as stored (D = 64)
};

// dalpha and deta of the chunk whose gates, sums and shares sit in L (wave
// 0, lane = token): t0 its first token, cv its valid tokens; NC shares of
// <A_out, D_in> (one per wave).
template <int D, int NC = D / 8>
__device__ __forceinline__ void chunk_gate_grads(const GradLds<D>& L, const BwdArgs& a, int64_t bh,
                                                 int64_t t0, int cv, int lane) {
  const int ir = kCk - 1 - lane;
  float c0 = 0.f;
#pragma unroll
  for (int w = 0; w < NC; ++w) c0 += L.c0[w];
  float ppl = 0.f, rr_r = 0.f, del = 0.f;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    ppl += L.pp[j][lane];
    rr_r += L.rr[j][ir];
    del += L.de[j][lane];
  }
  const float da = dalpha_f(L.rc, L.qk, ppl, rr_r, c0, lane);
  store4(buffer_rsrc(static_cast<float*>(a.dalpha_out) + bh * a.T + t0, cv * 4),
         static_cast<uint32_t>(lane * 4), da);
  store4(buffer_rsrc(static_cast<float*>(a.deta_out) + bh * a.T + t0, cv * 4),
         static_cast<uint32_t>(lane * 4), del);
}

template <int D>
__global__ __launch_bounds__(8 * D) __attribute__((amdgpu_waves_per_eu(4, 4))) void qkv_bwd_chunk(
    BwdArgs a, int n_grp) {
  constexpr int NT = 8 * D, NW = D / 8, NB = D / 16, NA = D / 32, KS = D / 32;
  __shared__ GradLds<D> L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int n = a.n_chunks;
  const int64_t bh = blockIdx.x / n_grp;
  const int grp = static_cast<int>(blockIdx.x % n_grp);
  const int c_beg = grp * a.grp_chunks, c_end = std::min(n, c_beg + a.grp_chunks);
  const int h = static_cast<int>(bh % a.H);
  const int64_t T = a.T;
  const int64_t dd = static_cast<int64_t>(D) * D;
  const uint32_t off = static_cast<uint32_t>(tid * 16);

  if constexpr (D == 64)
    put_unit<D>(L.W, tid,
                *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.W0) + h * dd + 8 * tid));
  // W0' stored [k][r] (D = 128): the given one if transposed, else the copy
  const uint16_t* wt = static_cast<const uint16_t*>(a.w0_t ? a.W0 : a.W0t) + h * dd;
  // the adjoint leaving the group (zero for the last one)
  f32x4 A[NA];
  {
    const float* pa = static_cast<const float*>(a.mf_lam) + (bh * n_grp + grp) * dd;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int b = NA * wave + i;
      A[i] = *reinterpret_cast<const f32x4*>(pa + ((b / NB) * 16 + l16) * D + (b % NB) * 16 +
                                             4 * g4);
    }
  }

  LaneOff<D> o = lane_off<D>(lane);
  LaneOff<kCk> o64 = lane_off<kCk>(lane);
  for (int c = c_end - 1; c >= c_beg; --c) {
    if constexpr (D == 128) {
      // Most of this kernel's LDS lies beyond the 64 KB reach of the LDS
      // instructions' offset field, so each (array, column block) address
      // needs a register of its own; hoisted out of the chunk loop they
      // overflow the 128 registers of sixteen waves.  An empty asm on the
      // lane offsets makes them new values every chunk: the addresses are
      // formed where they are used instead.
      asm volatile("" : "+v"(o.b), "+v"(o.t0), "+v"(o.t1), "+v"(o.w));
      asm volatile("" : "+v"(o64.b), "+v"(o64.t0), "+v"(o64.t1), "+v"(o64.w));
    }
    const int64_t t0 = static_cast<int64_t>(c) * kCk;
    const int cv = static_cast<int>(std::min<int64_t>(kCk, T - t0));
    const int64_t tok = (bh * T + t0) * D;
    // this chunk's tiles: one 16-byte unit per thread of q, k, v, dy
    // (8 D units each) and D / 64 of D_in; its lane's gates
    const auto rs = [&](const void* base) {
      return buffer_rsrc(static_cast<const uint16_t*>(base) + tok, cv * D * 2);
    };
    const u32x4 uq = __builtin_amdgcn_raw_buffer_load_b128(rs(a.q), off, 0, 0);
    const u32x4 uk = __builtin_amdgcn_raw_buffer_load_b128(rs(a.x), off, 0, 0);
    const u32x4 uv = __builtin_amdgcn_raw_buffer_load_b128(rs(a.g), off, 0, 0);
    const u32x4 ud = __builtin_amdgcn_raw_buffer_load_b128(rs(a.dy), off, 0, 0);
    const __amdgpu_buffer_rsrc_t rst =
        buffer_rsrc(static_cast<const uint16_t*>(a.states) + (bh * n + c) * dd, D * D * 2);
    u32x4 us[D / 64];
#pragma unroll
    for (int j = 0; j < D / 64; ++j)
      us[j] = __builtin_amdgcn_raw_buffer_load_b128(rst, off + NT * 16 * j, 0, 0);
    const uint32_t go = static_cast<uint32_t>(lane * 4);
    const float eta_l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        buffer_rsrc(static_cast<const float*>(a.eta) + bh * T + t0, cv * 4), go, 0, 0));
    const float al_l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        buffer_rsrc(static_cast<const float*>(a.alpha) + bh * T + t0, cv * 4), go, 0, 0));
    __syncthreads();  // the previous chunk is done with every tile and share
    if (wave == 0) {
      // dalpha and deta of the previous chunk in walk order (the one to the
      // right) from its gates, sums and shares, then this chunk's gates in
      // their place (the other arrays are rewritten only after the next barrier)
      if (c + 1 < c_end) {
        const int64_t tp = t0 + kCk;
        chunk_gate_grads<D>(L, a, bh, tp, static_cast<int>(std::min<int64_t>(kCk, T - tp)), lane);
      }
      gates_v(eta_l, lane < cv ? al_l : 1.f, L.rc, lane);
    }
    // P^T and Be^T start at zero (only the causal parts are written)
    if (tid < kCk * kCk / 8) {
      reinterpret_cast<u32x4*>(L.PT)[tid] = u32x4{0u, 0u, 0u, 0u};
      reinterpret_cast<u32x4*>(L.BT)[tid] = u32x4{0u, 0u, 0u, 0u};
    }
    put_unit<D>(L.Q, tid, uq);
    put_unit<D>(L.K, tid, uk);
    put_unit<D>(L.V, tid, uv);
    put_unit<D>(L.DY, tid, ud);
#pragma unroll
    for (int j = 0; j < D / 64; ++j) put_unit<D>(L.S, tid + NT * j, us[j]);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int b = NA * wave + i;
      put4<D>(L.A, o, (b / NB) * 16, (b % NB) * 16, pack4f(A[i]));
    }
    __syncthreads();

    // <A_out, D_in> over this wave's blocks (A_out in fp32)
    {
      float cp = 0.f;
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int b = NA * wave + i;
        cp += dot4f(A[i], unpack4f(get4<D>(L.S, o, (b / NB) * 16, (b % NB) * 16)));
      }
      cp = wave_sum(cp);
      if (lane == 0) L.c0[wave] = cp;
    }
    // ---- causal blocks (ten): Q K^T and DY V^T, decayed; P and Be
    // written transposed, the row / column sums of Be o (Q K^T)
    for (int b = wave; b < 10; b += NW) {
      __builtin_amdgcn_sched_barrier(0);
      const int ib = tri_i(b), jb = tri_j(b);
      f32x4 qk = zero4(), dv = zero4();
#pragma unroll
      for (int kb = 0; kb < KS; ++kb) {
        qk = mfma16x16x32(frag_s<D>(L.Q, o, ib * 16, kb * 32), frag_s<D>(L.K, o, jb * 16, kb * 32),
                          qk);
        dv = mfma16x16x32(frag_s<D>(L.DY, o, ib * 16, kb * 32), frag_s<D>(L.V, o, jb * 16, kb * 32),
                          dv);
      }
      const int col = jb * 16 + l16, r0 = ib * 16 + 4 * g4;
      const float lc = L.rc.li[col], nbc = L.rc.nb[col];
      f32x4 p, be, z;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool on = col < r0 + q;
        const float e = on ? fexp2(L.rc.lq[r0 + q] - lc) : 0.f;
        p[q] = qk[q] * e;
        be[q] = dv[q] * (e * nbc);
        z[q] = be[q] * qk[q];
      }
      put4<kCk>(L.PT, o64, jb * 16, ib * 16, pack4f(p));
      put4<kCk>(L.BT, o64, jb * 16, ib * 16, pack4f(be));
      f32x4 zr;
#pragma unroll
      for (int q = 0; q < 4; ++q) zr[q] = row16_sum(z[q]);
      if (l16 == 15) *reinterpret_cast<f32x4*>(&L.qk.qq[b][4 * g4]) = zr;
      const float t = sum_rows(z[0] + z[1] + z[2] + z[3]);
      if (g4 == 0) L.qk.kk[b][l16] = t;
    }
    __syncthreads();

    // ---- outputs, transposed (rows = columns of dq, dk, dv; columns =
    // tokens): token block tb = w % 4, column blocks cb = 2 (w / 4) + {0, 1}
    const int tb = wave & 3, cg = wave >> 2;
    const int ti = tb * 16 + l16;  // this lane's token
    const float eqi = L.rc.eq[ti], e2i = L.rc.e2[ti], nbi = L.rc.nb[ti];
    const __amdgpu_buffer_rsrc_t rdq = buffer_rsrc(static_cast<uint16_t*>(a.dq) + tok, cv * D * 2);
    const __amdgpu_buffer_rsrc_t rdk = buffer_rsrc(static_cast<uint16_t*>(a.dx) + tok, cv * D * 2);
    const __amdgpu_buffer_rsrc_t rdv = buffer_rsrc(static_cast<uint16_t*>(a.dg) + tok, cv * D * 2);
    float rr = 0.f, pp = 0.f, de = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      __builtin_amdgcn_sched_barrier(0);  // one column block's fragments live at a time
      const int cb = 2 * cg + h2;
      const uint32_t so = static_cast<uint32_t>((ti * D + cb * 16 + 4 * g4) * 2);
      // dq^T: (Be K)^T + W0'^T dy + e(lq) D_in^T dy (at D = 128 the W0'
      // fragments come from global memory: issued first, used last)
      bf16x8 wf[KS];
#pragma unroll
      for (int kr = 0; kr < KS; ++kr) {
        if constexpr (D == 64)
          wf[kr] = a.w0_t ? frag_s<D>(L.W, o, cb * 16, kr * 32) : frag_ts<D>(L.W, o, kr * 32, cb * 16);
        else
          wf[kr] = *reinterpret_cast<const bf16x8*>(wt + (cb * 16 + l16) * D + kr * 32 + 8 * g4);
      }
      f32x4 aq = zero4(), sq = zero4();
#pragma unroll
      for (int kr = 0; kr < KS; ++kr)
        sq = mfma16x16x32(frag_ts<D>(L.S, o, kr * 32, cb * 16), frag_s<D>(L.DY, o, tb * 16, kr * 32),
                          sq);
#pragma unroll
      for (int kj = 0; kj < 2; ++kj)
        aq = mfma16x16x32(frag_ts<D>(L.K, o, kj * 32, cb * 16),
                          frag_ts<kCk>(L.BT, o64, kj * 32, tb * 16), aq);
#pragma unroll
      for (int kr = 0; kr < KS; ++kr)
        aq = mfma16x16x32(wf[kr], frag_s<D>(L.DY, o, tb * 16, kr * 32), aq);
      const f32x4 qv = unpack4f(get4<D>(L.Q, o, tb * 16, cb * 16));  // q_t[k], k = cb 16 + 4 g4 ..
      rr += dot4f(qv, sq);
      store8(rdq, so, pack4f(aq + eqi * sq));
      __builtin_amdgcn_sched_barrier(0);
      // dk^T: (Be^T Q)^T - eta e(l_last - l) (A_out^T v)^T
      f32x4 ak = zero4(), sk = zero4();
#pragma unroll
      for (int ku = 0; ku < 2; ++ku)
        ak = mfma16x16x32(frag_ts<D>(L.Q, o, ku * 32, cb * 16),
                          frag_s<kCk>(L.BT, o64, tb * 16, ku * 32), ak);
#pragma unroll
      for (int kr = 0; kr < KS; ++kr)
        sk = mfma16x16x32(frag_ts<D>(L.A, o, kr * 32, cb * 16), frag_s<D>(L.V, o, tb * 16, kr * 32),
                          sk);
      store8(rdk, so, pack4f(ak + (nbi * e2i) * sk));
      __builtin_amdgcn_sched_barrier(0);
      // u^T: e(l_last - l) (A_out k)^T + (P^T dy)^T;  dv = -eta u
      f32x4 au = zero4(), su = zero4();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        su = mfma16x16x32(frag_s<D>(L.A, o, cb * 16, kk * 32), frag_s<D>(L.K, o, tb * 16, kk * 32),
                          su);
#pragma unroll
      for (int ku = 0; ku < 2; ++ku)
        au = mfma16x16x32(frag_ts<D>(L.DY, o, ku * 32, cb * 16),
                          frag_s<kCk>(L.PT, o64, tb * 16, ku * 32), au);
      const f32x4 u = au + e2i * su;
      const f32x4 vv = unpack4f(get4<D>(L.V, o, tb * 16, cb * 16));  // v_t[r], r = cb 16 + 4 g4 ..
      de -= dot4f(vv, u);
      pp += dot4f(vv, su);
      store8(rdv, so, pack4f(nbi * u));
    }
    // shares over this wave's 32 columns: sum over the four lane groups
    rr = sum_rows(rr);
    pp = sum_rows(pp);
    de = sum_rows(de);
    if (g4 == 0) {
      L.rr[cg][ti] = rr;
      L.pp[cg][ti] = pp;
      L.de[cg][ti] = de;
    }
    // ---- the adjoint entering this chunk, which leaves the one before it:
    // A <- e(l_last) A + sum_u e(lq_u) dy_u q_u^T (this wave's blocks;
    // operands swapped, so the product comes out in A's register layout)
    __builtin_amdgcn_sched_barrier(0);
    {
      const float gam = L.rc.gam;
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int b = NA * wave + i, rb = b / NB, cb = b % NB;
        f32x4 vi = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const f32x4 e0 = *reinterpret_cast<const f32x4*>(&L.rc.eq[kb * 32 + 8 * g4]);
          const f32x4 e1 = *reinterpret_cast<const f32x4*>(&L.rc.eq[kb * 32 + 8 * g4 + 4]);
          vi = mfma16x16x32(scale8(frag_ts<D>(L.Q, o, kb * 32, cb * 16), e0, e1),
                            frag_ts<D>(L.DY, o, kb * 32, rb * 16), vi);
        }
        A[i] = gam * A[i] + vi;
      }
    }
  }
  // dalpha and deta of the last chunk walked (the group's first)
  __syncthreads();
  if (wave == 0) {
    const int64_t t0 = static_cast<int64_t>(c_beg) * kCk;
    chunk_gate_grads<D>(L, a, bh, t0, static_cast<int>(std::min<int64_t>(kCk, T - t0)), lane);
  }
}

// ---- the gradients of every chunk at D = 128, eight waves ----
// The same walk and products as qkv_bwd_chunk, laid out for fewer LDS
// fragment reads: wave w forms the 32 x 32 block (columns 32 (w / 2) ..,
// tokens 32 (w % 2) ..) of every output, so each fragment it reads feeds two
// MFMAs, and keeps eight 16 x 16 blocks of the fp32 adjoint (row blocks
// 2 (w % 4) + {0, 1}, column blocks 4 (w / 4) + {0, .., 3}).  Two waves per
// SIMD with 256 registers each hold the next chunk's tiles (twelve 16-byte
// units per thread) while the current one is multiplied.
constexpr int kW8T = 512;  // threads

__global__ __launch_bounds__(kW8T) __attribute__((amdgpu_waves_per_eu(2, 2))) void qkv_bwd_chunk128(
    BwdArgs a, int n_grp) {
  constexpr int D = 128, NT = kW8T, NW = NT / 64, KS = D / 32;
  constexpr int NU = kCk * D / 8 / NT;  // 16-byte units of a token tile per thread (2)
  constexpr int NS = D * D / 8 / NT;    // of D_in (4)
  __shared__ GradLds<D> L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int n = a.n_chunks;
  const int64_t bh = blockIdx.x / n_grp;
  const int grp = static_cast<int>(blockIdx.x % n_grp);
  const int c_beg = grp * a.grp_chunks, c_end = std::min(n, c_beg + a.grp_chunks);
  const int h = static_cast<int>(bh % a.H);
  const int64_t T = a.T;
  const int64_t dd = static_cast<int64_t>(D) * D;
  // W0' stored [k][r]: the given one if transposed, else the copy
  const uint16_t* wt = static_cast<const uint16_t*>(a.w0_t ? a.W0 : a.W0t) + h * dd;
  // adjoint blocks of this wave: i -> row block 2 (w % 4) + i / 4, column block 4 (w / 4) + i % 4
  const int arb = 2 * (wave & 3), acb = 4 * (wave >> 2);
  // output blocks of this wave: column blocks 2 cg + {0, 1}, token blocks 2 tp + {0, 1}
  const int cg = wave >> 1, tp = wave & 1;
  // W0'^T fragments of this wave's two column blocks (the same for every chunk)
  bf16x8 wf[2][KS];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int kr = 0; kr < KS; ++kr)
      wf[h2][kr] = *reinterpret_cast<const bf16x8*>(wt + ((2 * cg + h2) * 16 + l16) * D + kr * 32 +
                                                    8 * g4);
  f32x4 A[8];
  {
    const float* pa = static_cast<const float*>(a.mf_lam) + (bh * n_grp + grp) * dd;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      A[i] = *reinterpret_cast<const f32x4*>(pa + ((arb + i / 4) * 16 + l16) * D +
                                             (acb + i % 4) * 16 + 4 * g4);
  }
  // the next chunk's tiles and gates, in registers
  u32x4 uq[NU], uk[NU], uv[NU], ud[NU], us[NS];
  float eta_l = 0.f, al_l = 1.f;
  const auto fetch = [&](int c) {
    const int64_t t0 = static_cast<int64_t>(c) * kCk;
    const int cv = static_cast<int>(std::min<int64_t>(kCk, T - t0));
    const int64_t tok = (bh * T + t0) * D;
    const auto rs = [&](const void* base) {
      return buffer_rsrc(static_cast<const uint16_t*>(base) + tok, cv * D * 2);
    };
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const uint32_t off = static_cast<uint32_t>((tid + NT * j) * 16);
      uq[j] = __builtin_amdgcn_raw_buffer_load_b128(rs(a.q), off, 0, 0);
      uk[j] = __builtin_amdgcn_raw_buffer_load_b128(rs(a.x), off, 0, 0);
      uv[j] = __builtin_amdgcn_raw_buffer_load_b128(rs(a.g), off, 0, 0);
      ud[j] = __builtin_amdgcn_raw_buffer_load_b128(rs(a.dy), off, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t rst =
        buffer_rsrc(static_cast<const uint16_t*>(a.states) + (bh * n + c) * dd, D * D * 2);
#pragma unroll
    for (int j = 0; j < NS; ++j)
      us[j] = __builtin_amdgcn_raw_buffer_load_b128(rst, static_cast<uint32_t>((tid + NT * j) * 16),
                                                    0, 0);
    const uint32_t go = static_cast<uint32_t>(lane * 4);
    eta_l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        buffer_rsrc(static_cast<const float*>(a.eta) + bh * T + t0, cv * 4), go, 0, 0));
    al_l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        buffer_rsrc(static_cast<const float*>(a.alpha) + bh * T + t0, cv * 4), go, 0, 0));
  };
  if (c_end > c_beg) fetch(c_end - 1);
  // the set-up loads done: the waits the compiler places inside the walk
  // then count only the walk's own loads and stores
  wait_vm<0>();

  LaneOff<D> o = lane_off<D>(lane);
  LaneOff<kCk> o64 = lane_off<kCk>(lane);
  for (int c = c_end - 1; c >= c_beg; --c) {
    // Most of the LDS lies beyond the 64 KB reach of the LDS instructions'
    // offset field; an empty asm on the lane offsets keeps the addresses
    // derived from them from being hoisted out of the loop.
    asm volatile("" : "+v"(o.b), "+v"(o.t0), "+v"(o.t1), "+v"(o.w));
    asm volatile("" : "+v"(o64.b), "+v"(o64.t0), "+v"(o64.t1), "+v"(o64.w));
    const int64_t t0 = static_cast<int64_t>(c) * kCk;
    const int cv = static_cast<int>(std::min<int64_t>(kCk, T - t0));
    const int64_t tok = (bh * T + t0) * D;
    __syncthreads();  // the previous chunk is done with every tile and share
    if (wave == 0) {
      // dalpha and deta of the previous chunk in walk order, then this
      // chunk's gates in their place
      // (also in the first step, with no valid tokens: the stores are then
      // dropped, and every step issues the same number of them)
      const int64_t tq = t0 + kCk;
      chunk_gate_grads<D, NW>(L, a, bh, tq,
                              c + 1 < c_end ? static_cast<int>(std::min<int64_t>(kCk, T - tq)) : 0,
                              lane);
      gates_v(eta_l, lane < cv ? al_l : 1.f, L.rc, lane);
    }
    // P^T and Be^T start at zero (only the causal parts are written)
    reinterpret_cast<u32x4*>(L.PT)[tid] = u32x4{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4*>(L.BT)[tid] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      put_unit<D>(L.Q, tid + NT * j, uq[j]);
      put_unit<D>(L.K, tid + NT * j, uk[j]);
      put_unit<D>(L.V, tid + NT * j, uv[j]);
      put_unit<D>(L.DY, tid + NT * j, ud[j]);
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) put_unit<D>(L.S, tid + NT * j, us[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) put4<D>(L.A, o, (arb + i / 4) * 16, (acb + i % 4) * 16, pack4f(A[i]));
    __syncthreads();

    // <A_out, D_in> over this wave's blocks (A_out in fp32)
    {
      float cp = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        cp += dot4f(A[i], unpack4f(get4<D>(L.S, o, (arb + i / 4) * 16, (acb + i % 4) * 16)));
      cp = wave_sum(cp);
      if (lane == 0) L.c0[wave] = cp;
    }
    // The next chunk's loads: issued here by the waves with one causal
    // block, after their second block by waves 0 and 1, so that they do not
    // hold up the tile writes above or the waves with the most work (the
    // loads have the rest of the step to arrive).
    if (wave >= 10 - NW && c > c_beg) fetch(c - 1);
    // ---- causal blocks (ten): Q K^T and DY V^T, decayed; P and Be
    // written transposed, the row / column sums of Be o (Q K^T)
    for (int b = wave; b < 10; b += NW) {
      __builtin_amdgcn_sched_barrier(0);
      const int ib = tri_i(b), jb = tri_j(b);
      f32x4 qk = zero4(), dv = zero4();
#pragma unroll
      for (int kb = 0; kb < KS; ++kb) {
        qk = mfma16x16x32(frag_s<D>(L.Q, o, ib * 16, kb * 32), frag_s<D>(L.K, o, jb * 16, kb * 32),
                          qk);
        dv = mfma16x16x32(frag_s<D>(L.DY, o, ib * 16, kb * 32), frag_s<D>(L.V, o, jb * 16, kb * 32),
                          dv);
      }
      const int col = jb * 16 + l16, r0 = ib * 16 + 4 * g4;
      const float lc = L.rc.li[col], nbc = L.rc.nb[col];
      f32x4 p, be, z;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool on = col < r0 + q;
        const float e = on ? fexp2(L.rc.lq[r0 + q] - lc) : 0.f;
        p[q] = qk[q] * e;
        be[q] = dv[q] * (e * nbc);
        z[q] = be[q] * qk[q];
      }
      put4<kCk>(L.PT, o64, jb * 16, ib * 16, pack4f(p));
      put4<kCk>(L.BT, o64, jb * 16, ib * 16, pack4f(be));
      f32x4 zr;
#pragma unroll
      for (int q = 0; q < 4; ++q) zr[q] = row16_sum(z[q]);
      if (l16 == 15) *reinterpret_cast<f32x4*>(&L.qk.qq[b][4 * g4]) = zr;
      const float t = sum_rows(z[0] + z[1] + z[2] + z[3]);
      if (g4 == 0) L.qk.kk[b][l16] = t;
    }
    if (wave < 10 - NW && c > c_beg) fetch(c - 1);
    __syncthreads();

    // ---- outputs, transposed (rows = columns of dq, dk, dv; columns =
    // tokens); tile [h2][hb]: column block 2 cg + h2, token block 2 tp + hb
    float eqi[2], sci[2], nbi[2], e2i[2];
    uint32_t so[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int ti = (2 * tp + hb) * 16 + l16;  // this lane's token
      eqi[hb] = L.rc.eq[ti];
      e2i[hb] = L.rc.e2[ti];
      nbi[hb] = L.rc.nb[ti];
      sci[hb] = nbi[hb] * e2i[hb];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        so[h2][hb] = static_cast<uint32_t>((ti * D + (2 * cg + h2) * 16 + 4 * g4) * 2);
    }
    const __amdgpu_buffer_rsrc_t rdq = buffer_rsrc(static_cast<uint16_t*>(a.dq) + tok, cv * D * 2);
    const __amdgpu_buffer_rsrc_t rdk = buffer_rsrc(static_cast<uint16_t*>(a.dx) + tok, cv * D * 2);
    const __amdgpu_buffer_rsrc_t rdv = buffer_rsrc(static_cast<uint16_t*>(a.dg) + tok, cv * D * 2);
    float rr[2] = {0.f, 0.f}, pp[2] = {0.f, 0.f}, de[2] = {0.f, 0.f};
    {
      // dq^T: (Be K)^T + W0'^T dy + e(lq) D_in^T dy
      f32x4 aq[2][2], sq[2][2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) aq[h2][hb] = sq[h2][hb] = zero4();
#pragma unroll
      for (int kj = 0; kj < 2; ++kj) {
        __builtin_amdgcn_sched_barrier(0);  // one K step of fragments live at a time
        bf16x8 kf[2], bf[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) kf[h2] = frag_ts<D>(L.K, o, kj * 32, (2 * cg + h2) * 16);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) bf[hb] = frag_ts<kCk>(L.BT, o64, kj * 32, (2 * tp + hb) * 16);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) aq[h2][hb] = mfma16x16x32(kf[h2], bf[hb], aq[h2][hb]);
      }
#pragma unroll
      for (int kr = 0; kr < KS; ++kr) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 sf[2], df[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) sf[h2] = frag_ts<D>(L.S, o, kr * 32, (2 * cg + h2) * 16);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) df[hb] = frag_s<D>(L.DY, o, (2 * tp + hb) * 16, kr * 32);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            sq[h2][hb] = mfma16x16x32(sf[h2], df[hb], sq[h2][hb]);
            aq[h2][hb] = mfma16x16x32(wf[h2][kr], df[hb], aq[h2][hb]);
          }
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          // q_t[k], k = (2 cg + h2) 16 + 4 g4 ..
          const f32x4 qv = unpack4f(get4<D>(L.Q, o, (2 * tp + hb) * 16, (2 * cg + h2) * 16));
          rr[hb] += dot4f(qv, sq[h2][hb]);
          store8(rdq, so[h2][hb], pack4f(aq[h2][hb] + eqi[hb] * sq[h2][hb]));
        }
    }
    {
      // dk^T: (Be^T Q)^T - eta e(l_last - l) (A_out^T v)^T
      f32x4 ak[2][2], sk[2][2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) ak[h2][hb] = sk[h2][hb] = zero4();
#pragma unroll
      for (int ku = 0; ku < 2; ++ku) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 qf[2], bf[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) qf[h2] = frag_ts<D>(L.Q, o, ku * 32, (2 * cg + h2) * 16);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) bf[hb] = frag_s<kCk>(L.BT, o64, (2 * tp + hb) * 16, ku * 32);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) ak[h2][hb] = mfma16x16x32(qf[h2], bf[hb], ak[h2][hb]);
      }
#pragma unroll
      for (int kr = 0; kr < KS; ++kr) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 af[2], vf[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) af[h2] = frag_ts<D>(L.A, o, kr * 32, (2 * cg + h2) * 16);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) vf[hb] = frag_s<D>(L.V, o, (2 * tp + hb) * 16, kr * 32);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) sk[h2][hb] = mfma16x16x32(af[h2], vf[hb], sk[h2][hb]);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          store8(rdk, so[h2][hb], pack4f(ak[h2][hb] + sci[hb] * sk[h2][hb]));
    }
    {
      // u^T: e(l_last - l) (A_out k)^T + (P^T dy)^T;  dv = -eta u
      f32x4 au[2][2], su[2][2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) au[h2][hb] = su[h2][hb] = zero4();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 af[2], kf[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) af[h2] = frag_s<D>(L.A, o, (2 * cg + h2) * 16, kk * 32);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) kf[hb] = frag_s<D>(L.K, o, (2 * tp + hb) * 16, kk * 32);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) su[h2][hb] = mfma16x16x32(af[h2], kf[hb], su[h2][hb]);
      }
#pragma unroll
      for (int ku = 0; ku < 2; ++ku) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 df[2], pf[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) df[h2] = frag_ts<D>(L.DY, o, ku * 32, (2 * cg + h2) * 16);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) pf[hb] = frag_s<kCk>(L.PT, o64, (2 * tp + hb) * 16, ku * 32);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) au[h2][hb] = mfma16x16x32(df[h2], pf[hb], au[h2][hb]);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const f32x4 u = au[h2][hb] + e2i[hb] * su[h2][hb];
          // v_t[r], r = (2 cg + h2) 16 + 4 g4 ..
          const f32x4 vv = unpack4f(get4<D>(L.V, o, (2 * tp + hb) * 16, (2 * cg + h2) * 16));
          de[hb] -= dot4f(vv, u);
          pp[hb] += dot4f(vv, su[h2][hb]);
          store8(rdv, so[h2][hb], pack4f(nbi[hb] * u));
        }
    }
    // shares over this wave's 32 columns: sum over the four lane groups
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float r1 = sum_rows(rr[hb]), p1 = sum_rows(pp[hb]), d1 = sum_rows(de[hb]);
      if (g4 == 0) {
        const int ti = (2 * tp + hb) * 16 + l16;
        L.rr[cg][ti] = r1;
        L.pp[cg][ti] = p1;
        L.de[cg][ti] = d1;
      }
    }
    // ---- the adjoint entering this chunk, which leaves the one before it:
    // A <- e(l_last) A + sum_u e(lq_u) dy_u q_u^T (operands swapped, so the
    // product comes out in A's register layout)
    __builtin_amdgcn_sched_barrier(0);
    {
      const float gam = L.rc.gam;
      f32x4 vi[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) vi[i] = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(&L.rc.eq[kb * 32 + 8 * g4]);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(&L.rc.eq[kb * 32 + 8 * g4 + 4]);
        bf16x8 qf[4], df[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) qf[j] = scale8(frag_ts<D>(L.Q, o, kb * 32, (acb + j) * 16), e0, e1);
#pragma unroll
        for (int j = 0; j < 2; ++j) df[j] = frag_ts<D>(L.DY, o, kb * 32, (arb + j) * 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) vi[i] = mfma16x16x32(qf[i % 4], df[i / 4], vi[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) A[i] = gam * A[i] + vi[i];
    }
  }
  // dalpha and deta of the last chunk walked (the group's first)
  __syncthreads();
  if (wave == 0 && c_end > c_beg) {
    const int64_t t0 = static_cast<int64_t>(c_beg) * kCk;
    chunk_gate_grads<D, NW>(L, a, bh, t0, static_cast<int>(std::min<int64_t>(kCk, T - t0)), lane);
  }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t s) {
  const int64_t BH = a.B * a.H;
  const int n = a.n_chunks;
  FwdArgs f;  // chunk-start states of the write-key scan (x = k, g = v)
  f.x = a.x; f.g = a.g; f.eta = a.eta; f.alpha = a.alpha; f.W0 = a.W0;
  f.y = nullptr; f.states = const_cast<void*>(a.states);
  f.B = a.B; f.H = a.H; f.T = a.T;
  f.d_in = D; f.d_out = D;
  f.chunk = kCk; f.n_chunks = n; f.ckpt_every = 1; f.n_ckpt = n;
  f.seg_chunks = n; f.n_seg = 1;
  hipError_t e = launch_mfma_fwd(f, s);
  if (e != hipSuccess) return e;
  if (D == 128 && !a.w0_t) {
    const int64_t total = a.H * static_cast<int64_t>(D) * D;
    hipLaunchKernelGGL(qkv_w0_transpose, dim3(static_cast<unsigned>((total + 255) / 256)),
                       dim3(256), 0, s, static_cast<const uint16_t*>(a.W0),
                       static_cast<uint16_t*>(const_cast<void*>(a.W0t)), D, total);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_grp = mfma_qkv_bwd_groups(n, a.grp_chunks);
  const dim3 grid(static_cast<unsigned>(BH * n_grp));
  hipLaunchKernelGGL(qkv_bwd_inc<D>, grid, dim3(4 * D), 0, s, a, n_grp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_eb = D * D / 4 / kCarryT;
  hipLaunchKernelGGL(qkv_grp_carry, dim3(static_cast<unsigned>(BH * n_eb)), dim3(kCarryT), 0, s,
                     static_cast<float*>(a.mf_lam), static_cast<const float*>(a.mf_gam), n_grp,
                     D * D, n_eb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D == 128)
    hipLaunchKernelGGL(qkv_bwd_chunk128, grid, dim3(kW8T), 0, s, a, n_grp);
  else
    hipLaunchKernelGGL(qkv_bwd_chunk<D>, grid, dim3(8 * D), 0, s, a, n_grp);
  return hipGetLastError();
}

}  // namespace

bool mfma_qkv_bwd_ok(int io, int dk, int dv) {
  return io == IO_BF16 && dk == dv && (dk == 64 || dk == 128);
}

int mfma_qkv_bwd_groups(int n_chunks, int grp_chunks) {
  return (n_chunks + grp_chunks - 1) / grp_chunks;
}

// Sixteen chunks per group, halved (down to four) while the gradient kernel
// would have fewer work-groups than the GPU runs at once (two per CU at
// d = 64, one at d = 128, 256 CUs).  Longer groups write fewer dW0' shares
// and carries and walk more chunks per work-group.
int mfma_qkv_bwd_group_chunks(int64_t BH, int n_chunks, int d) {
  const int64_t want = d == 64 ? 512 : 256;
  int g = 16;
  while (g > 4 && BH * mfma_qkv_bwd_groups(n_chunks, g) < want) g /= 2;
  return g;
}

// a: x = k (write key), g = v, q the read vector; dx <- dk, dg <- dv, dq;
// in the workspace: states (bf16 [BH][n][D][D]), mf_lam (fp32
// [BH][groups][D][D]), mf_gam (fp32 [BH][groups]), part_dW0 (fp32
// [groups][BH][D][D]) and, at D = 128 with W0' not given transposed, W0t
// (bf16 [H][D][D]); deta_out / dalpha_out.
hipError_t launch_mfma_qkv_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.d_in != a.d_out || (a.d_in != 64 && a.d_in != 128)) return hipErrorInvalidValue;
  if (a.d_in == 128 && !a.w0_t && !a.W0t) return hipErrorInvalidValue;
  if (a.B * a.H * a.n_chunks == 0) return hipSuccess;
  return a.d_in == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace gls
