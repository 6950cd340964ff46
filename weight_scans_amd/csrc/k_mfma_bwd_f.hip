// k_mfma_bwd_f.hip -- fused matrix-core reverse scan for bf16 io,
// d_in = d_out = 64 (gfx950, v_mfma_f32_16x16x32_bf16).
//
// One work-group walks the chunks of one (segment, sequence-head) from right
// to left carrying the adjoint Lam = dL/dD (the exact adjoint of the forward
// scan, GradLev abstract, omanscience.com) in fp32 registers, and emits every
// gradient of the chunk it passes.  With P, Be, M = Be + Be^T and the Be dots
// as in bwd_fused.hpp:
//   u_i   = e(l_last - l_i) Lam_out x_i + sum_{u>i} P_ui dy_u
//   dg_i  = -eta_i u_i,  deta_i = -g_i . u_i
//   dx_i  = W0^T dy_i + e(lq_i) D_in^T dy_i + (M X)_i - eta_i e(l_last - l_i) Lam_out^T g_i
//   dW0  += sum_u dy_u x_u^T
//   Lam_in = e(l_last) Lam_out + sum_u e(lq_u) dy_u x_u^T
// and dalpha from pp_i = g_i . (Lam_out x_i), rr_i = x_i . (D_in^T dy_i), the
// Be dots and <Lam_out, D_in>.  D_in is the chunk-start state the forward
// kernel stores.
//
// Sixteen waves, one of each role on every SIMD (role = wave / 4, quadrant =
// wave % 4; 32 x 32 output quadrants, so every fragment read serves two
// MFMAs):
//   0  dx^T quadrant (columns k, tokens i), its rr share; causal block q of
//      the next chunk;
//   1  Lam^T and dW0^T quadrant (columns k, rows r) in fp32 registers, the
//      <Lam_out, D_in> share, the bf16 copy of the next Lam_out; causal
//      block 4 + q of the next chunk;
//   2  u^T quadrant (rows r, tokens i): dg, the deta and pp shares;
//   3  loaders: tile q (x, g, dy, D_in) of the chunk two ahead and a gate
//      row; waves 12-13 causal blocks 8-9, wave 14 the gates two chunks
//      ahead, wave 15 dalpha and deta of the previous chunk.
// Chunk tiles come by direct buffer loads into a ring of three slots: while
// the chunk of step j is finished and the causal blocks of chunk j + 1 are
// formed, chunk j + 2 is in flight.  One barrier per chunk.  Each role walks
// in its own copy of the loop (registers are allocated per role); only the
// loaders issue loads and wait for them, and each of them issues the same
// loads and stores every step, so that wait is a constant.
#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "bwd_fused.hpp"

namespace gls {
namespace {

constexpr int kD = 64;          // d_in = d_out
constexpr int kC = 64;          // tokens per chunk
constexpr int kNW = 16;         // waves per work-group
constexpr int kNT = 64 * kNW;   // threads
constexpr int kGateWave = 14;   // derives the gates two chunks ahead
constexpr int kAlphaWave = 15;  // dalpha and deta one chunk behind
constexpr int kLoaderStores = 2;  // stores per loader wave (role 3) per step

struct alignas(16) SlotF {
  __bf16 X[kC * kD];    // x, swizzled [token][k]
  __bf16 G[kC * kD];    // g, swizzled [token][r]
  __bf16 DY[kC * kD];   // dy, swizzled [token][r]
  __bf16 S[kD * kD];    // D_in, swizzled [r][k]
  float q[2][kC];       // eta, alpha of the chunk after (in walk order)
};

struct alignas(16) PartF {  // per-token shares of one chunk
  float pp[2][kC], rr[2][kC], de[2][kC];
  float c0[4];
};

// Per-lane byte offsets of a [64][64] bf16 tile load into a swizzled LDS
// tile: instruction wi (of 8) fills 16-byte slots wi * 64 + lane, and reads
// global bytes wi * 1024 + off[wi & 1] (the swizzle of a row depends on the
// row's low three bits, from the lane, and bit 3, from wi).
struct DmaOffF {
  uint32_t e, o;
};
__device__ __forceinline__ DmaOffF dma_off_f(int lane) {
  DmaOffF d;
  const int rl = lane >> 3, u = lane & 7;
  d.e = static_cast<uint32_t>(rl * kD * 2 + 16 * (u ^ swz<kD>(rl)));
  d.o = static_cast<uint32_t>(rl * kD * 2 + 16 * (u ^ swz<kD>(8 + rl)));
  return d;
}

// Loader wave ld (0..3) of a chunk: the whole tile ld (x, g, dy, D_in) of
// chunk k (negative: zero fill) in eight instructions, then the eta (even
// ld) or alpha (odd ld) row of chunk kq.
__device__ __forceinline__ void issue_f(SlotF& sl, const DmaOffF& od, uint32_t oq,
                                        const uint16_t* x, const uint16_t* g, const uint16_t* dy,
                                        const uint16_t* st, const float* eta, const float* alpha,
                                        int64_t T, int k, int kq, int ld) {
  const bool in = k >= 0;
  const int64_t t0 = in ? static_cast<int64_t>(k) * kC : 0;
  const int cv = in ? static_cast<int>(std::min<int64_t>(kC, T - t0)) : 0;
  const int64_t s0 = (in ? static_cast<int64_t>(k) : 0) * kD * kD;
  const __amdgpu_buffer_rsrc_t r =
      ld == 3 ? buffer_rsrc(st + s0, in ? kD * kD * 2 : 0)
              : buffer_rsrc((ld == 0 ? x : ld == 1 ? g : dy) + t0 * kD, cv * kD * 2);
  char* base = reinterpret_cast<char*>(&sl) +
               (ld == 0 ? offsetof(SlotF, X) : ld == 1 ? offsetof(SlotF, G)
                : ld == 2 ? offsetof(SlotF, DY) : offsetof(SlotF, S));
#pragma unroll
  for (int wi = 0; wi < 8; ++wi)
    dma16(r, (wi & 1 ? od.o : od.e) + wi * 1024, base + wi * 1024);
  const bool inq = kq >= 0;
  const int64_t tq = inq ? static_cast<int64_t>(kq) * kC : 0;
  const int cq = inq ? static_cast<int>(std::min<int64_t>(kC, T - tq)) : 0;
  dma4(buffer_rsrc(((ld & 1) == 0 ? eta : alpha) + tq, cq * 4), oq, sl.q[ld & 1]);
}

template <bool F32>
__global__ __launch_bounds__(kNT) void bwd_f64(BwdArgs a) {
  constexpr int OE = F32 ? 4 : 2;  // bytes per element of dx, dg
  __shared__ SlotF ring0, ring1, ring2;
  __shared__ __bf16 PT_s[2][kC * kC];  // P^T by chunk parity (W0 staging at the start)
  __shared__ __bf16 M_s[2][kC * kC + kMPad];  // Be + Be^T by chunk parity (+ pad)
  __shared__ __bf16 L_s[2][kD * kD];   // Lam_out (bf16, [r][k]) by chunk parity
  __shared__ RecF rec[4];
  __shared__ PartF part[2];
  __shared__ QkF qk[3];
  SlotF* const rs[3] = {&ring0, &ring1, &ring2};

  const int64_t BH = a.B * a.H, T = a.T;
  const int n = a.n_chunks;
  const int64_t bh = blockIdx.x % BH;
  const int seg = static_cast<int>(blockIdx.x / BH);
  const int c_beg = seg * a.seg_chunks;
  const int c_end = std::min(n, c_beg + a.seg_chunks);
  const int nloc = c_end - c_beg;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave >> 2, qd = wave & 3;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int hq = qd >> 1, lq2 = qd & 1;  // quadrant: high / low half
  const int h = static_cast<int>(bh % a.H);
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * kD;
  const uint16_t* g = static_cast<const uint16_t*>(a.g) + bh * T * kD;
  const uint16_t* dy = static_cast<const uint16_t*>(a.dy) + bh * T * kD;
  const float* eta = static_cast<const float*>(a.eta) + bh * T;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * kD * kD;
  const uint16_t* st = static_cast<const uint16_t*>(a.states) + bh * static_cast<int64_t>(n) * kD * kD;
  char* dx = static_cast<char*>(a.dx) + bh * T * kD * OE;
  char* dg = static_cast<char*>(a.dg) + bh * T * kD * OE;
  float* dal = static_cast<float*>(a.dalpha_out) + bh * T;
  float* det = static_cast<float*>(a.deta_out) + bh * T;

  const LaneOff<kD> o_in = lane_off<kD>(lane);
  const LaneOff<kD>& o = o_in;
  const DmaOffF od = dma_off_f(lane);
  const uint32_t oq = static_cast<uint32_t>(lane * 4);
  const __amdgpu_buffer_rsrc_t r_none = buffer_rsrc(a.x, 0);

  // chunk visited v-th (-1: none)
  const auto chunk_at = [&](int v) { return (v >= 0 && v < nloc) ? c_end - 1 - v : -1; };
  const auto cv_of = [&](int c) {
    return c < 0 ? 0 : static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };

  // ---- set-up: loads of the first chunk (into slot 1, with the gate rows of
  // the second) and of its own gate rows (slot 0), W0, the entering adjoint
  if (role == 3) {
    issue_f(*rs[1], od, oq, x, g, dy, st, eta, alpha, T, chunk_at(0), chunk_at(1), qd);
    const int c0 = chunk_at(0);
    dma4(buffer_rsrc(((qd & 1) == 0 ? eta : alpha) + (c0 >= 0 ? static_cast<int64_t>(c0) * kC : 0),
                     cv_of(c0) * 4),
         oq, rs[0]->q[qd & 1]);
  }
  // W0 (bf16 [r][k]) staged in PT_s[1]; dx waves keep W0^T fragments
  for (int idx = tid; idx < kD * kD / 8; idx += kNT) {
    const int r = idx >> 3, cc = 8 * (idx & 7);
    *reinterpret_cast<uint4*>(&PT_s[1][sidx<kD>(r, cc)]) =
        *reinterpret_cast<const uint4*>(W0 + static_cast<int64_t>(r) * kD + cc);
  }
  // Registers a wave keeps for the whole walk, by role (one array, so that
  // the roles share them):
  //   role 0: pr[2a + kk] = W0^T fragment (column block 2hq + a, K block kk of r)
  //   role 1: pr[2a + b] = Lam^T block, pr[4 + 2a + b] = dW0^T block
  //           (k block 2hq + a, r block 2lq2 + b; lane: k = 4 g4 + q, r = l16)
  f32x4 pr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) pr[e] = zero4();
  if (role == 1 && a.seg_lam) {
    // adjoint entering from the right: given (the adjoint-only pass's
    // segment ending where this one ends), or composed here from the
    // adjoint-only pass's segments to the right, nearest last:
    // Lam <- 2^(lg_s) Lam + L_s
    const int ln = a.lam_n ? a.lam_n : a.n_seg, end = (seg + 1) * a.lam_r;
    const int s_lo = a.seg_lg_in ? end : end - 1;
    const int s_hi = a.seg_lg_in ? ln - 1 : end - 1;
    // four segments at a time: their loads (from clamped, valid addresses)
    // are all issued before the first is folded in
    for (int s0 = s_hi; s0 >= s_lo; s0 -= 4) {
      f32x4 t[4][4];
      float gsv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s2 = s0 - j >= s_lo ? s0 - j : s_lo;
        const float* sl = a.seg_lam + (bh * ln + s2) * kD * kD;
        gsv[j] = a.seg_lg_in ? a.seg_lg_in[bh * ln + s2] : 0.f;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb)
            t[j][2 * aa + bb] = *reinterpret_cast<const f32x4*>(
                sl + ((2 * lq2 + bb) * 16 + l16) * kD + (2 * hq + aa) * 16 + 4 * g4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool use = s0 - j >= s_lo;
        const float gs = a.seg_lg_in ? fexp2(gsv[j]) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[e] = use ? pr[e] * gs + t[j][e] : pr[e];
      }
    }
  }
  wait_vm<0>();
  __syncthreads();
  if (role == 0) {
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        pr[2 * aa + kk] =
            __builtin_bit_cast(f32x4, frag_ts<kD>(PT_s[1], o, kk * 32, (2 * hq + aa) * 16));
  }
  __syncthreads();
  for (int idx = tid; idx < 2 * kC * kC / 8; idx += kNT)
    reinterpret_cast<uint4*>(&PT_s[0][0])[idx] = make_uint4(0, 0, 0, 0);
  if (role == 1) {
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
        put4<kD>(L_s[0], o, (2 * lq2 + bb) * 16, (2 * hq + aa) * 16, pack4f(pr[2 * aa + bb]));
  }
  if (wave == kGateWave) gates_f(rs[0]->q[0], rs[0]->q[1], rec[0], cv_of(chunk_at(0)), lane);

  // per-lane offsets of the dx / dg stores: token 16(2 lq2 + b) + l16,
  // columns 16(2 hq + a) + 4 g4 ..
  const uint32_t o8_in = static_cast<uint32_t>((2 * lq2 * 16 + l16) * kD * 2 + (2 * hq * 16 + 4 * g4) * 2);

  // step j: chunk v = j finished (slot K), causal blocks of v = j + 1, loads
  // of v = j + 2; K = (j + 1) % 3
  const auto step = [&](auto RC, auto KC, int j) {
    constexpr int R = decltype(RC)::value;
    constexpr int K = decltype(KC)::value;
    SlotF& cur = *rs[K];
    SlotF& nx = *rs[(K + 1) % 3];
    SlotF& dst = *rs[(K + 2) % 3];
    // loader waves: chunk j + 1 loaded (after its loads come only the
    // previous step's stores); then every wave: the slot about to be refilled
    // is no longer read
    if constexpr (R == 3) wait_vm<kLoaderStores>();
    lds_barrier();
    // per-lane offsets passed through an empty asm: the addresses derived
    // from them are formed inside the step instead of being kept live
    // across the whole walk for every slot and role
    LaneOff<kD> o = o_in;
    uint32_t o8 = o8_in;
    asm volatile("" : "+v"(o.b), "+v"(o.t0), "+v"(o.t1), "+v"(o.w), "+v"(o8));
    if constexpr (R == 3)
      issue_f(dst, od, oq, x, g, dy, st, eta, alpha, T, chunk_at(j + 2), chunk_at(j + 3), qd);
    // causal block b of chunk j + 1 (blocks 0-3: dx waves, 4-7: adjoint
    // waves, 8-9: loader waves 12 and 13)
    const auto causal_next = [&](int b) {
      if (chunk_at(j + 1) >= 0)
        causal_f<kD>(nx.X, nx.G, nx.DY, rec[(j + 1) & 3], PT_s[(j + 1) & 1], M_s[(j + 1) & 1],
                     qk[(K + 1) % 3], o, o, b, lane);
    };

    const int c = chunk_at(j);
    const int64_t t0 = c >= 0 ? static_cast<int64_t>(c) * kC : 0;
    const int cv = cv_of(c);
    out4_t<F32> s8[2][2];
    float s4a = 0.f, s4b = 0.f;
    __amdgpu_buffer_rsrc_t ra = r_none, rb = r_none;

    if constexpr (R == 0) {
      if (c >= 0) {
        // dx^T[k][i]: k block 2hq + a, token block 2lq2 + b
        const RecF& rc = rec[j & 3];
        const __bf16* L = L_s[j & 1];
        const __bf16* M = M_s[j & 1];
        float sc[2], eqv[2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int i = (2 * lq2 + bb) * 16 + l16;
          sc[bb] = rc.nb[i] * rc.e2[i];
          eqv[bb] = rc.eq[i];
        }
        f32x4 acc[2][2];
        {
          // -eta_i e(l_last - l_i) Lam_out^T g_i
          f32x4 t[2][2];
#pragma unroll
          for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) t[aa][bb] = zero4();
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            __builtin_amdgcn_sched_barrier(0);  // one K step of fragments live at a time
            bf16x8 lf[2], gf[2];
#pragma unroll
            for (int aa = 0; aa < 2; ++aa) lf[aa] = frag_ts<kD>(L, o, kk * 32, (2 * hq + aa) * 16);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) gf[bb] = frag_s<kD>(cur.G, o, (2 * lq2 + bb) * 16, kk * 32);
#pragma unroll
            for (int aa = 0; aa < 2; ++aa)
#pragma unroll
              for (int bb = 0; bb < 2; ++bb) t[aa][bb] = mfma16x16x32(lf[aa], gf[bb], t[aa][bb]);
          }
#pragma unroll
          for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) acc[aa][bb] = t[aa][bb] * sc[bb];
        }
        {
          // e(lq_i) D_in^T dy_i, and rr_i = x_i . (D_in^T dy_i) over this k half
          f32x4 t[2][2];
#pragma unroll
          for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) t[aa][bb] = zero4();
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            __builtin_amdgcn_sched_barrier(0);  // one K step of fragments live at a time
            bf16x8 sf[2], df[2];
#pragma unroll
            for (int aa = 0; aa < 2; ++aa) sf[aa] = frag_ts<kD>(cur.S, o, kk * 32, (2 * hq + aa) * 16);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) df[bb] = frag_s<kD>(cur.DY, o, (2 * lq2 + bb) * 16, kk * 32);
#pragma unroll
            for (int aa = 0; aa < 2; ++aa)
#pragma unroll
              for (int bb = 0; bb < 2; ++bb) t[aa][bb] = mfma16x16x32(sf[aa], df[bb], t[aa][bb]);
          }
          PartF& pw = part[j & 1];
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            float rp = 0.f;
#pragma unroll
            for (int aa = 0; aa < 2; ++aa) {
              const f32x4 xv = unpack4f(get4<kD>(cur.X, o, (2 * lq2 + bb) * 16, (2 * hq + aa) * 16));
              rp += dot4f(xv, t[aa][bb]);
              acc[aa][bb] += t[aa][bb] * eqv[bb];
            }
            rp = sum_rows(rp);
            if (g4 == 0) pw.rr[hq][(2 * lq2 + bb) * 16 + l16] = rp;
          }
        }
        // W0^T dy_i + (M X)_i
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          __builtin_amdgcn_sched_barrier(0);  // one K step of fragments live at a time
          bf16x8 df[2], mf[2], xf[2];
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            df[bb] = frag_s<kD>(cur.DY, o, (2 * lq2 + bb) * 16, kk * 32);
            mf[bb] = frag_s<kC>(M, o, (2 * lq2 + bb) * 16, kk * 32);
          }
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) xf[aa] = frag_ts<kD>(cur.X, o, kk * 32, (2 * hq + aa) * 16);
#pragma unroll
          for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
              acc[aa][bb] = mfma16x16x32(__builtin_bit_cast(bf16x8, pr[2 * aa + kk]), df[bb],
                                         acc[aa][bb]);
              acc[aa][bb] = mfma16x16x32(xf[aa], mf[bb], acc[aa][bb]);
            }
        }
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) s8[aa][bb] = pack_out<F32>(acc[aa][bb]);
        const __amdgpu_buffer_rsrc_t r8 = buffer_rsrc(dx + t0 * kD * OE, cv * kD * OE);
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb)
            store_out<F32>(r8, o8 + aa * 32 + bb * 16 * kD * 2, s8[aa][bb]);
      }
      causal_next(qd);
    } else if constexpr (R == 1) {
      if (c >= 0) {
        // <Lam_out, D_in> share, then Lam^T <- Gamma Lam^T + X^T (e(lq) dy),
        // dW0^T += X^T dy; k block 2hq + a, r block 2lq2 + b
        const RecF& rc = rec[j & 3];
        float c0p = 0.f;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb)
            c0p += dot4f(unpack4f(get4<kD>(cur.S, o, (2 * lq2 + bb) * 16, (2 * hq + aa) * 16)),
                         pr[2 * aa + bb]);
        c0p = wave_sum(c0p);
        if (lane == 0) part[j & 1].c0[qd] = c0p;
        const float gam = rc.gam;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) pr[2 * aa + bb] = pr[2 * aa + bb] * gam;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          __builtin_amdgcn_sched_barrier(0);  // one K step of fragments live at a time
          bf16x8 xf[2], df[2], de[2];
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) xf[aa] = frag_ts<kD>(cur.X, o, kk * 32, (2 * hq + aa) * 16);
          const f32x4 e0 = *reinterpret_cast<const f32x4*>(&rc.eq[kk * 32 + 8 * g4]);
          const f32x4 e1 = *reinterpret_cast<const f32x4*>(&rc.eq[kk * 32 + 8 * g4 + 4]);
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            df[bb] = frag_ts<kD>(cur.DY, o, kk * 32, (2 * lq2 + bb) * 16);
            de[bb] = scale8(df[bb], e0, e1);
          }
#pragma unroll
          for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
              pr[4 + 2 * aa + bb] = mfma16x16x32(xf[aa], df[bb], pr[4 + 2 * aa + bb]);
              pr[2 * aa + bb] = mfma16x16x32(xf[aa], de[bb], pr[2 * aa + bb]);
            }
        }
        __bf16* Ln = L_s[(j + 1) & 1];
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb)
            put4<kD>(Ln, o, (2 * lq2 + bb) * 16, (2 * hq + aa) * 16, pack4f(pr[2 * aa + bb]));
      }
      causal_next(4 + qd);
    } else if constexpr (R == 2) {
      if (c >= 0) {
        // u^T[r][i]: r block 2hq + a, token block 2lq2 + b
        const RecF& rc = rec[j & 3];
        const __bf16* L = L_s[j & 1];
        const __bf16* PT = PT_s[j & 1];
        f32x4 ain[2][2], apd[2][2];
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            ain[aa][bb] = zero4();
            apd[aa][bb] = zero4();
          }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          __builtin_amdgcn_sched_barrier(0);  // one K step of fragments live at a time
          bf16x8 lf[2], xf[2];
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) lf[aa] = frag_s<kD>(L, o, (2 * hq + aa) * 16, kk * 32);
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) xf[bb] = frag_s<kD>(cur.X, o, (2 * lq2 + bb) * 16, kk * 32);
#pragma unroll
          for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) ain[aa][bb] = mfma16x16x32(lf[aa], xf[bb], ain[aa][bb]);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          __builtin_amdgcn_sched_barrier(0);  // one K step of fragments live at a time
          bf16x8 tf[2], pf[2];
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) tf[aa] = frag_ts<kD>(cur.DY, o, kk * 32, (2 * hq + aa) * 16);
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) pf[bb] = frag_s<kC>(PT, o, (2 * lq2 + bb) * 16, kk * 32);
#pragma unroll
          for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) apd[aa][bb] = mfma16x16x32(tf[aa], pf[bb], apd[aa][bb]);
        }
        PartF& pw = part[j & 1];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int i = (2 * lq2 + bb) * 16 + l16;
          const float e2i = rc.e2[i], nbi = rc.nb[i];
          float dp = 0.f, pp = 0.f;
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) {
            const f32x4 u = ain[aa][bb] * e2i + apd[aa][bb];
            const f32x4 gv = unpack4f(get4<kD>(cur.G, o, (2 * lq2 + bb) * 16, (2 * hq + aa) * 16));
            dp += dot4f(gv, u);
            pp += dot4f(gv, ain[aa][bb]);
            s8[aa][bb] = pack_out<F32>(u * nbi);
          }
          dp = sum_rows(dp);
          pp = sum_rows(pp);
          if (g4 == 0) {
            pw.de[hq][i] = -dp;
            pw.pp[hq][i] = pp;
          }
        }
        const __amdgpu_buffer_rsrc_t r8 = buffer_rsrc(dg + t0 * kD * OE, cv * kD * OE);
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb)
            store_out<F32>(r8, o8 + aa * 32 + bb * 16 * kD * 2, s8[aa][bb]);
      }
    } else {
      if (qd < 2) causal_next(8 + qd);
      if (wave == kGateWave) {
        const int c2 = chunk_at(j + 2);
        if (c2 >= 0) gates_f(nx.q[0], nx.q[1], rec[(j + 2) & 3], cv_of(c2), lane);
      }
      if (wave == kAlphaWave) {
        const int cp = chunk_at(j - 1);
        if (cp >= 0) {
          // dalpha and deta of the chunk finished one step ago
          const RecF& rp = rec[(j - 1) & 3];
          const PartF& pr = part[(j - 1) & 1];
          const QkF& qr = qk[(K + 2) % 3];
          const int ir = kC - 1 - lane;
          const float c0 = (pr.c0[0] + pr.c0[1]) + (pr.c0[2] + pr.c0[3]);
          s4a = dalpha_f(rp, qr, pr.pp[0][lane] + pr.pp[1][lane], pr.rr[0][ir] + pr.rr[1][ir], c0,
                         lane);
          s4b = pr.de[0][lane] + pr.de[1][lane];
          const int64_t tp = static_cast<int64_t>(cp) * kC;
          ra = buffer_rsrc(dal + tp, cv_of(cp) * 4);
          rb = buffer_rsrc(det + tp, cv_of(cp) * 4);
        }
      }
      // the same two stores in every loader wave (zero-byte buffers drop
      // them), so that its wait at the top of a step is a constant
      store4(ra, oq, s4a);
      store4(rb, oq, s4b);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // each role walks in its own copy of the loop (same barriers), so
  // registers are allocated per role
  const auto walk = [&](auto RC) {
    for (int j = -1; j <= nloc; j += 3) {
      step(RC, I0{}, j);
      if (j + 1 > nloc) break;
      step(RC, I1{}, j + 1);
      if (j + 2 > nloc) break;
      step(RC, I2{}, j + 2);
    }
  };
  // (the loader role first: with this order the compiler's wait analysis
  // keeps the loaders' loads in flight out of the other roles' loops)
  if (role == 3)
    walk(I3{});
  else if (role == 2)
    walk(I2{});
  else if (role == 1)
    walk(I1{});
  else
    walk(I0{});
  wait_vm<0>();  // no load into LDS may outlive the work-group
  if (role == 1) {
    // dW0 partial of this (segment, sequence-head): dW0[r][k], fp32
    float* pw = static_cast<float*>(a.part_dW0) + (static_cast<int64_t>(seg) * BH + bh) * kD * kD;
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
        *reinterpret_cast<f32x4*>(pw + ((2 * lq2 + bb) * 16 + l16) * kD + (2 * hq + aa) * 16 +
                                  4 * g4) = pr[4 + 2 * aa + bb];
  }
}

}  // namespace

hipError_t launch_mfma_bwd_f64(const BwdArgs& a, hipStream_t s) {
  const int64_t groups = a.B * a.H * a.n_seg;
  if (groups == 0) return hipSuccess;
  if (a.out_f32)
    hipLaunchKernelGGL(bwd_f64<true>, dim3(static_cast<unsigned>(groups)), dim3(kNT), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_f64<false>, dim3(static_cast<unsigned>(groups)), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace gls
