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
// i.e. the discounted sum of rank-one updates of "Parallelize the Training,
// Keep the Learning Serial" (cognaptus.com, section "Once the gradient signals
// are known, the weight trajectory becomes parallelizable") composed as an
// affine scan across chunks.  Every exponent is <= 0.
//
// Pipeline: chunk tiles are copied HBM -> LDS by direct loads
// (global_load_lds) into a ring of kRing slots, kRing - 2 chunks ahead of the
// chunk being finished, so the serial chain over chunks does not wait for
// memory latency.  The scores of chunk c + 1 are formed while chunk c is
// finished, which leaves one work-group barrier per chunk.  All LDS tiles are
// XOR-swizzled (mfma.hpp) so that fragment reads are free of bank conflicts.
//
// `states` (optional) receives D_in of every chunk in bf16:
// [B*H][n_chunks][D (row r)][D (col c)] -- read by the matrix-core backward.
#include <algorithm>
#include <type_traits>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kC = 64;     // tokens per chunk
constexpr int kTN = 32;    // rows of the adaptation per work-group
constexpr int kNT = 256;   // threads (4 waves)
constexpr int kRing = 5;   // chunk slots: 2 in use, 3 in flight

template <int D>
struct alignas(16) Slot {
  __bf16 X[kC * D];        // x of the chunk, swizzled [token][D]
  __bf16 G[kC * kTN];      // g of the row tile, swizzled [token][kTN]
  float q[4][kC];          // raw gates: eta, alpha (rows 2, 3: zero fill)
  float lq[kC], li[kC], nb[kC], bk[kC];      // l_{i-1}, l_i, -eta_i, e(l_last - l_i)(-eta_i)
};

// Vector-memory instructions one wave issues per chunk load: D/32 for x, one
// for g, one for the gates.
template <int D>
constexpr int kLoadOps = D / 32 + 2;

// Per-lane byte offsets of the chunk loads (loop invariant).
template <int D>
struct DmaOff {
  uint32_t x[D / 32];  // x rows: wave instruction wave + 4 s covers 16-byte units 64 (wave + 4 s) ..
  uint32_t g;          // g tile: units 64 wave ..
  uint32_t q;          // gates: lane * 4
};
template <int D>
__device__ __forceinline__ DmaOff<D> dma_off(int wave, int lane) {
  constexpr int U = D / 8;  // 16-byte units per row of x
  DmaOff<D> o;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const int p = (wave + 4 * s) * 64 + lane;
    const int row = p / U, kl = (p % U) ^ swz<D>(row);
    o.x[s] = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  }
  const int p = wave * 64 + lane;
  const int row = p >> 2, kl = (p & 3) ^ swz<kTN>(row);
  o.g = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  o.q = static_cast<uint32_t>(lane * 4);
  return o;
}

// Queue the loads of chunk k into `sl`.  Rows past the sequence end, and
// chunks past the last one, are zero-filled by the buffer bounds (every wave
// always issues the same number of loads).
template <int D>
__device__ __forceinline__ void issue_chunk(Slot<D>& sl, const DmaOff<D>& o, const uint16_t* x,
                                            const uint16_t* g, const float* eta,
                                            const float* alpha, int64_t T, int k, int n_chunks,
                                            int r0, int wave) {
  const bool in = k < n_chunks;
  const int64_t t0 = in ? static_cast<int64_t>(k) * kC : 0;
  const int cv = in ? static_cast<int>(std::min<int64_t>(kC, T - t0)) : 0;
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + t0 * D, cv * D * 2);
#pragma unroll
  for (int s = 0; s < D / 32; ++s) dma16(rx, o.x[s], sl.X + (wave + 4 * s) * 512);
  const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g + t0 * D + r0, cv > 0 ? (cv * D - r0) * 2 : 0);
  dma16(rg, o.g, sl.G + wave * 512);
  const __amdgpu_buffer_rsrc_t rq = buffer_rsrc((wave == 0 ? eta : alpha) + t0, wave < 2 ? cv * 4 : 0);
  dma4(rq, o.q, sl.q[wave]);
}

// Gates of a chunk, lane = token (every wave computes them and writes the
// same values).  Returns Gamma = e(l_last).
template <int D>
__device__ __forceinline__ float prep_gates(Slot<D>& sl, int cv, int lane) {
  const float et = lane < cv ? sl.q[0][lane] : 0.f;
  const ChunkGates gt = chunk_gates(lane < cv ? sl.q[1][lane] : 1.f, lane);
  sl.lq[lane] = gt.lq;
  sl.li[lane] = gt.l;
  sl.nb[lane] = -et;
  sl.bk[lane] = -et * fexp2(gt.llast - gt.l);
  return fexp2(gt.llast);
}

// Causal decayed scores of a chunk, written transposed: AT[j][i] = A_ij.
// Blocks above the diagonal are never written (they stay zero).
template <int D>
__device__ __forceinline__ void scores(const Slot<D>& sl, __bf16* AT, const LaneOff<D>& oX,
                                       const LaneOff<kC>& oA, int wave, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int b = wave + 4 * s;
    if (b < 10) {
      const int ib = tri_i(b), jb = tri_j(b);
      f32x4 xx = zero4();
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
        xx = mfma16x16x32(frag_s<D>(sl.X, oX, ib * 16, kb * 32),
                          frag_s<D>(sl.X, oX, jb * 16, kb * 32), xx);
      const int j = jb * 16 + l16, i0 = ib * 16 + 4 * g4;
      const float lj = sl.li[j], nj = sl.nb[j];
      const f32x4 lqi = *reinterpret_cast<const f32x4*>(&sl.lq[i0]);
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float e = xx[q] * fexp2(lqi[q] - lj) * nj;
        v[q] = (j < i0 + q) ? e : 0.f;
      }
      uint2 pk;
      pk.x = pack2(v[0], v[1]);
      pk.y = pack2(v[2], v[3]);
      put4<kC>(AT, oA, jb * 16, ib * 16, pk);
    }
  }
}

// bf16x8 fragment scaled element-wise by 8 floats (rounded back to bf16).
__device__ __forceinline__ bf16x8 scale8(const bf16x8& v, const f32x4& s0, const f32x4& s1) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  uint4 r;
  r.x = pack2(bf16_val(u.x & 0xffffu) * s0[0], bf16_val(u.x >> 16) * s0[1]);
  r.y = pack2(bf16_val(u.y & 0xffffu) * s0[2], bf16_val(u.y >> 16) * s0[3]);
  r.z = pack2(bf16_val(u.z & 0xffffu) * s1[0], bf16_val(u.z >> 16) * s1[1]);
  r.w = pack2(bf16_val(u.w & 0xffffu) * s1[2], bf16_val(u.w >> 16) * s1[3]);
  return __builtin_bit_cast(bf16x8, r);
}

template <int D, bool HAS_Y, bool HAS_ST>
__global__ __launch_bounds__(kNT) void fwd_mfma(FwdArgs a) {
  static_assert(D == 64 || D == 128, "D");
  constexpr int NTILE = D / kTN;
  constexpr int NS = D / 32;  // 16x16 state blocks per wave
  constexpr int P = kLoadOps<D>;
  constexpr int S = (HAS_Y ? 2 : 0) + (HAS_ST ? NS : 0);  // stores per wave per chunk
  // Each ring slot is a separate LDS object, and every reference to one is
  // static (the chunk loop is unrolled by kRing), so the compiler can tell a
  // slot being read from the slots still being filled and adds no waits.
  __shared__ Slot<D> ring0, ring1, ring2, ring3, ring4;
  __shared__ __bf16 AT_s[2][kC * kC];  // AT[j][i] = A_ij, swizzled, by chunk parity
  __shared__ __bf16 S_s[2][kTN * D];   // D_in of the tile, bf16, swizzled [row][col], by parity
  static_assert(kRing == 5, "ring objects");
  Slot<D>* const rs[kRing] = {&ring0, &ring1, &ring2, &ring3, &ring4};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int g4 = lane >> 4, l16 = lane & 15;
  // 8 consecutive sequence-heads and all their row tiles share one XCD
  // (work-groups are dealt to the 8 XCDs round-robin), so the x chunk that
  // every tile reads is fetched from HBM once into that XCD's L2.
  const int grp = blockIdx.x / (8 * NTILE), within = blockIdx.x % (8 * NTILE);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  const int tile = within >> 3;
  if (bh >= a.B * a.H) return;
  const int r0 = tile * kTN;
  const int h = static_cast<int>(bh % a.H);
  const int64_t T = a.T;
  const int n = a.n_chunks;
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * D;
  const uint16_t* g = static_cast<const uint16_t*>(a.g) + bh * T * D;
  const float* eta = static_cast<const float*>(a.eta) + bh * T;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * D * D;
  uint16_t* y = HAS_Y ? static_cast<uint16_t*>(a.y) + bh * T * D : nullptr;
  uint16_t* st = HAS_ST ? static_cast<uint16_t*>(a.states) + bh * static_cast<int64_t>(n) * D * D
                        : nullptr;

  // W0 rows of the tile as MFMA A fragments, held in registers throughout
  bf16x8 wf[2][D / 32];
  if (HAS_Y) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
        wf[rb][kb] = *reinterpret_cast<const bf16x8*>(
            W0 + static_cast<int64_t>(r0 + rb * 16 + l16) * D + kb * 32 + 8 * g4);
  }
  for (int idx = tid; idx < kTN * D / 8; idx += kNT)
    reinterpret_cast<uint4*>(S_s[0])[idx] = make_uint4(0, 0, 0, 0);
  if (HAS_Y)
    for (int idx = tid; idx < 2 * kC * kC / 8; idx += kNT)
      reinterpret_cast<uint4*>(&AT_s[0][0])[idx] = make_uint4(0, 0, 0, 0);
  wait_vm<0>();

  const auto cv_of = [&](int c) {
    return static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };

  const DmaOff<D> od = dma_off<D>(wave, lane);
  const __amdgpu_buffer_rsrc_t r_none = buffer_rsrc(y ? static_cast<const void*>(y) : a.x, 0);
  // per-lane byte offsets of the stores (loop invariant; the buffer base
  // moves per chunk and its byte count drops rows past the sequence end)
  uint32_t oy[2], os[NS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
    oy[rb] = static_cast<uint32_t>(((wave * 16 + l16) * D + r0 + rb * 16 + 4 * g4) * 2);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int b = wave + 4 * s, cb = b >> 1, rb = b & 1;
    os[s] = static_cast<uint32_t>(((r0 + rb * 16 + l16) * D + cb * 16 + 4 * g4) * 2);
  }
  // Initial loads, each followed by S stores into a zero-byte buffer (they
  // are dropped) so that the vector-memory instruction stream has the same
  // shape as in the loop: chunk load, S stores, chunk load, ...  Then the
  // wait at the top of every iteration is the same constant.
#pragma unroll
  for (int k = 0; k < kRing - 1; ++k) {
    issue_chunk<D>(*rs[k], od, x, g, eta, alpha, T, k, n, r0, wave);
    // distinct offsets, so that none of them is merged away
    if (HAS_ST)
#pragma unroll
      for (int s = 0; s < NS; ++s) store8(r_none, os[s] + k, make_uint2(0, 0));
    if (HAS_Y)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) store8(r_none, oy[rb] + k, make_uint2(0, 0));
  }
  // chunk 0 done: after it come kRing - 2 more chunk loads and kRing - 1 store groups
  wait_vm<(kRing - 2) * P + (kRing - 1) * S>();
  lds_barrier();
  const LaneOff<D> oX = lane_off<D>(lane);
  const LaneOff<kTN> oG = lane_off<kTN>(lane);
  const LaneOff<kC> oA = lane_off<kC>(lane);
  float gam = prep_gates<D>(*rs[0], cv_of(0), lane);
  if (HAS_Y) scores<D>(*rs[0], AT_s[0], oX, oA, wave, lane);

  f32x4 sacc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) sacc[s] = zero4();

  // one chunk; K = c % kRing is a compile-time constant
  const auto step = [&](auto KC, int c) {
    constexpr int K = decltype(KC)::value;
    Slot<D>& cur = *rs[K];
    Slot<D>& nxt = *rs[(K + 1) % kRing];
    Slot<D>& dst = *rs[(K + kRing - 1) % kRing];
    const int64_t t0 = static_cast<int64_t>(c) * kC;
    const int cv = cv_of(c);
    const bool more = c + 1 < n;
    // chunk c + 1 done: issued after it are the stores of its own group and
    // (kRing - 3) x (chunk load + stores); past the end it is a zero fill
    wait_vm<(kRing - 3) * P + (kRing - 2) * S>();
    lds_barrier();  // chunk c + 1 loaded; scores of c, D_in of c, gates of c visible
    issue_chunk<D>(dst, od, x, g, eta, alpha, T, c + kRing - 1, n, r0, wave);

    if (HAS_ST) {
      // chunk-start state of this tile (rows r0.., natural layout, bf16)
      const __amdgpu_buffer_rsrc_t rs_st = buffer_rsrc(st + static_cast<int64_t>(c) * D * D, D * D * 2);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        uint2 v;
        v.x = pack2(sacc[s][0], sacc[s][1]);
        v.y = pack2(sacc[s][2], sacc[s][3]);
        store8(rs_st, os[s], v);
      }
    }

    float gam_next = 1.f;
    if (more) {
      gam_next = prep_gates<D>(nxt, cv_of(c + 1), lane);
      if (HAS_Y) scores<D>(nxt, AT_s[(c + 1) & 1], oX, oA, wave, lane);
    }

    const __bf16* S_in = S_s[c & 1];
    if (HAS_Y) {
      // y^T[r][i] for i in this wave's token block, both row blocks; each lane
      // stores 4 consecutive rows of one token straight from the accumulators
      const int w = wave;
      const __bf16* AT = AT_s[c & 1];
      f32x4 ya[2] = {zero4(), zero4()}, yb[2] = {zero4(), zero4()};
      for (int kb = 0; kb < (w + 2) / 2; ++kb) {
        const bf16x8 af = frag_ts<kC>(AT, oA, kb * 32, w * 16);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          ya[rb] = mfma16x16x32(frag_ts<kTN>(cur.G, oG, kb * 32, rb * 16), af, ya[rb]);
      }
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8 xf = frag_s<D>(cur.X, oX, w * 16, kb * 32);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          ya[rb] = mfma16x16x32(wf[rb][kb], xf, ya[rb]);
          yb[rb] = mfma16x16x32(frag_s<D>(S_in, oX, rb * 16, kb * 32), xf, yb[rb]);
        }
      }
      const int i = w * 16 + l16;
      const float eqi = fexp2(cur.lq[i]);
      const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(y + t0 * D, cv * D * 2);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        uint2 pk;
        pk.x = pack2(ya[rb][0] + eqi * yb[rb][0], ya[rb][1] + eqi * yb[rb][1]);
        pk.y = pack2(ya[rb][2] + eqi * yb[rb][2], ya[rb][3] + eqi * yb[rb][3]);
        store8(ry, oy[rb], pk);
      }
    }

    // state update, transposed: D^T[c][r] = Gamma D^T + sum_j x_j[c] (bk_j g_j[r]),
    // into the other state buffer (the current one may still be read)
    {
      const int rbw = wave & 1;
      bf16x8 gs[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int k0 = kb * 32 + 8 * g4;
        gs[kb] = scale8(frag_ts<kTN>(cur.G, oG, kb * 32, rbw * 16),
                        *reinterpret_cast<const f32x4*>(&cur.bk[k0]),
                        *reinterpret_cast<const f32x4*>(&cur.bk[k0 + 4]));
      }
      __bf16* S_out = S_s[(c + 1) & 1];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int cb = (wave >> 1) + 2 * s;
        sacc[s] = sacc[s] * gam;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sacc[s] = mfma16x16x32(frag_ts<D>(cur.X, oX, kb * 32, cb * 16), gs[kb], sacc[s]);
        uint2 pk;
        pk.x = pack2(sacc[s][0], sacc[s][1]);
        pk.y = pack2(sacc[s][2], sacc[s][3]);
        put4<D>(S_out, oX, rbw * 16, cb * 16, pk);
      }
    }
    gam = gam_next;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  for (int c = 0; c < n; c += kRing) {
    step(I0{}, c);
    if (c + 1 >= n) break;
    step(I1{}, c + 1);
    if (c + 2 >= n) break;
    step(I2{}, c + 2);
    if (c + 3 >= n) break;
    step(I3{}, c + 3);
    if (c + 4 >= n) break;
    step(I4{}, c + 4);
  }
  wait_vm<0>();  // no load into LDS may outlive the work-group
}

template <int D, bool HAS_Y, bool HAS_ST>
hipError_t launch_v(const FwdArgs& a, hipStream_t s) {
  const int64_t groups = (a.B * a.H + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (D / kTN)));
  hipLaunchKernelGGL((fwd_mfma<D, HAS_Y, HAS_ST>), grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  if (a.y && a.states) return launch_v<D, true, true>(a, s);
  if (a.y) return launch_v<D, true, false>(a, s);
  if (a.states) return launch_v<D, false, true>(a, s);
  return hipSuccess;
}

}  // namespace

hipError_t launch_mfma_fwd(const FwdArgs& a, hipStream_t s) {
  return a.d_in == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace gls
