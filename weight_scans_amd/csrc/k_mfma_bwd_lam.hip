// k_mfma_bwd_lam.hip -- adjoint-only pass of the segmented matrix-core
// reverse scan (bf16 io, d_in = d_out = D in {64, 128}; gfx950).
//
// The reverse scan carries the adjoint Lam = dL/dD from the right end of the
// sequence (the exact adjoint of the forward scan, GradLev abstract,
// omanscience.com):
//   Lam_in = e(l_last) Lam_out + sum_u e(lq_u) dy_u x_u^T
// (chunk-local l = inclusive cumsum of log2 alpha, lq_u = l_{u-1},
// e(.) = 2^(.)).  When a sequence is cut into segments, this pass runs the
// recurrence over each segment s >= 1 from a zero start and reports its
// result L_s (at the segment's left end) and the segment's summed log2
// alpha; composing these from the right gives every segment the adjoint
// entering it (the associative combine of "Parallelize the Training, Keep
// the Learning Serial", cognaptus.com, section "Once the gradient signals are
// known, the weight trajectory becomes parallelizable", run in reverse).
// Segment 0's own result is never needed, so it is not computed.
//
// One work-group per (segment, sequence-head, tile of TR rows r of Lam),
// eight waves; x and the dy rows of the tile come by direct buffer loads into
// two slots, one chunk ahead; two barriers per chunk (slot free, then e(lq) dy
// visible to the matrix-core update).  What bounds the pass is the address
// unit's throughput of direct loads, so no load carries bytes nobody uses:
// the alpha row is one 4-byte load per lane, and where the dy rows need fewer
// loads than there are waves, the others load nothing (4 bytes from an empty
// buffer) to keep one count of loads per wave.  Each tile reads the whole x
// chunk, so fewer tiles read it fewer times: at d = 64 one tile holds the
// whole adjoint (half-height tiles ran about 3 us longer at [8,16,4096,64]);
// at d = 128 half-height tiles (x read twice) and whole ones (one work-group
// per CU) take the same time, and 32-row tiles ran about 30% longer.
#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "dev_common.hpp"
#include "internal.hpp"
#include "mfma.hpp"

namespace gls {
namespace {

constexpr int kC = 64;         // tokens per chunk
constexpr int kNW = 8;         // waves per work-group
constexpr int kNT = 64 * kNW;  // threads

// TR = rows r of Lam per work-group (D: the whole adjoint, D / 2: half).
template <int D, int TR>
struct alignas(16) SlotL {
  __bf16 X[kC * D];     // x of the chunk, swizzled [token][D]
  __bf16 Dr[kC * TR];   // dy of the row tile, swizzled [token][TR]
  float q[kC];          // alpha of the chunk
  float pad[kC];        // target of the empty loads
};

struct alignas(16) GatesL {
  float eq[kC];  // e(lq) of the chunk's tokens
};

// dy tile loads of 1 KB: TR / 8 in all, kLT<TR> per wave (waves past the
// tile's loads issue one empty 4-byte load instead)
template <int TR>
constexpr int kLT = (TR / 8 + kNW - 1) / kNW;

template <int D, int TR>
struct DmaOffL {
  uint32_t x[D / 64];
  uint32_t t[kLT<TR>];
  uint32_t q;
};
template <int D, int TR>
__device__ __forceinline__ DmaOffL<D, TR> dma_off_l(int wave, int lane) {
  constexpr int U = D / 8;
  DmaOffL<D, TR> o;
#pragma unroll
  for (int s = 0; s < D / 64; ++s) {
    const int p = (wave + 8 * s) * 64 + lane;
    const int row = p / U, kl = (p % U) ^ swz<D>(row);
    o.x[s] = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  }
  constexpr int UT = TR / 8;  // 16-byte units per row of the dy tile
#pragma unroll
  for (int s = 0; s < kLT<TR>; ++s) {
    const int p = ((wave + 8 * s) % (TR / 8)) * 64 + lane;  // (unused past the tile's loads)
    const int row = p / UT, kl = (p % UT) ^ swz<TR>(row);
    o.t[s] = static_cast<uint32_t>(row * D * 2 + 16 * kl);
  }
  o.q = static_cast<uint32_t>(lane * 4);
  return o;
}

// Loads of chunk k (negative: zero fill): x (all waves), the dy rows of the
// tile, the alpha row (every wave, the same bytes).
template <int D, int TR>
__device__ __forceinline__ void issue_chunk_l(SlotL<D, TR>& sl, const DmaOffL<D, TR>& o,
                                              const uint16_t* x, const uint16_t* dy,
                                              const float* alpha, int64_t T, int k, int r0,
                                              int wave) {
  const bool in = k >= 0;
  const int64_t t0 = in ? static_cast<int64_t>(k) * kC : 0;
  const int cv = in ? static_cast<int>(std::min<int64_t>(kC, T - t0)) : 0;
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + t0 * D, cv * D * 2);
#pragma unroll
  for (int s = 0; s < D / 64; ++s) dma16(rx, o.x[s], sl.X + (wave + 8 * s) * 512);
  // dy rows of the tile (64 x TR: TR / 8 loads of 1 KB); where they take
  // fewer loads than there are waves, the other waves issue a 4-byte load of
  // nothing into a pad instead (the same count of loads in every wave)
  constexpr int NLT = kC * TR / 512;
  const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(dy + t0 * D + r0, cv > 0 ? (cv * D - r0) * 2 : 0);
#pragma unroll
  for (int s = 0; s < kLT<TR>; ++s) {
    if (NLT >= kNW || wave < NLT)
      dma16(rd, o.t[s], sl.Dr + (wave + 8 * s) * 512);
    else
      dma4(buffer_rsrc(dy, 0), o.q, sl.pad);
  }
  dma4(buffer_rsrc(alpha + t0, cv * 4), o.q, sl.q);
}

template <int D, int TR>
__global__ __launch_bounds__(kNT) void bwd_lam(BwdArgs a) {
  static_assert(D == 64 || D == 128, "D");
  static_assert(TR == D || TR == D / 2, "TR");
  constexpr int NTILE = D / TR;
  constexpr int NRB = TR / 16, NKB = D / 16;  // r and k blocks of the tile
  constexpr int NBW = NRB * NKB / kNW;        // blocks per wave
  constexpr int RPW = NBW >= 8 ? 2 : 1;       // r blocks per wave
  constexpr int KPW = NBW / RPW;              // k blocks per wave
  constexpr int NRW = NRB / RPW;              // waves along r
  static_assert(NRW * (NKB / KPW) == kNW, "every block owned once");
  constexpr int EPT = kC * TR / kNT;          // elements of the dy tile per thread
  static_assert(EPT == 4 || EPT % 8 == 0, "EPT");
  __shared__ SlotL<D, TR> ring0, ring1;
  __shared__ __bf16 DS_s[kC * TR];  // e(lq_u) dy_u of the row tile
  __shared__ GatesL gs;
  SlotL<D, TR>* const rs[2] = {&ring0, &ring1};

  const int per_seg = static_cast<int>((a.B * a.H + 7) / 8) * 8 * NTILE;
  // segments seg_first .. n_seg - 1 (8 consecutive heads and their tiles share an XCD)
  const int seg = a.seg_first + static_cast<int>(blockIdx.x / per_seg), bid = blockIdx.x % per_seg;
  const int grp = bid / (8 * NTILE), within = bid % (8 * NTILE);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  if (bh >= a.B * a.H) return;
  const int tile = within >> 3;
  const int r0 = tile * TR;
  const int64_t T = a.T;
  const int n = a.n_chunks;
  const int c_beg = seg * a.seg_chunks;
  const int c_end = std::min(n, c_beg + a.seg_chunks);
  const int nloc = c_end - c_beg;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  // r blocks RPW rw .., k blocks KPW kw .. of the tile
  const int rw = wave % NRW, kw = wave / NRW;
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * D;
  const uint16_t* dy = static_cast<const uint16_t*>(a.dy) + bh * T * D;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;

  const LaneOff<D> oX = lane_off<D>(lane);
  const LaneOff<TR> oT = lane_off<TR>(lane);
  const DmaOffL<D, TR> od = dma_off_l<D, TR>(wave, lane);
  // this thread's elements of the dy tile: row tid / 8, columns EPT (tid % 8) ..
  const int ds_row = tid >> 3;
  constexpr int NU = EPT >= 8 ? EPT / 8 : 1;  // 16-byte units (EPT >= 8)
  uint32_t ds_off[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u)
    ds_off[u] = static_cast<uint32_t>(sidx<TR>(ds_row, EPT * (tid & 7) + 8 * u) * 2);
  const auto cv_of = [&](int c) {
    return static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };

  // Lam^T blocks of the tile (k block KPW kw + j, r block RPW rw + i), fp32, from zero
  f32x4 lam[RPW][KPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int j = 0; j < KPW; ++j) lam[i][j] = zero4();
  float lsum = 0.f;  // summed log2 alpha of the segment

  issue_chunk_l<D, TR>(*rs[0], od, x, dy, alpha, T, c_end - 1, r0, wave);
  const auto step = [&](auto KC, int vis) {
    constexpr int K = decltype(KC)::value;
    SlotL<D, TR>& cur = *rs[K];
    const int c = c_end - 1 - vis;
    const int cv = cv_of(c);
    wait_vm<0>();   // chunk c loaded
    lds_barrier();  // and the previous chunk's reads of the other slot done
    issue_chunk_l<D, TR>(*rs[K ^ 1], od, x, dy, alpha, T, c - 1 >= c_beg ? c - 1 : -1, r0, wave);
    // gates: every wave derives them and writes the same e(lq) row, then
    // reads back only entries it wrote itself (one wave's LDS accesses land
    // in order), so no barrier is needed before the scaling
    const ChunkGates gt = chunk_gates(lane < cv ? cur.q[lane] : 1.f, lane);
    gs.eq[lane] = fexp2(gt.lq);
    const float gam = fexp2(gt.llast);
    lsum += gt.llast;
    {
      const float e = gs.eq[ds_row];
      if constexpr (EPT == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(cur.Dr) + ds_off[0]);
        uint2 r;
        r.x = pack2(bf16_val(v.x & 0xffffu) * e, bf16_val(v.x >> 16) * e);
        r.y = pack2(bf16_val(v.y & 0xffffu) * e, bf16_val(v.y >> 16) * e);
        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(DS_s) + ds_off[0]) = r;
      } else {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(cur.Dr) + ds_off[u]);
          uint4 r;
          r.x = pack2(bf16_val(v.x & 0xffffu) * e, bf16_val(v.x >> 16) * e);
          r.y = pack2(bf16_val(v.y & 0xffffu) * e, bf16_val(v.y >> 16) * e);
          r.z = pack2(bf16_val(v.z & 0xffffu) * e, bf16_val(v.z >> 16) * e);
          r.w = pack2(bf16_val(v.w & 0xffffu) * e, bf16_val(v.w >> 16) * e);
          *reinterpret_cast<uint4*>(reinterpret_cast<char*>(DS_s) + ds_off[u]) = r;
        }
      }
    }
    lds_barrier();  // e(lq) dy visible
    // Lam^T[k][r] <- Gamma Lam^T + sum_u x_u[k] e(lq_u) dy_u[r]
    bf16x8 dsf[RPW][2];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dsf[i][kb] = frag_ts<TR>(DS_s, oT, kb * 32, (RPW * rw + i) * 16);
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) lam[i][j] = lam[i][j] * gam;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 xf = frag_ts<D>(cur.X, oX, kb * 32, (KPW * kw + j) * 16);
#pragma unroll
        for (int i = 0; i < RPW; ++i) lam[i][j] = mfma16x16x32(xf, dsf[i][kb], lam[i][j]);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  for (int vis = 0; vis < nloc; vis += 2) {
    step(I0{}, vis);
    if (vis + 1 >= nloc) break;
    step(I1{}, vis + 1);
  }
  wait_vm<0>();  // no load into LDS may outlive the work-group
  float* so = a.seg_out + (bh * a.n_seg + seg) * D * D;
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int j = 0; j < KPW; ++j)
      *reinterpret_cast<f32x4*>(so + (r0 + (RPW * rw + i) * 16 + l16) * D + (KPW * kw + j) * 16 +
                                4 * g4) = lam[i][j];
  if (tile == 0 && wave == 0 && lane == 0) a.seg_lg[bh * a.n_seg + seg] = lsum;
}

template <int D, int TR>
hipError_t launch_lam(const BwdArgs& a, hipStream_t s) {
  if (a.n_seg - a.seg_first <= 0) return hipSuccess;
  const int64_t groups = (a.B * a.H + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (D / TR) * (a.n_seg - a.seg_first)));
  hipLaunchKernelGGL((bwd_lam<D, TR>), grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_bwd_lam(const BwdArgs& a, hipStream_t s) {
  // d = 64: the whole adjoint per work-group; d = 128: half of its rows
  return a.d_in == 128 ? launch_lam<128, 64>(a, s) : launch_lam<64, 64>(a, s);
}

}  // namespace gls
