// k_mfma_bwd_chain.hip -- the serial part of the chunk-parallel reverse scan
// (bf16 io, d_in = d_out = 64; gfx950, v_mfma_f32_16x16x32_bf16).
//
// The adjoint Lam = dL/dD of the reverse scan (GradLev abstract,
// omanscience.com; the exact adjoint of the forward scan) runs backwards over
// the chunks as
//   Lam_in = e(l_last) Lam_out + sum_u e(lq_u) dy_u x_u^T
// (chunk-local l = inclusive cumsum of log2 alpha, lq_u = l_{u-1},
// e(.) = 2^(.)).  This file holds the two kernels that produce Lam_out of
// every chunk for the chunk-parallel pass (k_mfma_bwd_c.hip):
//   chunk_gates_eq: e(lq) per token and e(l_last) per chunk, one wave per
//                   chunk, all chunks in parallel;
//   bwd_chain64:    one work-group per (segment, sequence-head, 32-row tile
//                   of Lam), walking the chunks backwards with Lam in fp32
//                   accumulators and storing it (bf16) before each update.
// The chain kernel has no scans on its path: chunk tiles come kRing chunks
// deep through an LDS ring filled by direct buffer loads (deep enough to keep
// the work-group's HBM requests overlapping); each wave scales by e(lq) the
// part of the dy tile its own MFMA reads (so no other wave waits for it), and
// one barrier separates the chunks.
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
constexpr int kT = 32;          // rows of Lam per work-group
constexpr int kNW = 8;          // waves per work-group
constexpr int kNT = 64 * kNW;   // threads
constexpr int kRing = 3;        // ring slots of two chunks each
constexpr int kGateThreads = 256;

// e(lq) of every token and e(l_last) of every chunk (one wave per chunk).
__global__ __launch_bounds__(kGateThreads) void chunk_gates_eq(const float* alpha, float* eq,
                                                               float* gam, int64_t BH, int64_t T,
                                                               int n_chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * (kGateThreads / 64) + (threadIdx.x >> 6);
  if (item >= BH * n_chunks) return;
  const int64_t bh = item / n_chunks;
  const int c = static_cast<int>(item % n_chunks);
  const int64_t t0 = static_cast<int64_t>(c) * kC;
  const int cv = static_cast<int>(std::min<int64_t>(kC, T - t0));
  const ChunkGates gt = chunk_gates(lane < cv ? alpha[bh * T + t0 + lane] : 1.f, lane);
  if (lane < cv) eq[bh * T + t0 + lane] = fexp2(gt.lq);
  if (lane == 0) gam[item] = fexp2(gt.llast);
}

struct alignas(16) ChunkL {
  __bf16 X[kC * kD];   // x of the chunk, swizzled [token][D]
  __bf16 Dr[kC * kT];  // dy of the row tile, swizzled [token][kT]
  float eq[kC];        // e(lq) of the chunk's tokens
  float gm[kC];        // gm[0] = e(l_last) of the chunk (the rest: zero fill)
};
// A ring slot holds two consecutive chunks of the walk (three slot objects,
// four chunks in flight).
struct alignas(16) SlotL {
  ChunkL ch[2];
};

__global__ __launch_bounds__(kNT) void bwd_chain64(BwdArgs a) {
  constexpr int NTILE = kD / kT;
  constexpr int P = 8;  // loads per wave per pair of chunks: x, dy rows, e(lq), e(l_last) each
  constexpr int S = 2;  // stores per wave per pair: its block of Lam_out, twice
  __shared__ SlotL ring0, ring1, ring2;
  __shared__ __bf16 DS0[kC * kT], DS1[kC * kT];  // e(lq_u) dy_u of the row tile, per chunk of a pair
  SlotL* const rs[kRing] = {&ring0, &ring1, &ring2};
  __bf16* const ds[2] = {DS0, DS1};

  const int per_seg = static_cast<int>((a.B * a.H + 7) / 8) * 8 * NTILE;
  const int seg = blockIdx.x / per_seg, bid = blockIdx.x % per_seg;
  const int grp = bid / (8 * NTILE), within = bid % (8 * NTILE);
  const int64_t bh = static_cast<int64_t>(grp) * 8 + (within & 7);
  const int tile = within >> 3;
  if (bh >= a.B * a.H) return;
  const int r0 = tile * kT;
  const int64_t T = a.T;
  const int n = a.n_chunks;
  const int c_beg = seg * a.seg_chunks;
  const int c_end = std::min(n, c_beg + a.seg_chunks);
  const int nloc = c_end - c_beg;
  const int npair = (nloc + 1) / 2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int cb = wave >> 1, rbw = wave & 1;  // this wave's block: columns cb, rows rbw of the tile
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * kD;
  const uint16_t* dy = static_cast<const uint16_t*>(a.dy) + bh * T * kD;
  const float* eqg = a.gate_eq + bh * T;
  const float* gam = a.gate_gam + bh * n;
  uint16_t* lo = static_cast<uint16_t*>(a.lam_out) + bh * static_cast<int64_t>(n) * kD * kD;

  const LaneOff<kD> oX = lane_off<kD>(lane);
  const LaneOff<kT> oT = lane_off<kT>(lane);

  // Lam rows of the tile entering from the right (fp32 accumulators)
  f32x4 lam = zero4();
  if (a.seg_lam)
    lam = *reinterpret_cast<const f32x4*>(a.seg_lam + (bh * a.n_seg + seg) * kD * kD +
                                          (r0 + rbw * 16 + l16) * kD + cb * 16 + 4 * g4);
  wait_vm<0>();

  // per-lane load offsets: x instruction w of 8; a quarter of the dy row tile
  // (waves 4-7 repeat 0-3: same bytes); the gate rows (all waves, same bytes)
  uint32_t ox, odr;
  {
    const int p = wave * 64 + lane;
    const int row = p >> 3, kl = (p & 7) ^ swz<kD>(row);
    ox = static_cast<uint32_t>(row * kD * 2 + 16 * kl);
    const int p2 = (wave & 3) * 64 + lane;
    const int row2 = p2 >> 2, kl2 = (p2 & 3) ^ swz<kT>(row2);
    odr = static_cast<uint32_t>(row2 * kD * 2 + 16 * kl2);
  }
  const uint32_t oeq = static_cast<uint32_t>(lane * 4);
  const uint32_t olo = static_cast<uint32_t>(((r0 + rbw * 16 + l16) * kD + cb * 16 + 4 * g4) * 2);
  const __amdgpu_buffer_rsrc_t r_none = buffer_rsrc(a.x, 0);

  // chunk visited k-th (-1: none -> zero fill)
  const auto chunk_at = [&](int k) { return c_end - 1 - k >= c_beg ? c_end - 1 - k : -1; };
  const auto issue1 = [&](ChunkL& cl, int k) {
    const bool in = k >= 0;
    const int64_t t0 = in ? static_cast<int64_t>(k) * kC : 0;
    const int cv = in ? static_cast<int>(std::min<int64_t>(kC, T - t0)) : 0;
    dma16(buffer_rsrc(x + t0 * kD, cv * kD * 2), ox, cl.X + wave * 512);
    dma16(buffer_rsrc(dy + t0 * kD + r0, cv > 0 ? (cv * kD - r0) * 2 : 0), odr,
          cl.Dr + (wave & 3) * 512);
    dma4(buffer_rsrc(eqg + t0, cv * 4), oeq, cl.eq);
    dma4(buffer_rsrc(gam + (in ? k : 0), in ? 4 : 0), oeq, cl.gm);
  };
  // pair j: chunks visited 2j and 2j + 1
  const auto issue = [&](SlotL& sl, int j) {
    issue1(sl.ch[0], chunk_at(2 * j));
    issue1(sl.ch[1], chunk_at(2 * j + 1));
  };
  // e(lq_u) dy_u[r] for this wave's 16 rows of the tile (rows rbw of the
  // MFMA operand), all 64 tokens: 4 x 4 elements per lane.  The four waves
  // with the same rbw write the same values.
  const auto scale = [&](const ChunkL& cl, __bf16* DS) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = 16 * k + (lane >> 2), cc = rbw * 16 + 4 * (lane & 3);
      const uint32_t off = static_cast<uint32_t>(sidx<kT>(u, cc) * 2);
      const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(cl.Dr) + off);
      const float e = cl.eq[u];
      uint2 r;
      r.x = pack2(bf16_val(v.x & 0xffffu) * e, bf16_val(v.x >> 16) * e);
      r.y = pack2(bf16_val(v.y & 0xffffu) * e, bf16_val(v.y >> 16) * e);
      *reinterpret_cast<uint2*>(reinterpret_cast<char*>(DS) + off) = r;
    }
  };
  // one chunk: Lam_out stored, then Lam <- Gamma Lam + sum_u e(lq_u) dy_u x_u^T
  const auto apply = [&](const ChunkL& cl, __bf16* DS, int k) {
    const int c = chunk_at(k);
    const __amdgpu_buffer_rsrc_t r_lo =
        c >= 0 ? buffer_rsrc(lo + static_cast<int64_t>(c) * kD * kD, kD * kD * 2) : r_none;
    uint2 pk;
    pk.x = pack2(lam[0], lam[1]);
    pk.y = pack2(lam[2], lam[3]);
    store8(r_lo, olo, pk);
    scale(cl, DS);
    lam = lam * cl.gm[0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      lam = mfma16x16x32(frag_ts<kD>(cl.X, oX, kb * 32, cb * 16),
                         frag_ts<kT>(DS, oT, kb * 32, rbw * 16), lam);
  };

  // the first two pairs, each followed by S dropped stores (stream shape as
  // in the loop)
  issue(*rs[0], 0);
  store8(r_none, olo, make_uint2(0, 0));
  store8(r_none, olo + 64, make_uint2(0, 0));  // spaced: not merged
  issue(*rs[1], 1);
  store8(r_none, olo + 128, make_uint2(0, 0));
  store8(r_none, olo + 192, make_uint2(0, 0));

  // step j: the pair j in slot j % 3.  A missing second chunk (odd chunk
  // count, last pair only) is a zero fill: its Lam_out store is dropped and
  // the Lam it leaves (zero) is never read.
  const auto step = [&](auto KC, int j) {
    constexpr int K = decltype(KC)::value;
    // pair j loaded: after it come its S stores, pair j + 1 and its S stores
    wait_vm<P + 2 * S>();
    lds_barrier();  // slot (j + 2) % 3 and both DS buffers free
    issue(*rs[(K + 2) % kRing], j + 2);
    apply(rs[K]->ch[0], ds[0], 2 * j);
    apply(rs[K]->ch[1], ds[1], 2 * j + 1);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  for (int j = 0; j < npair; j += kRing) {
    step(I0{}, j);
    if (j + 1 >= npair) break;
    step(I1{}, j + 1);
    if (j + 2 >= npair) break;
    step(I2{}, j + 2);
  }
  wait_vm<0>();  // no load into LDS may outlive the work-group
}

}  // namespace

hipError_t launch_mfma_bwd_chain64(const BwdArgs& a, hipStream_t s) {
  const int64_t BH = a.B * a.H;
  const int64_t items = BH * a.n_chunks;
  const int64_t per_block = kGateThreads / 64;
  hipLaunchKernelGGL(chunk_gates_eq, dim3(static_cast<unsigned>((items + per_block - 1) / per_block)),
                     dim3(kGateThreads), 0, s, static_cast<const float*>(a.alpha), a.gate_eq,
                     a.gate_gam, BH, a.T, a.n_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t groups = (BH + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (kD / kT) * a.n_seg));
  hipLaunchKernelGGL(bwd_chain64, grid, dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace gls
