// k_mfma_bwd_f128.hip -- fused matrix-core reverse scan for bf16 io,
// d_in = d_out = 128 (gfx950, v_mfma_f32_16x16x32_bf16).
//
// The same per-chunk mathematics as the d = 64 kernel (k_mfma_bwd_f.hip; P,
// Be, M = Be + Be^T and the Be dots in bwd_fused.hpp; the exact adjoint of the
// forward scan, GradLev abstract, omanscience.com):
//   u_i   = e(l_last - l_i) Lam_out x_i + sum_{u>i} P_ui dy_u
//   dg_i  = -eta_i u_i,  deta_i = -g_i . u_i
//   dx_i  = W0^T dy_i + e(lq_i) D_in^T dy_i + (M X)_i - eta_i e(l_last - l_i) Lam_out^T g_i
//   dW0  += sum_u dy_u x_u^T,  Lam_in = e(l_last) Lam_out + sum_u e(lq_u) dy_u x_u^T
// One work-group per (segment, sequence-head) walks its chunks from the
// right with the whole 128 x 128 adjoint and dW0 in fp32 registers.
//
// A chunk's tiles (x, g, dy: 16 KB each; D_in: 32 KB) fill one LDS slot; the
// next chunk is loaded into registers (ten 16-byte units per thread) while
// this one is worked on, and written into the slot at the top of the next
// step -- so the slot is single and 80 KB of loads are in flight per CU.
// Eight waves (two per SIMD: the adjoint, dW0 and the staged chunk need the
// register room); wave w holds the 32 x 64 region (k rows 32 (w % 4) ..,
// r columns 64 (w / 4) ..) of Lam and dW0.  Three barriers per step:
//   top:     the staged chunk into the slot, the bf16 copy of Lam_out, the
//            first loads of the next chunk (and the gate rows of the one
//            after; the other loads are issued at the start of A and B);
//   phase A: causal blocks (P^T, M, the Be dots: block w, and 8, 9 on waves
//            2, 3); every wave its region of Lam and dW0 (<Lam_out, D_in>
//            share, then the update); wave 0 the gates of the next chunk,
//            wave 1 dalpha and deta of the chunk before (its shares are
//            complete after the first barrier);
//   phase B: every wave 16 columns of dx (all tokens) with its rr share, and
//            the 32 x 32 block (rows 32 (w % 4) .., tokens 32 (w / 4) ..) of
//            u: dg, the deta and pp shares.
// All loads go to registers (the compiler places the waits); no
// direct-to-LDS loads are involved.
#include <type_traits>

#include "bwd_fused.hpp"

namespace gls {
namespace {

constexpr int kD = 128;        // d_in = d_out
constexpr int kC = kFC;        // tokens per chunk
constexpr int kNW = 8;         // waves per work-group
constexpr int kNT = 64 * kNW;  // threads
constexpr int kRowWave = 1;    // eta / alpha rows of the chunk after next
constexpr int kGateWave = 0;   // gates of the next chunk (phase A)
constexpr int kAlphaWave = 1;  // dalpha and deta one chunk behind (phase A)

struct alignas(16) SlotH {
  __bf16 X[kC * kD];   // x, swizzled [token][k]
  __bf16 G[kC * kD];   // g, swizzled [token][r]
  __bf16 DY[kC * kD];  // dy, swizzled [token][r]
  __bf16 S[kD * kD];   // D_in, swizzled [r][k]
};

struct alignas(16) PartH {  // per-token shares of one chunk
  float pp[4][kC], de[4][kC];  // over u rows 32 q .. (q = wave % 4)
  float rr[kNW][kC];           // over dx columns 16 w ..
  float c0[kNW];               // <Lam_out, D_in> over each wave's region
};

// 16-byte unit u of a [rows][128] bf16 tile (16 units per row): read from
// byte u * 16, written to its swizzled place.
__device__ __forceinline__ uint32_t unit_lds(int u) {
  return static_cast<uint32_t>(sidx<kD>(u >> 4, 8 * (u & 15)) * 2);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

template <bool F32>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(1, 2)))
void bwd_f128(BwdArgs a) {
  constexpr int OE = F32 ? 4 : 2;  // bytes per element of dx, dg
  __shared__ SlotH sl;
  __shared__ __bf16 L_s[kD * kD];           // Lam_out, bf16 [r][k]; W0 staging at the start
  __shared__ __bf16 PT_s[kC * kC];          // P^T
  __shared__ __bf16 M_s[kC * kC + kMPad];   // Be + Be^T (+ pad)
  __shared__ float rows_s[2][2][kC];        // eta, alpha rows by chunk parity
  __shared__ RecF rec[4];
  __shared__ PartH part[2];
  __shared__ QkF qk[2];

  const int64_t BH = a.B * a.H, T = a.T;
  const int n = a.n_chunks;
  const int64_t bh = blockIdx.x % BH;
  const int seg = static_cast<int>(blockIdx.x / BH);
  const int c_beg = seg * a.seg_chunks;
  const int c_end = std::min(n, c_beg + a.seg_chunks);
  const int nloc = c_end - c_beg;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  // this wave's region of Lam^T and dW0^T: k blocks 2 kq + a, r blocks 4 rh + b
  const int kq = wave & 3, rh = wave >> 2;
  const int h = static_cast<int>(bh % a.H);
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + bh * T * kD;
  const uint16_t* g = static_cast<const uint16_t*>(a.g) + bh * T * kD;
  const uint16_t* dy = static_cast<const uint16_t*>(a.dy) + bh * T * kD;
  const float* eta = static_cast<const float*>(a.eta) + bh * T;
  const float* alpha = static_cast<const float*>(a.alpha) + bh * T;
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0) + static_cast<int64_t>(h) * kD * kD;
  const uint16_t* st = static_cast<const uint16_t*>(a.states) + bh * static_cast<int64_t>(n) * kD * kD;
  char* dxp = static_cast<char*>(a.dx) + bh * T * kD * OE;
  char* dgp = static_cast<char*>(a.dg) + bh * T * kD * OE;
  float* dal = static_cast<float*>(a.dalpha_out) + bh * T;
  float* det = static_cast<float*>(a.deta_out) + bh * T;

  const LaneOff<kD> o_in = lane_off<kD>(lane);
  const LaneOff<kC> o64_in = lane_off<kC>(lane);

  const auto chunk_at = [&](int v) { return (v >= 0 && v < nloc) ? c_end - 1 - v : -1; };
  const auto cv_of = [&](int c) {
    return c < 0 ? 0 : static_cast<int>(std::min<int64_t>(kC, T - static_cast<int64_t>(c) * kC));
  };

  // ---- staged loads: x, g, dy units tid and tid + 512; D_in units tid +
  // 512 j (j < 4); the eta / alpha rows (wave 1, lanes 0-31)
  u32x4 sx[2], sg[2], sdy[2], ss[4], sqe, sqa;
  // issued in three parts, one per phase of the step, so that the address
  // unit works through them while the matrix cores do (all at once, the
  // waves issuing last stall behind the queue)
  const auto load_chunk = [&](int c, auto PC) {
    constexpr int P = decltype(PC)::value;  // part: 0 x, g; 1 dy, D_in rows 0-31; 2 the rest of D_in
    const bool in = c >= 0;
    const int64_t t0 = in ? static_cast<int64_t>(c) * kC : 0;
    const int cv = cv_of(c);
    if constexpr (P == 0) {
      const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + t0 * kD, cv * kD * 2);
      const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g + t0 * kD, cv * kD * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t off = static_cast<uint32_t>((tid + kNT * j) * 16);
        sx[j] = load16(rx, off);
        sg[j] = load16(rg, off);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rs =
          buffer_rsrc(st + (in ? static_cast<int64_t>(c) : 0) * kD * kD, in ? kD * kD * 2 : 0);
      if constexpr (P == 1) {
        const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(dy + t0 * kD, cv * kD * 2);
#pragma unroll
        for (int j = 0; j < 2; ++j) sdy[j] = load16(rd, static_cast<uint32_t>((tid + kNT * j) * 16));
        ss[0] = load16(rs, static_cast<uint32_t>(tid * 16));
      } else {
#pragma unroll
        for (int j = 1; j < 4; ++j) ss[j] = load16(rs, static_cast<uint32_t>((tid + kNT * j) * 16));
      }
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  const auto load_rows = [&](int c) {
    if (wave == kRowWave) {
      const int64_t t0 = c >= 0 ? static_cast<int64_t>(c) * kC : 0;
      const int cv = cv_of(c);
      const uint32_t off = static_cast<uint32_t>((lane & 15) * 16);
      // (selected only when written out: a select here would wait for the loads)
      sqe = load16(buffer_rsrc(eta + t0, cv * 4), off);
      sqa = load16(buffer_rsrc(alpha + t0, cv * 4), off);
    }
  };
  const auto put_chunk = [&]() {
    char* b = reinterpret_cast<char*>(&sl);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t u = unit_lds(tid + kNT * j);
      *reinterpret_cast<u32x4*>(b + offsetof(SlotH, X) + u) = sx[j];
      *reinterpret_cast<u32x4*>(b + offsetof(SlotH, G) + u) = sg[j];
      *reinterpret_cast<u32x4*>(b + offsetof(SlotH, DY) + u) = sdy[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(b + offsetof(SlotH, S) + unit_lds(tid + kNT * j)) = ss[j];
  };
  const auto put_rows = [&](float (*rw)[kC]) {
    if (wave == kRowWave && lane < 32)
      *reinterpret_cast<u32x4*>(&rw[lane >> 4][4 * (lane & 15)]) = lane < 16 ? sqe : sqa;
  };

  // ---- set-up: first chunk and the gate rows of the first chunk in flight;
  // W0 staged in L_s for the dx waves' W0^T fragments; the entering adjoint
  // (given, or composed from the segments to the right)
  load_chunk(chunk_at(0), P0{});
  load_chunk(chunk_at(0), P1{});
  load_chunk(chunk_at(0), P2{});
  load_rows(chunk_at(0));
  // W0 into L_s (bf16, swizzled), all four loads in flight before the first write
  const auto stage_w0 = [&]() {
    uint4 w0v[kD * kD / 8 / kNT];
#pragma unroll
    for (int j = 0; j < kD * kD / 8 / kNT; ++j) {
      const int idx = tid + kNT * j, r = idx >> 4, cc = 8 * (idx & 15);
      w0v[j] = *reinterpret_cast<const uint4*>(W0 + static_cast<int64_t>(r) * kD + cc);
    }
#pragma unroll
    for (int j = 0; j < kD * kD / 8 / kNT; ++j) {
      const int idx = tid + kNT * j, r = idx >> 4, cc = 8 * (idx & 15);
      *reinterpret_cast<uint4*>(&L_s[sidx<kD>(r, cc)]) = w0v[j];
    }
  };
  f32x4 lam[2][4], dw[2][4];  // Lam^T / dW0^T blocks (k block 2 kq + a, r block 4 rh + b)
#pragma unroll
  for (int aa = 0; aa < 2; ++aa)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      lam[aa][b] = zero4();
      dw[aa][b] = zero4();
    }
  if (a.seg_lam) {
    // (the adjoint-only pass's segments: lam_r per fused segment, lam_n in all)
    const int ln = a.lam_n ? a.lam_n : a.n_seg, end = (seg + 1) * a.lam_r;
    const int s_lo = a.seg_lg_in ? end : end - 1;
    const int s_hi = a.seg_lg_in ? ln - 1 : end - 1;
    // this thread's elements of segment s2's tile; the next tile's loads are
    // issued before the current one is folded in
    const auto tile = [&](int s2, f32x4 (&t)[2][4]) {
      const float* sp = a.seg_lam + (bh * ln + s2) * kD * kD;
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          t[aa][b] = *reinterpret_cast<const f32x4*>(sp + ((4 * rh + b) * 16 + l16) * kD +
                                                     (2 * kq + aa) * 16 + 4 * g4);
    };
    f32x4 cur[2][4], nxt[2][4];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
      for (int b = 0; b < 4; ++b) nxt[aa][b] = zero4();
    if (s_hi >= s_lo) tile(s_hi, cur);
    stage_w0();  // (its loads overlap those of the first tile)
    for (int s2 = s_hi; s2 >= s_lo; --s2) {
      if (s2 - 1 >= s_lo) tile(s2 - 1, nxt);
      const float gs = a.seg_lg_in ? fexp2(a.seg_lg_in[bh * ln + s2]) : 0.f;
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          lam[aa][b] = lam[aa][b] * gs + cur[aa][b];
          cur[aa][b] = nxt[aa][b];
        }
    }
  }
  if (!a.seg_lam) stage_w0();
  put_rows(rows_s[0]);
  __syncthreads();
  bf16x8 wf[4];  // W0^T fragments of this wave's dx columns (k block `wave`, K block kk)
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) wf[kk] = frag_ts<kD>(L_s, o_in, kk * 32, wave * 16);
  if (wave == kGateWave) gates_f(rows_s[0][0], rows_s[0][1], rec[0], cv_of(chunk_at(0)), lane);
  for (int idx = tid; idx < kC * kC / 8; idx += kNT)
    reinterpret_cast<uint4*>(PT_s)[idx] = make_uint4(0, 0, 0, 0);
  load_rows(chunk_at(1));

  // step v: chunk v of the walk (slot), causal blocks and gates in phase A,
  // outputs in phase B, dalpha of chunk v - 1
  const auto step = [&](int v) {
    const int c = chunk_at(v);
    lds_barrier();  // B1: the previous step no longer reads the slot, L, P^T or M
    LaneOff<kD> o = o_in;
    LaneOff<kC> o64 = o64_in;
    asm volatile("" : "+v"(o.b), "+v"(o.t0), "+v"(o.t1), "+v"(o.w), "+v"(o64.b), "+v"(o64.w));
    put_chunk();
    put_rows(rows_s[(v + 1) & 1]);
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        put4<kD>(L_s, o, (4 * rh + b) * 16, (2 * kq + aa) * 16, pack4f(lam[aa][b]));
    load_chunk(chunk_at(v + 1), P0{});
    load_rows(chunk_at(v + 2));
    lds_barrier();  // B2: chunk v, Lam_out, gate rows of v + 1 visible

    // ---- phase A
    load_chunk(chunk_at(v + 1), P1{});
    const RecF& rc = rec[v & 3];
    if (c >= 0) {
      causal_f<kD>(sl.X, sl.G, sl.DY, rc, PT_s, M_s, qk[v & 1], o, o64, wave, lane);
      if (wave == 2 || wave == 3)
        causal_f<kD>(sl.X, sl.G, sl.DY, rc, PT_s, M_s, qk[v & 1], o, o64, wave + 6, lane);
      // <Lam_out, D_in> over this wave's region, then
      // Lam^T <- Gamma Lam^T + X^T (e(lq) dy),  dW0^T += X^T dy
      float c0p = 0.f;
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          c0p += dot4f(unpack4f(get4<kD>(sl.S, o, (4 * rh + b) * 16, (2 * kq + aa) * 16)),
                       lam[aa][b]);
      c0p = wave_sum(c0p);
      if (lane == 0) part[v & 1].c0[wave] = c0p;
      const float gam = rc.gam;
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int b = 0; b < 4; ++b) lam[aa][b] = lam[aa][b] * gam;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        // the per-token factor e(lq_u) goes on the x fragments (two per K
        // step) rather than on the four dy fragments: X^T (e o dy) = (e o X)^T dy
        bf16x8 xf[2], xe[2];
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(&rc.eq[kk * 32 + 8 * g4]);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(&rc.eq[kk * 32 + 8 * g4 + 4]);
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          xf[aa] = frag_ts<kD>(sl.X, o, kk * 32, (2 * kq + aa) * 16);
          xe[aa] = scale8(xf[aa], e0, e1);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bf16x8 df = frag_ts<kD>(sl.DY, o, kk * 32, (4 * rh + b) * 16);
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) {
            dw[aa][b] = mfma16x16x32(xf[aa], df, dw[aa][b]);
            lam[aa][b] = mfma16x16x32(xe[aa], df, lam[aa][b]);
          }
        }
      }
    }
    if (wave == kAlphaWave) {
      const int cp = chunk_at(v - 1);
      if (cp >= 0) {
        // dalpha and deta of the chunk finished one step ago
        const PartH& pr = part[(v - 1) & 1];
        const int ir = kC - 1 - lane;
        float c0 = 0.f, pp = 0.f, de = 0.f, rr_r = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
          c0 += pr.c0[w];
          rr_r += pr.rr[w][ir];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pp += pr.pp[w][lane];
          de += pr.de[w][lane];
        }
        const float da = dalpha_f(rec[(v - 1) & 3], qk[(v - 1) & 1], pp, rr_r, c0, lane);
        const int64_t tp = static_cast<int64_t>(cp) * kC;
        store4(buffer_rsrc(dal + tp, cv_of(cp) * 4), static_cast<uint32_t>(lane * 4), da);
        store4(buffer_rsrc(det + tp, cv_of(cp) * 4), static_cast<uint32_t>(lane * 4), de);
      }
    }
    if (wave == kGateWave) {
      // gates of the next chunk (its rows were written before B2)
      const int cn = chunk_at(v + 1);
      if (cn >= 0)
        gates_f(rows_s[(v + 1) & 1][0], rows_s[(v + 1) & 1][1], rec[(v + 1) & 3], cv_of(cn), lane);
    }
    lds_barrier();  // B3: P^T, M, the Be dots visible

    // ---- phase B: 16 columns of dx (all tokens), the 32 x 32 block (r blocks
    // 2 kq + a, token blocks 2 th + b) of u^T, th = wave / 4
    load_chunk(chunk_at(v + 1), P2{});
    const int64_t t0 = c >= 0 ? static_cast<int64_t>(c) * kC : 0;
    const int cv = cv_of(c);
    if (c >= 0) {
      PartH& pw = part[v & 1];
      const int th = rh;
      float e2v[2], nbv[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int i = (2 * th + b) * 16 + l16;
        nbv[b] = rc.nb[i];
        e2v[b] = rc.e2[i];
      }
      {
        // dx for columns 16 w .., all tokens:
        // -eta_i e(l_last - l_i) Lam_out^T g_i + W0^T dy_i + e(lq_i) D_in^T dy_i
        // + (M X)_i; rr_i = x_i . D_in^T dy_i over these 16 columns
        const __amdgpu_buffer_rsrc_t rdx = buffer_rsrc(dxp + t0 * kD * OE, cv * kD * OE);
        f32x4 acc[4], t[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) t[b] = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8 lf = frag_ts<kD>(L_s, o, kk * 32, wave * 16);
#pragma unroll
          for (int b = 0; b < 4; ++b) t[b] = mfma16x16x32(lf, frag_s<kD>(sl.G, o, b * 16, kk * 32), t[b]);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = b * 16 + l16;
          acc[b] = t[b] * (rc.nb[i] * rc.e2[i]);
          t[b] = zero4();
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8 sf = frag_ts<kD>(sl.S, o, kk * 32, wave * 16);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const bf16x8 df = frag_s<kD>(sl.DY, o, b * 16, kk * 32);
            t[b] = mfma16x16x32(sf, df, t[b]);
            acc[b] = mfma16x16x32(wf[kk], df, acc[b]);
          }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = b * 16 + l16;
          const float rp = sum_rows(dot4f(unpack4f(get4<kD>(sl.X, o, b * 16, wave * 16)), t[b]));
          if (g4 == 0) pw.rr[wave][i] = rp;
          acc[b] += t[b] * rc.eq[i];
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8 xf = frag_ts<kD>(sl.X, o, kk * 32, wave * 16);
#pragma unroll
          for (int b = 0; b < 4; ++b)
            acc[b] = mfma16x16x32(xf, frag_s<kC>(M_s, o64, b * 16, kk * 32), acc[b]);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
          store_out<F32>(rdx, static_cast<uint32_t>(((b * 16 + l16) * kD + wave * 16 + 4 * g4) * 2),
                         pack_out<F32>(acc[b]));
      }
      {
        // u = e(l_last - l_i) Lam_out x_i + sum_u P_ui dy_u for rows 32 kq ..: dg,
        // and the deta, pp shares over these 32 rows
        const __amdgpu_buffer_rsrc_t rdg = buffer_rsrc(dgp + t0 * kD * OE, cv * kD * OE);
        f32x4 ain[2][2], apd[2][2];
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            ain[aa][b] = zero4();
            apd[aa][b] = zero4();
          }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          __builtin_amdgcn_sched_barrier(0);
          bf16x8 lf[2], xf[2];
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) lf[aa] = frag_s<kD>(L_s, o, (2 * kq + aa) * 16, kk * 32);
#pragma unroll
          for (int b = 0; b < 2; ++b) xf[b] = frag_s<kD>(sl.X, o, (2 * th + b) * 16, kk * 32);
#pragma unroll
          for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int b = 0; b < 2; ++b) ain[aa][b] = mfma16x16x32(lf[aa], xf[b], ain[aa][b]);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          __builtin_amdgcn_sched_barrier(0);
          bf16x8 tf[2], pf[2];
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) tf[aa] = frag_ts<kD>(sl.DY, o, kk * 32, (2 * kq + aa) * 16);
#pragma unroll
          for (int b = 0; b < 2; ++b) pf[b] = frag_s<kC>(PT_s, o64, (2 * th + b) * 16, kk * 32);
#pragma unroll
          for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int b = 0; b < 2; ++b) apd[aa][b] = mfma16x16x32(tf[aa], pf[b], apd[aa][b]);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int i = (2 * th + b) * 16 + l16;
          float dp = 0.f, pp = 0.f;
#pragma unroll
          for (int aa = 0; aa < 2; ++aa) {
            const f32x4 u = ain[aa][b] * e2v[b] + apd[aa][b];
            const f32x4 gv = unpack4f(get4<kD>(sl.G, o, (2 * th + b) * 16, (2 * kq + aa) * 16));
            dp += dot4f(gv, u);
            pp += dot4f(gv, ain[aa][b]);
            store_out<F32>(rdg, static_cast<uint32_t>((i * kD + (2 * kq + aa) * 16 + 4 * g4) * 2),
                           pack_out<F32>(u * nbv[b]));
          }
          dp = sum_rows(dp);
          pp = sum_rows(pp);
          if (g4 == 0) {
            pw.de[kq][i] = -dp;
            pw.pp[kq][i] = pp;
          }
        }
      }
    }
  };
  for (int v = 0; v <= nloc; ++v) step(v);
  // dW0 partial of this (segment, sequence-head): dW0[r][k], fp32
  float* pw = static_cast<float*>(a.part_dW0) + (static_cast<int64_t>(seg) * BH + bh) * kD * kD;
#pragma unroll
  for (int aa = 0; aa < 2; ++aa)
#pragma unroll
    for (int b = 0; b < 4; ++b)
      *reinterpret_cast<f32x4*>(pw + ((4 * rh + b) * 16 + l16) * kD + (2 * kq + aa) * 16 + 4 * g4) =
          dw[aa][b];
}

}  // namespace

hipError_t launch_mfma_bwd_f128(const BwdArgs& a, hipStream_t s) {
  const int64_t groups = a.B * a.H * a.n_seg;
  if (groups == 0) return hipSuccess;
  if (a.out_f32)
    hipLaunchKernelGGL(bwd_f128<true>, dim3(static_cast<unsigned>(groups)), dim3(kNT), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_f128<false>, dim3(static_cast<unsigned>(groups)), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace gls
