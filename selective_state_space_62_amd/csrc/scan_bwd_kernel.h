// Backward pass of the selective scan (ss_scan_bwd) for gfx950: the main kernel
// template and its launch dispatch, instantiated by scan_bwd.hip (first-order
// input term) and scan_bwd_zoh.hip (zero-order hold).
//
// Training runs the scan forward and then backward.  In the pages' design the
// expanded state is never saved for the gradient: the backward derives it again
// from the inputs (reader's notes, kurisu.si, "What they did", Selective SSM
// item).  The gradients are those of the forward definition
//   Delta_t = softplus(dt_t + dt_bias),  Abar = exp(Delta_t A_n),
//   h_t[n] = Abar h_(t-1)[n] + Delta_t B_t[n] x_t,
//   y_t = r_t silu(z_t),  r_t = C_t . h_t + Dskip x_t,
// taken in reverse token order with the adjoint state lam_t = dLoss/dh_t:
//   dr_t = dy_t silu(z_t),  dz_t = dy_t r_t silu'(z_t),
//   lam_t = Abar_(t+1) lam_(t+1) + dr_t C_t  (lam_L = dh_final),
//   dC_t[n] += dr_t h_t[n],  dB_t[n] += lam_t[n] Delta_t x_t   (summed over channels),
//   with dAbar = lam_t h_(t-1):  dDelta += dAbar Abar A,  dA += dAbar Abar Delta,
//   dDelta += x_t sum_n lam_t[n] B_t[n],  dx_t = Delta_t sum_n lam_t[n] B_t[n] + dr_t Dskip,
//   ddt_t = dDelta sigmoid(dt_t + dt_bias),  dh0 = Abar_0 lam_0.
//
// One workgroup owns 64/K channels of one batch row, laid out like the forward
// kernel: G waves, K adjacent lanes per channel, each lane NS = N/(G K) state
// components.  Work goes in chunks of CK = 2 G K tokens; each lane owns 2 tokens
// of a chunk for the per-(token, channel) work (Delta, the gate, dx, ddt, dz).
//  1. A forward sweep over the sequence stores the state at every chunk start
//     (the checkpoints, in the workspace).
//  2. Chunks are then visited last to first.  The chunk's states (and their
//     decay factors Abar) are recomputed from its checkpoint into registers, with
//     the readout (dz needs r_t); the owner of each token forms dr and dz; then
//     every lane runs the adjoint state back through the chunk, reusing the
//     recomputed Abar.  The sums over state components (for dx and dDelta) reach
//     the token's owner through LDS, as the forward's readout does.
// dB and dC are sums over channels.  Every wave holds all of the workgroup's
// channels (for its own state components), so a wave forms the workgroup's sums
// by itself: a swap of wave halves between two registers (v_permlane32_swap)
// and an add, a swap of row pairs (v_permlane16_swap) and an add, then DPP adds
// within the 16-lane rows.  A chunk's sums stay in registers and are written
// to the workspace, one partial per (workgroup, output, token), each chunk's
// outputs in one contiguous block (token fastest); bwd_reduce_bc_kernel adds a
// batch row's partials in a fixed order.  dA, dDskip and dt_bias's gradient
// are summed per (segment, row, channel) in registers and over segments and
// rows by bwd_reduce_param_kernel.  All sums have a fixed order:
// results are deterministic.  The next chunk's global operands are fetched while
// the current one computes, and whole chunks run without per-token guards.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ssscan {
namespace bwd_detail {

using namespace dev;

constexpr int kSpan = 2;   // tokens of a chunk owned per lane

// Workgroup index -> logical block so that the channel blocks of one batch row
// share an XCD (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int64_t bwd_logical_block(int64_t wg, int64_t nwg) {
  if ((nwg & 7) != 0) return wg;
  return (wg & 7) * (nwg >> 3) + (wg >> 3);
}

// sigmoid(v) given v2 = v log2(e); 0 when e^-v overflows
__device__ __forceinline__ float sigmoid2(float v2) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v2));
}

// dB and dC of one token summed over the channels of a wave (lane = K c + hk):
// the result in row r (16 lanes) is, for NS == 2, dB[0], dC[0], dB[1], dC[1] for
// r = 0..3, and for NS == 1, dB, dB, dC, dC; within a row, lanes with the same
// hk (lane mod K) hold the same sum.  The order of the additions is fixed.
template <int NS, int K>
__device__ __forceinline__ float bc_channel_sum(const float (&dB)[NS], const float (&dC)[NS]) {
  static_assert(NS == 1 || NS == 2, "one or two state components per lane");
  auto swap32 = [](float a, float b) {   // ([a lower half, b lower half], [a upper half, b upper half])
    return __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  };
  auto swap16 = [](float a, float b) {   // ([a r0, b r0, a r2, b r2], [a r1, b r1, a r3, b r3])
    return __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  };
  float u;
  if constexpr (NS == 2) {
    const auto pb = swap32(dB[0], dB[1]);
    const auto pc = swap32(dC[0], dC[1]);
    const float sb = __uint_as_float(pb[0]) + __uint_as_float(pb[1]);   // lower half dB[0], upper dB[1]
    const float sc = __uint_as_float(pc[0]) + __uint_as_float(pc[1]);
    const auto q = swap16(sb, sc);
    u = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  } else {
    const auto pv = swap32(dB[0], dC[0]);
    const float sv = __uint_as_float(pv[0]) + __uint_as_float(pv[1]);   // lower half dB, upper dC
    const auto q = swap16(sv, sv);
    u = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  }
  u += __builtin_amdgcn_update_dpp(0.0f, u, 0x128, 0xf, 0xf, false);   // row_ror:8
  u += __builtin_amdgcn_update_dpp(0.0f, u, 0x124, 0xf, 0xf, false);   // row_ror:4
  u += __builtin_amdgcn_update_dpp(0.0f, u, 0x4E, 0xf, 0xf, false);    // lanes 2 apart
  if constexpr (K == 1) u += __builtin_amdgcn_update_dpp(0.0f, u, 0xB1, 0xf, 0xf, false);   // neighbours
  // formed by every lane here: only some lanes store the sums, and an add sunk
  // into their branch would split the last DPP add into three instructions
  __asm__ volatile("" : "+v"(u));
  return u;
}

// psi(u) = (u e^u - e^u + 1) / u^2: the zero-order-hold input coefficient
// c = (e^(Delta A) - 1) / A has dc/dA = Delta^2 psi(Delta A).  Takes u2 = u
// log2(e) and E = e^u.  |u| < 1: the series sum_k (k + 1) u^k / (k + 2)! to
// degree 9 (the first dropped term is below 1e-7 relative); otherwise
// ((u - 1) E + 1) / u^2 with one fma, whose rounding is ~1e-7 / u^2 relative.
__device__ __forceinline__ float zoh_psi(float u2, float E) {
  const float u = u2 * kLn2;
  float p = fmaf(u, 1.0f / 3991680.0f, 1.0f / 403200.0f);
  p = fmaf(p, u, 1.0f / 45360.0f);
  p = fmaf(p, u, 1.0f / 5760.0f);
  p = fmaf(p, u, 1.0f / 840.0f);
  p = fmaf(p, u, 1.0f / 144.0f);
  p = fmaf(p, u, 1.0f / 30.0f);
  p = fmaf(p, u, 1.0f / 8.0f);
  p = fmaf(p, u, 1.0f / 3.0f);
  p = fmaf(p, u, 0.5f);
  const float q = fmaf(u - 1.0f, E, 1.0f) * __builtin_amdgcn_rcpf(u * u);
  return fabsf(u) < 1.0f ? p : q;
}

// Three waves per SIMD at N = 16 (about 160 VGPRs); at most 32 KB of LDS.
// ZOH: the zero-order-hold input term, c = Delta phi(Delta A) in place of Delta.
// VEC: every row's lane spans are aligned for one vector access (an even
// length).  It is a template parameter so that the chunk loop has no runtime
// choice between a vector load and element loads: with one, the compiler cannot
// count the memory operations in flight and waits for all of them (the previous
// chunk's stores included) before using the next chunk's operands.
// SIN: the reverse pass's operands go through LDS in whole row pieces (bf16,
// first order, rows a multiple of 8 tokens; see s_in below).
template <int N, int G, int K, typename IO, bool ZOH, bool VEC, bool SIN>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(3, 10))) void scan_bwd_kernel(
    const BwdDims dm, const BwdPtrs p) {
  using T = typename IO::T;
  // per token and channel in LDS: (Delta, Delta x), and for ZOH also (x, x Delta^2)
  using DD = std::conditional_t<ZOH, float4, float2>;
  constexpr int CPB = 64 / K;          // channels per workgroup
  constexpr int SG = G * K;            // state groups
  constexpr int NS = N / SG;           // state components per lane
  constexpr int CK = kSpan * SG;       // chunk length (tokens)
  constexpr int NOUT = 2 * N;          // dB and dC values per token
  constexpr int NPART = bwd_part_outputs(N);   // partial outputs: dB, dC, then the per-row ddt
  constexpr int THREADS = 64 * G;
  constexpr int SW = SpanT<IO, kSpan>::kWords;
  static_assert(NS >= 1 && N % SG == 0, "G * K must divide N");
  static_assert(K == 1 || K == 2, "one or two lanes per channel");
  static_assert(CK * N <= THREADS, "one B/C piece per thread");
  static_assert(CK == bwd_chunk_tokens(N), "the chunk length the forward's checkpoints assume");

  __shared__ DD s_dd[CK][CPB];         // (Delta, Delta x[, x, x Delta^2]) per token and channel
  __shared__ float s_bc[CK][2 * N];    // B_n, C_n of the chunk's tokens
  __shared__ float2 s_pp[CK][G][CPB];  // per-wave partial sums (readout; dDelta and sum lam B)
  __shared__ float s_dr[CK][CPB];      // dr per token and channel
  // dx, ddt and dz are gathered in LDS over the 128 bytes of a row that one
  // cache line holds (64 bf16 or 32 fp32 tokens, several chunks) and written as
  // whole lines once the group's lowest chunk is done (chunks run last to
  // first): a lane's own 4 or 8 bytes per row and chunk, stored directly, reach
  // HBM as partial lines.  Rows are padded to 34 words so that the owners'
  // writes fall in distinct banks.  The zero-order-hold form keeps direct
  // stores: it runs four workgroups per CU, which the extra 13 KB would not fit.
  constexpr bool STAGE = !ZOH;
  constexpr int GT = 128 / (int)sizeof(T);   // tokens per staged group
  constexpr int ROWW = 128 / 4 + 2;          // words per staged row
  static_assert(GT % CK == 0 && kSpan == 2, "a group holds whole chunks; a lane owns two tokens");
  __shared__ __attribute__((aligned(16))) uint32_t s_out[STAGE ? 3 : 1][STAGE ? CPB : 1][ROWW];
  // With SIN the reverse pass's operand rows (x, dt, z, dy) go through LDS as
  // well, in 16-byte row spans: each wave loads the chunk's 32 bytes of 8 rows
  // of all four operands (two lanes per row and operand), so a row's piece is
  // requested once per chunk instead of a quarter by each wave.  When a
  // workgroup's rows share their offset within the memory pages (rows of
  // 2^20 bf16 tokens lie 2 MB apart), the vector L1 loses the line between
  // the waves' requests and every quarter went to L2.  Chunk k's pieces sit in
  // buffer k & 1, written at the end of chunk k + 1.  Rows are padded to 10
  // words so that the owners' 4-byte reads fall in distinct banks.
  constexpr bool STAGE_IN = SIN;
  static_assert(!SIN || (STAGE && sizeof(T) == 2 && VEC && G == 4 && K == 2 && CK == 16),
                "whole-piece loads: bf16 first order, 4 waves of 32 channels, 16-token chunks");
  constexpr int IN_ROWW = CK * (int)sizeof(T) / 4 + 2;
  __shared__ __attribute__((aligned(16))) uint32_t s_in[STAGE_IN ? 2 : 1][STAGE_IN ? 4 : 1][STAGE_IN ? CPB : 1]
                                                       [STAGE_IN ? IN_ROWW : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int c = lane / K;
  const int hk = lane % K;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sg = w * K + hk;

  // logical block -> (segment, batch row, channel block), channel block fastest
  const int64_t nwg = dm.cblocks * dm.batch * dm.nseg;
  const int64_t lb = bwd_logical_block(blockIdx.x, nwg);
  const int64_t cb = lb % dm.cblocks;
  const int64_t b = (lb / dm.cblocks) % dm.batch;
  const int64_t seg = lb / (dm.cblocks * dm.batch);
  const int64_t d = cb * CPB + c;
  const bool act = d < dm.dim;
  const int64_t dc = act ? d : dm.dim - 1;   // inactive lanes run a valid row with zero gradients
  const int64_t L = dm.seqlen;
  const int64_t ch = b * dm.dim + dc;
  const int64_t row = ch * L;
  const int64_t dt_row = dm.dt_row ? b * L : row;   // dt per (row, token) is shared by the row's channels
  constexpr bool vec = VEC;
  const bool has_z = p.z != nullptr;
  const int64_t nck = (L + CK - 1) / CK;   // chunks of the whole sequence
  // this workgroup's chunks [kb, ke): its segment of the sequence
  const int64_t kb = seg * dm.seg_len / CK;
  const int64_t ke = (seg + 1) * dm.seg_len / CK < nck ? (seg + 1) * dm.seg_len / CK : nck;
  const int64_t kfull = ke < L / CK ? ke : L / CK;   // chunks below kfull lie wholly inside the sequence

  const T* __restrict__ x = static_cast<const T*>(p.x);
  const T* __restrict__ dt = static_cast<const T*>(p.dt);
  const T* __restrict__ z = static_cast<const T*>(p.z);
  const T* __restrict__ dy = static_cast<const T*>(p.dy);

  float A2[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) A2[s] = p.A[dc * N + sg * NS + s] * kLog2e;
  // Zero-order hold: the input coefficient c = Delta phi(Delta A) from zoh_coef,
  // as in the forward: (E - 1)/A from the E = e^(Delta A) at hand where
  // |Delta A| >= 1/20, a Taylor polynomial below (A = 0 included), with no
  // reciprocal per element; dc/dA = Delta^2 psi(Delta A) keeps its series and
  // closed form (its closed form in terms of c cancels digits for small
  // Delta A).
  float inv_a[ZOH ? NS : 1];
  if constexpr (ZOH) {
#pragma unroll
    for (int s = 0; s < NS; ++s) inv_a[s] = 1.0f / p.A[dc * N + sg * NS + s];
  }
  // the zero-order-hold input term c x B, with the forward's operations; o is
  // the token's (Delta, Delta x, x, x Delta^2)
  auto zoh_in = [&](int s, float u2, float E, float Bv, const auto& o) {
    return zoh_coef(u2, E, o.x, inv_a[ZOH ? s : 0]) * (o.z * Bv);
  };
  const float bias2 = p.dt_bias ? p.dt_bias[dc] * kLog2e : 0.0f;
  const float skip = p.Dskip ? p.Dskip[dc] : 0.0f;
  const float* __restrict__ bc_row = p.bc + b * L * (2 * N);
  // checkpoints (batch, chunk, dim, N): a workgroup's channels are contiguous per chunk
  float* __restrict__ ck_row = p.ckpt + (b * nck * dm.dim + dc) * N + sg * NS;
  const int64_t ck_stride = dm.dim * N;

  const int j_own = sg * kSpan;   // first token of a chunk this lane owns
  auto chunk_end = [&](int64_t k) { return (k * CK + CK < L) ? k * CK + CK : L; };
  auto own_valid = [&](int64_t k) {
    const int64_t v = chunk_end(k) - (k * CK + j_own);
    return (int)(v < 0 ? 0 : (v < kSpan ? v : kSpan));
  };

  // A chunk's global operands, fetched one chunk ahead of their use.  WHOLE (a
  // compile-time tag): every token of chunk k lies inside the sequence, so the
  // loads need no per-lane bounds.
  struct Fetch {
    uint32_t x[SW], dt[SW], z[SW], dy[SW];
    float2 bc;
  };
  auto fetch = [&](auto whole_tag, int64_t k, bool grads, Fetch& f) {
    constexpr bool WHOLE = decltype(whole_tag)::value;
    const int64_t t0 = k * CK;
    const int valid = WHOLE ? kSpan : own_valid(k);
    load_span<IO, kSpan>(x, row + t0 + j_own, valid, vec, f.x);
    load_span<IO, kSpan>(dt, dt_row + t0 + j_own, valid, vec, f.dt);
    if (grads) {
      // without z, x stands in (its values are never used): no branch around the load
      load_span<IO, kSpan>(has_z ? z : x, row + t0 + j_own, valid, vec, f.z);
      load_span<IO, kSpan>(dy, row + t0 + j_own, valid, vec, f.dy);
    }
    f.bc = make_float2(0.0f, 0.0f);
    if ((CK * N >= THREADS || tid < CK * N) && (WHOLE || t0 + tid / N < chunk_end(k)))
      f.bc = reinterpret_cast<const float2*>(bc_row + t0 * (2 * N))[tid];
  };
  // The reverse pass's loader lanes: operand in_a (x, dt, z, dy), row in_r of
  // the block, 16-byte half in_h of the row's chunk piece
  struct FetchIn {
    uint32_t v[4];
    float2 bc;
  };
  const int in_a = lane >> 4;
  const int in_r = w * 8 + ((lane >> 1) & 7);
  const int in_h = lane & 1;
  const int64_t in_d = cb * CPB + in_r;
  const int64_t in_row = (b * dm.dim + (in_d < dm.dim ? in_d : dm.dim - 1)) * L;   // clamped like dc
  const T* __restrict__ in_src = in_a == 0 ? x : (in_a == 1 ? dt : (in_a == 2 ? (has_z ? z : x) : dy));
  const int64_t in_base = (in_a == 1 && dm.dt_row ? b * L : in_row) + in_h * 8;
  auto fetch_in = [&](auto whole_tag, int64_t k, FetchIn& f) {
    constexpr bool WHOLE = decltype(whole_tag)::value;
    const int64_t t0 = k * CK;
    int valid = 8;
    if constexpr (!WHOLE) {
      const int64_t v = chunk_end(k) - (t0 + in_h * 8);
      valid = v < 0 ? 0 : (v < 8 ? (int)v : 8);
    }
    if constexpr (STAGE_IN) load_span<IO, 8>(in_src, in_base + t0, valid, true, f.v);
    f.bc = make_float2(0.0f, 0.0f);
    if ((CK * N >= THREADS || tid < CK * N) && (WHOLE || t0 + tid / N < chunk_end(k)))
      f.bc = reinterpret_cast<const float2*>(bc_row + t0 * (2 * N))[tid];
  };
  // a fetched chunk into LDS buffer bi, with its B and C
  auto put_in = [&](int bi, const FetchIn& f) {
    uint32_t* dst = &s_in[STAGE_IN ? bi : 0][STAGE_IN ? in_a : 0][STAGE_IN ? in_r : 0][STAGE_IN ? in_h * 4 : 0];
    if constexpr (STAGE_IN) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(f.v[0], f.v[1]);
      *reinterpret_cast<uint2*>(dst + 2) = make_uint2(f.v[2], f.v[3]);
    }
    if (CK * N >= THREADS || tid < CK * N) reinterpret_cast<float2*>(&s_bc[0][0])[tid] = f.bc;
  };
  // operand o (0 x, 1 dt, 2 z, 3 dy) of this lane's two owned tokens from buffer bi
  auto in_word = [&](int bi, int o) -> uint32_t {
    return s_in[STAGE_IN ? bi : 0][STAGE_IN ? o : 0][STAGE_IN ? c : 0][STAGE_IN ? j_own >> 1 : 0];
  };

  // Delta and Delta x of the owned tokens into LDS (zero Delta for padding
  // tokens), and the chunk's B and C
  auto stage = [&](int valid, const Fetch& f, float (&xv)[kSpan], float (&dl)[kSpan], float (&v2)[kSpan]) {
#pragma unroll
    for (int i = 0; i < kSpan; ++i) {
      xv[i] = span_elem<IO>(f.x, i);
      v2[i] = fmaf(span_elem<IO>(f.dt, i), kLog2e, bias2);
      dl[i] = (i < valid) ? softplus_dt(span_elem<IO>(f.dt, i), bias2) : 0.0f;
      if constexpr (ZOH) s_dd[j_own + i][c] = make_float4(dl[i], dl[i] * xv[i], xv[i], dl[i] * dl[i] * xv[i]);
      else s_dd[j_own + i][c] = make_float2(dl[i], dl[i] * xv[i]);
    }
    if (CK * N >= THREADS || tid < CK * N) reinterpret_cast<float2*>(&s_bc[0][0])[tid] = f.bc;
  };

  // ---- 1. forward sweep: the state at every chunk start (unless the forward
  // pass already stored them) ----
  if (!dm.have_ckpt) {
    float h[NS];
    // the state entering the segment: h0 for the first, else from the segments' combine
    const float* hs0 = seg > 0 ? p.h_seg + (ch * dm.nseg + seg) * N : (p.h0 ? p.h0 + ch * N : nullptr);
#pragma unroll
    for (int s = 0; s < NS; ++s) h[s] = hs0 ? hs0[sg * NS + s] : 0.0f;
    Fetch f;
    if (kb < kfull) fetch(std::true_type{}, kb, false, f);
    else fetch(std::false_type{}, kb, false, f);
    // FULL (a compile-time tag): all CK tokens of the chunk lie inside the sequence
    auto sweep = [&](auto full_tag, int64_t k) {
      constexpr bool FULL = decltype(full_tag)::value;
      if (act) {
#pragma unroll
        for (int s = 0; s < NS; ++s) ck_row[k * ck_stride + s] = h[s];
      }
      float xv[kSpan], dl[kSpan], v2[kSpan];
      stage(FULL ? kSpan : own_valid(k), f, xv, dl, v2);
      if (k + 1 < kfull) fetch(std::true_type{}, k + 1, false, f);
      else if (k + 1 < ke) fetch(std::false_type{}, k + 1, false, f);
      __syncthreads();
      const int nj = FULL ? CK : (int)(chunk_end(k) - k * CK);
#pragma unroll
      for (int j = 0; j < CK; ++j) {
        if (FULL || j < nj) {
          const DD o = s_dd[j][c];
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            float u2 = o.x * A2[s];
            if constexpr (ZOH) __asm__ volatile("" : "+v"(u2) : "v"(h[s]));   // token by token (registers)
            const float E = __builtin_amdgcn_exp2f(u2);
            float in;
            if constexpr (ZOH) in = zoh_in(s, u2, E, s_bc[j][2 * (sg * NS + s)], o);
            else in = o.y * s_bc[j][2 * (sg * NS + s)];
            h[s] = fmaf(E, h[s], in);
          }
        }
      }
      __syncthreads();
    };
    for (int64_t k = kb; k < kfull; ++k) sweep(std::true_type{}, k);
    if (kfull < ke) sweep(std::false_type{}, kfull);
  }

  // ---- 2. chunks last to first ----
  float lam[NS], dAacc[NS];
  // the adjoint carried in from the tokens after the segment: dh_final for the
  // last, else from the segments' combine
  const float* lam0 = p.lam_seg ? p.lam_seg + (ch * dm.nseg + seg) * N : (p.dh_final ? p.dh_final + ch * N : nullptr);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    lam[s] = (act && lam0) ? lam0[sg * NS + s] : 0.0f;
    dAacc[s] = 0.0f;
  }
  float dD_acc = 0.0f, dbias_acc = 0.0f;
  // dB/dC partials (batch, channel block, output, token), tokens padded to whole chunks
  // dB/dC partials (batch, channel block, chunk, output, chunk token): a chunk's
  // outputs are contiguous, one block per chunk
  float* __restrict__ part_blk = p.part + (b * dm.cblocks + cb) * nck * (NPART * CK);
  // the lanes that write them: the first K lanes of each row that holds a sum (all
  // rows for NS == 2, rows 0 and 2 for NS == 1), and the output each one writes.
  // The sums cover the whole workgroup (channels past dim add zeros), so a
  // writing lane writes whether or not its own channel is active.
  const int prow = lane >> 4;
  const bool pw = (lane & 15) < K && (NS == 2 || (prow & 1) == 0);
  const int pwhich = NS == 2 ? (prow & 1) : (prow >> 1);   // 0: dB, 1: dC
  const int ps = NS == 2 ? (prow >> 1) : 0;
  // this lane's first partial within a chunk's block (bytes)
  const uint32_t pofs = (uint32_t)((pwhich * N + sg * NS + ps) * CK * 4);

  Fetch f;
  FetchIn fi;
  if constexpr (STAGE_IN) {
    if (ke == kfull) fetch_in(std::true_type{}, ke - 1, fi);
    else fetch_in(std::false_type{}, ke - 1, fi);
    put_in((int)((ke - 1) & 1), fi);
    __syncthreads();
  } else {
    if (ke == kfull) fetch(std::true_type{}, ke - 1, true, f);
    else fetch(std::false_type{}, ke - 1, true, f);
  }
  float ckn[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) ckn[s] = act ? ck_row[(ke - 1) * ck_stride + s] : 0.0f;

  // the owned tokens' values of output o (0 dx, 1 ddt, 2 dz) into the staged
  // group of chunk k
  auto stage_out = [&](int o, int64_t k, const float (&v)[kSpan]) {
    const int tg = (int)(k * CK % GT) + j_own;   // even: a lane owns a token pair
    if constexpr (sizeof(T) == 2) {
      s_out[o][c][tg >> 1] = pack_bf16x2(v[0], v[1]);
    } else {
      *reinterpret_cast<uint2*>(&s_out[o][c][tg]) = make_uint2(__float_as_uint(v[0]), __float_as_uint(v[1]));
    }
  };
  // The staged group starting at token g0 (a multiple of GT) to HBM, one
  // 16-byte piece of a row per thread and step; rows past dim and tokens past
  // the sequence are not written.  Whole pieces of 16-byte aligned rows go out
  // as one vector store.
  auto flush_out = [&](int64_t g0) {
    constexpr int EPP = 16 / (int)sizeof(T);   // elements per piece
    const int64_t gend = (g0 + GT < L) ? g0 + GT : L;
#pragma unroll
    for (int o = 0; o < 3; ++o) {
      if ((o == 1 && dm.dt_row) || (o == 2 && !has_z)) continue;
      T* __restrict__ dst = static_cast<T*>(o == 0 ? p.dx : (o == 1 ? p.ddt : p.dz));
      const bool al16 = (L * (int64_t)sizeof(T)) % 16 == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
#pragma unroll
      for (int pc = tid; pc < CPB * 8; pc += THREADS) {
        const int r = pc >> 3, q = pc & 7;
        const int64_t dr_ = cb * CPB + r;
        const int64_t t = g0 + q * EPP;
        if (dr_ >= dm.dim || t >= gend) continue;
        const uint2 lo = *reinterpret_cast<const uint2*>(&s_out[o][r][q * 4]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&s_out[o][r][q * 4 + 2]);
        T* const out = dst + (b * dm.dim + dr_) * L + t;
        if (al16 && t + EPP <= gend) {
          *reinterpret_cast<uint4*>(out) = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
          const uint32_t wd[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int e = 0; e < EPP; ++e) {
            if (t + e < gend) {
              if constexpr (sizeof(T) == 2) out[e] = (T)(wd[e >> 1] >> (16 * (e & 1)));
              else out[e] = __uint_as_float(wd[e]);
            }
          }
        }
      }
    }
  };

  auto chunk = [&](auto full_tag, int64_t k) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int64_t t0 = k * CK;
    // the chunk's block of dB/dC partials (NPART outputs x CK tokens, fp32)
    const __amdgpu_buffer_rsrc_t rs_part = make_rsrc(part_blk + k * (NPART * CK), NPART * CK * 4);
    const int64_t t1 = chunk_end(k);
    const int nj = FULL ? CK : (int)(t1 - t0);
    const int64_t tf = t0 + j_own;
    const int valid = FULL ? kSpan : own_valid(k);
    float xv[kSpan], dl[kSpan], v2[kSpan];
    // z and dy of the owned tokens stay raw until the owners use them
    uint32_t cz[SW], cdy[SW];
    const int bi = (int)(k & 1);
    if constexpr (STAGE_IN) {
      const uint32_t xw[1] = {in_word(bi, 0)}, dw[1] = {in_word(bi, 1)};
#pragma unroll
      for (int i = 0; i < kSpan; ++i) {
        xv[i] = span_elem<IO>(xw, i);
        const float dtv = span_elem<IO>(dw, i);
        v2[i] = fmaf(dtv, kLog2e, bias2);
        dl[i] = (i < valid) ? softplus_dt(dtv, bias2) : 0.0f;
        s_dd[j_own + i][c] = make_float2(dl[i], dl[i] * xv[i]);
      }
    } else {
      stage(valid, f, xv, dl, v2);
#pragma unroll
      for (int q = 0; q < SW; ++q) {
        cz[q] = f.z[q];
        cdy[q] = f.dy[q];
      }
    }
    float hs[CK + 1][NS];   // hs[j] = the state before chunk token j
    // Es[j] = Abar of chunk token j, kept for the adjoint step (first order; the
    // zero-order-hold form needs the registers for phi and psi and recomputes it)
    float Es[ZOH ? 1 : CK][NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) hs[0][s] = ckn[s];
    if (k > kb) {
      // every chunk before the last is whole
      if constexpr (STAGE_IN) fetch_in(std::true_type{}, k - 1, fi);
      else fetch(std::true_type{}, k - 1, true, f);
#pragma unroll
      // inactive lanes read their clamped (valid) row: an unmasked load, whose
      // values give them finite states and, with their zero dy, zero gradients
      for (int s = 0; s < NS; ++s) ckn[s] = ck_row[(k - 1) * ck_stride + s];
    }
    __syncthreads();

    // recompute the chunk's states, with the readout
#pragma unroll
    for (int j = 0; j < CK; ++j) {
      if (FULL || j < nj) {
        const DD o = s_dd[j][c];
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          float u2 = o.x * A2[s];
          if constexpr (ZOH) __asm__ volatile("" : "+v"(u2) : "v"(hs[j][s]));   // token by token (registers)
          const float E = __builtin_amdgcn_exp2f(u2);
          if constexpr (!ZOH) Es[j][s] = E;
          float in;
          if constexpr (ZOH) in = zoh_in(s, u2, E, s_bc[j][2 * (sg * NS + s)], o);
          else in = o.y * s_bc[j][2 * (sg * NS + s)];
          hs[j + 1][s] = fmaf(E, hs[j][s], in);
          acc = fmaf(s_bc[j][2 * (sg * NS + s) + 1], hs[j + 1][s], acc);
        }
        if constexpr (K == 2) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0xB1, 0xf, 0xf, false);
        s_pp[j][w][c].x = acc;   // both lanes of a channel hold the sum and store it
      }
    }
    __syncthreads();

    // owners: r, dr = dy silu(z), dz = dy r silu'(z)
    {
      float dzv[kSpan];
#pragma unroll
      for (int i = 0; i < kSpan; ++i) {
        const int j = j_own + i;
        float r = 0.0f;
        if (FULL || i < valid) {
#pragma unroll
          for (int g = 0; g < G; ++g) r += s_pp[j][g][c].x;
        }
        r = fmaf(skip, xv[i], r);
        if constexpr (STAGE_IN) {
          cdy[0] = in_word(bi, 3);
          cz[0] = in_word(bi, 2);
        }
        const float dyv = act ? span_elem<IO>(cdy, i) : 0.0f;   // padding tokens load as zero
        float gate = 1.0f;
        dzv[i] = 0.0f;
        if (has_z) {
          const float zv = span_elem<IO>(cz, i);
          const float sz = sigmoid2(zv * kLog2e);
          gate = zv * sz;
          dzv[i] = dyv * r * (sz * fmaf(zv, 1.0f - sz, 1.0f));
        }
        const float drv = dyv * gate;
        dD_acc = fmaf(drv, xv[i], dD_acc);
        s_dr[j][c] = drv;
      }
      if constexpr (STAGE) {
        if (has_z) stage_out(2, k, dzv);
      } else {
        if (has_z && act && (FULL || valid > 0)) store_span<IO, kSpan>(static_cast<T*>(p.dz), row + tf, valid, vec, dzv);
      }
    }
    __syncthreads();

    // the adjoint state back through the chunk, at a raised wave priority
    // (back to the default for the owners' phase): a SIMD's issue then favours
    // the waves in this, the longest phase (about 4% faster at the 2.8B shape)
    __builtin_amdgcn_s_setprio(2);
    float uo[CK];   // this lane's dB/dC sum per chunk token (kept by the writing lanes)
#pragma unroll
    for (int j = 0; j < CK; ++j) uo[j] = 0.0f;
#pragma unroll
    for (int j = CK - 1; j >= 0; --j) {
      if (FULL || j < nj) {
        const float dr = s_dr[j][c];
        const DD o = s_dd[j][c];
        float ddp = 0.0f, sB = 0.0f;   // first order: ddp in units of A log2(e), scaled by ln 2 by the owner
        float sE = 0.0f;               // ZOH: sum lam e^u B, the input term's dDelta factor
        float dBv[NS], dCv[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const float Bv = s_bc[j][2 * (sg * NS + s)];
          const float Cv = s_bc[j][2 * (sg * NS + s) + 1];
          lam[s] = fmaf(dr, Cv, lam[s]);
          dCv[s] = dr * hs[j + 1][s];
          float u2 = o.x * A2[s];
          if constexpr (ZOH) __asm__ volatile("" : "+v"(u2) : "v"(lam[s]));   // token by token (registers)
          const float E = ZOH ? __builtin_amdgcn_exp2f(u2) : Es[ZOH ? 0 : j][s];
          const float lamE = lam[s] * E;   // the next token's adjoint before its dr C term
          const float ga = lamE * hs[j][s];
          ddp = fmaf(ga, A2[s], ddp);
          dAacc[s] = fmaf(ga, o.x, dAacc[s]);
          if constexpr (ZOH) {
            // c = Delta phi: dx and dB carry c; dc/dDelta = e^u; dc/dA = Delta^2 psi.
            // lp = lam c: sB holds sum lam c B (dx needs no further Delta), and
            // dB = lam c x
            const float lp = lam[s] * zoh_coef(u2, E, o.x, inv_a[ZOH ? s : 0]);
            const float lB = lam[s] * Bv;
            sB = fmaf(lp, Bv, sB);
            dBv[s] = lp * o.z;
            sE = fmaf(lB, E, sE);
            dAacc[s] = fmaf(lB, o.w * zoh_psi(u2, E), dAacc[s]);
            // keep the update here: sunk to the end of the chunk, it would hold
            // every token's u and Abar in registers until then
            __asm__ volatile("" : "+v"(dAacc[s]));
          } else {
            sB = fmaf(lam[s], Bv, sB);
            dBv[s] = lam[s] * o.y;
          }
          lam[s] = lamE;
        }
        if constexpr (ZOH) ddp = fmaf(ddp, kLn2, o.z * sE);   // the whole dDelta, in natural units
        if constexpr (K == 2) {
          ddp += __builtin_amdgcn_update_dpp(0.0f, ddp, 0xB1, 0xf, 0xf, false);
          sB += __builtin_amdgcn_update_dpp(0.0f, sB, 0xB1, 0xf, 0xf, false);
        }
        s_pp[j][w][c] = make_float2(ddp, sB);   // both lanes of a channel hold the sums
        uo[j] = bc_channel_sum<NS, K>(dBv, dCv);
      }
      // the dB/dC partials of a group of consecutive tokens, stored once the
      // group is done (padding tokens of the ragged last chunk write zeros,
      // which nothing reads)
      // Every lane issues the store: lanes that hold no sum store past the end of
      // the chunk's block, which the hardware drops.  A masked store could be
      // skipped as a whole, and the compiler would then wait for every memory
      // operation in flight before using the next chunk's operands.
      constexpr int SV = (CK % 4 == 0) ? 4 : 2;
      if (j % SV == 0) {
        float pv[SV];
#pragma unroll
        for (int e = 0; e < SV; ++e) pv[e] = uo[j + e];
        buf_store_span<F32, SV>(rs_part, pw ? pofs + (uint32_t)(j * 4) : 0x80000000u, 0u, pv);
      }
    }
    __syncthreads();
    // owners: dx = Delta sum lam B + dr Dskip, ddt = (dDelta) sigmoid(v)
    __builtin_amdgcn_s_setprio(0);
    {
      float dxv[kSpan], ddtv[kSpan];
#pragma unroll
      for (int i = 0; i < kSpan; ++i) {
        const int j = j_own + i;
        float ddp = 0.0f, sB = 0.0f;
        if (FULL || i < valid) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float2 pv = s_pp[j][g][c];
            ddp += pv.x;
            sB += pv.y;
          }
        }
        // Delta and dr of the owned token from LDS (the fast form's sB carries Delta)
        dxv[i] = ZOH ? sB + s_dr[j][c] * skip : fmaf(sB, s_dd[j][c].x, s_dr[j][c] * skip);
        // Euler: dDelta = (decay part) ln 2 + x sum lam B; ZOH: the lanes already added x sum lam e^u B
        const float dv = (ZOH ? ddp : fmaf(ddp, kLn2, sB * xv[i])) * sigmoid2(v2[i]);
        ddtv[i] = dv;   // zero for padding tokens and inactive channels
        if (FULL || i < valid) dbias_acc += dv;
      }
      if constexpr (STAGE) {
        stage_out(0, k, dxv);
        if (!dm.dt_row) stage_out(1, k, ddtv);
      } else if (act && (FULL || valid > 0)) {
        store_span<IO, kSpan>(static_cast<T*>(p.dx), row + tf, valid, vec, dxv);
        if (!dm.dt_row) store_span<IO, kSpan>(static_cast<T*>(p.ddt), row + tf, valid, vec, ddtv);
      }
      if (dm.dt_row) {
        // a shared dt's gradient is the sum over channels: every owner of this
        // lane's two tokens sits in this wave (one lane per channel), so the
        // channel sum is formed in the wave; row 0 of the result holds the first
        // owned token's sum and row 2 the second's, for each lane parity hk
        static_assert(kSpan == 2, "two owned tokens per lane");
        const float d0[1] = {ddtv[0]}, d1[1] = {ddtv[1]};
        const float u = bc_channel_sum<1, K>(d0, d1);
        if ((lane & 15) < K && (prow & 1) == 0 && (FULL || t0 + j_own + (prow >> 1) < t1))
          part_blk[(k * NPART + NOUT) * CK + j_own + (prow >> 1)] = u;
      }
      if constexpr (STAGE_IN) {
        if (k > kb) put_in((int)((k - 1) & 1), fi);   // LDS free: chunk k + 1 is done with it
      }
    }
    __syncthreads();
    if constexpr (STAGE) {
      if (t0 % GT == 0) flush_out(t0);
    }
  };
  {
    int64_t k = ke - 1;
    if (ke > kfull) chunk(std::false_type{}, k--);   // the sequence's ragged last chunk comes first
    for (; k >= kb; --k) chunk(std::true_type{}, k);
  }

  // dh0 = Abar_0 lam_0 (lam already carries the factor; the first segment's
  // workgroups); per-(segment, row, channel) sums
  const int64_t pch = seg * dm.batch * dm.dim + ch;
  if (act) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (p.dh0 && seg == 0) p.dh0[ch * N + sg * NS + s] = lam[s];
      p.dA_p[pch * N + sg * NS + s] = dAacc[s];
    }
  }
  s_pp[sg][0][c] = make_float2(dD_acc, dbias_acc);   // CK >= SG rows
  __syncthreads();
  if (sg == 0 && act) {
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int g = 0; g < SG; ++g) {
      const float2 v = s_pp[g][0][c];
      a0 += v.x;
      a1 += v.y;
    }
    p.dD_p[pch] = a0;
    p.dbias_p[pch] = a1;
  }
}

// A split sequence's aggregates, in one pass back through each segment (tokens
// t0 .. t1-1):
//  - the adjoint: going back through the segment the carried adjoint obeys
//    mu <- Abar_t (mu + dr_t C_t), so what leaves the segment is
//    exp(A sum Delta) mu_in + M_s, with M_s = sum_t (prod_{t0 <= t' <= t}
//    Abar_t') dr_t C_t the value that leaves when nothing enters;
//  - with FWD (no forward-saved checkpoints), the state: from a zero start the
//    segment ends in H_s = sum_t (prod_{t < t' < t1} Abar_t') c_t B_t x_t, the
//    forward's chunk aggregate, summed here from the last token with a running
//    product of Abar (c_t = Delta_t, or Delta_t phi(Delta_t A) for ZOH);
//  - the segment's sum of Delta, the exponent of both decay factors.
// dr = dy silu(z) needs no state, so every segment is independent; combines
// then give the state and the adjoint entering every segment.  Segments 1 ..
// nseg-1 need M_s and 0 .. nseg-2 need H_s, so the pass covers all of them
// with FWD and the segments after the first without.  Same lanes as the main
// kernel (G waves, K lanes per channel, NS state components per lane); work
// goes in stages of 16 bytes of every operand row per lane (AS tokens, AS * G
// * K per stage, which divides every segment length): the owner of each token
// stages Delta, dr (and Delta x), and every lane runs its components back
// through the stage.
// VEC: as for scan_bwd_kernel (no runtime choice between vector and element loads).
// ROWS (rows of at least 1 MB): the owners of a stage's tokens are the 8 lanes
// of a row, lane l of wave w owning tokens 8 (l % 8) .. + 7 of row 8 w + l / 8,
// so each wave's load covers a whole 128-byte line of 8 rows (as the scan's
// row-segment owners; with a lane's own channel each line was read a quarter
// by each wave, and with rows 2 MB apart every quarter went to L2).
template <int N, int G, int K, typename IO, bool ZOH, bool FWD, bool VEC, bool ROWS>
__global__ __launch_bounds__(64 * G) void bwd_segment_agg_kernel(const BwdDims dm, const BwdPtrs p) {
  using T = typename IO::T;
  constexpr int CPB = 64 / K;
  constexpr int SG = G * K;
  constexpr int NS = N / SG;
  constexpr int AS = IO::kPerSpan;            // tokens per lane and stage
  constexpr int ST = AS * SG;                 // tokens per stage (at most 64)
  constexpr int SW = SpanT<IO, AS>::kWords;
  constexpr int THREADS = 64 * G;
  constexpr int CPT = (ST * N + THREADS - 1) / THREADS;   // (B, C) pairs (C alone without FWD) each thread stages
  static_assert(64 % ST == 0, "a stage divides every segment length");
  static_assert(FWD || !ZOH, "the discretisation only enters the state's aggregate");
  static_assert(!ROWS || (K == 2 && G == 4 && CPB == 8 * G && ST == 8 * AS), "row owners: 8 lanes per row");
  using BCV = std::conditional_t<FWD, float2, float>;
  // (the row owners' writes need the rows padded by one channel to spread banks)
  __shared__ float2 s_dr[ST][CPB + (ROWS ? 1 : 0)];               // (Delta, dr) per token and channel
  __shared__ float s_dx[FWD ? ST : 1][CPB + (ROWS ? 1 : 0)];      // Delta x per token and channel
  __shared__ BCV s_bc[ST][N];                    // (B_n, C_n), or C_n, of the stage's tokens

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int c = lane / K;
  const int hk = lane % K;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sg = w * K + hk;

  // logical block -> (segment, batch row, channel block): every segment with
  // FWD, else segments 1 .. nseg-1
  const int64_t seg0 = FWD ? 0 : 1;
  const int64_t nwg = dm.cblocks * dm.batch * (dm.nseg - seg0);
  const int64_t lb = bwd_logical_block(blockIdx.x, nwg);
  const int64_t cb = lb % dm.cblocks;
  const int64_t b = (lb / dm.cblocks) % dm.batch;
  const int64_t seg = seg0 + lb / (dm.cblocks * dm.batch);
  const int64_t d = cb * CPB + c;
  const bool act = d < dm.dim;
  const int64_t dc = act ? d : dm.dim - 1;
  const int64_t L = dm.seqlen;
  const int64_t ch = b * dm.dim + dc;
  constexpr bool vec = VEC;   // every lane's span is 16-byte aligned
  const bool has_z = p.z != nullptr;
  const int64_t t_begin = seg * dm.seg_len;
  const int64_t t_end = t_begin + dm.seg_len < L ? t_begin + dm.seg_len : L;
  const int64_t sb = t_begin / ST;
  const int64_t se = (t_end + ST - 1) / ST;
  const int j_own = sg * AS;
  // the owner of the stage tokens this lane loads and stages (its own channel unless ROWS)
  const int oc = ROWS ? w * 8 + (lane >> 3) : c;
  const int otok = ROWS ? (lane & 7) * AS : j_own;
  const int64_t od = cb * CPB + oc;
  const bool oact = od < dm.dim;
  const int64_t orow = (b * dm.dim + (oact ? od : dm.dim - 1)) * L;
  const int64_t odt_row = dm.dt_row ? b * L : orow;

  const T* __restrict__ x = static_cast<const T*>(p.x);
  const T* __restrict__ dt = static_cast<const T*>(p.dt);
  const T* __restrict__ z = static_cast<const T*>(p.z);
  const T* __restrict__ dy = static_cast<const T*>(p.dy);
  float A2[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) A2[s] = p.A[dc * N + sg * NS + s] * kLog2e;
  const float bias2 = p.dt_bias ? p.dt_bias[oact ? od : dm.dim - 1] * kLog2e : 0.0f;   // the owner's
  const float* __restrict__ bc_row = p.bc + b * L * (2 * N);   // (token, n, {B, C})

  struct Fetch {
    uint32_t x[FWD ? SW : 1], dt[SW], z[SW], dy[SW];
    BCV bc[CPT];
  };
  // WHOLE (a compile-time tag): every token of stage k lies inside the segment,
  // so no load of the stage is masked or branched (which would make the
  // compiler wait for every memory operation in flight before the next use)
  auto fetch = [&](auto whole_tag, int64_t k, Fetch& f) {
    constexpr bool WHOLE = decltype(whole_tag)::value;
    const int64_t t0 = k * ST;
    const int64_t v = t_end - (t0 + otok);
    const int valid = WHOLE ? AS : (int)(v < 0 ? 0 : (v < AS ? v : AS));
    if constexpr (FWD) load_span<IO, AS>(x, orow + t0 + otok, valid, vec, f.x);
    load_span<IO, AS>(dt, odt_row + t0 + otok, valid, vec, f.dt);
    // without z, x stands in (its values are never used)
    load_span<IO, AS>(has_z ? z : x, orow + t0 + otok, valid, vec, f.z);
    load_span<IO, AS>(dy, orow + t0 + otok, valid, vec, f.dy);
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int idx = tid + q * THREADS;
      const bool in = (ST * N % THREADS == 0 || idx < ST * N) && (WHOLE || t0 + idx / N < t_end);
      if constexpr (FWD) f.bc[q] = in ? reinterpret_cast<const float2*>(bc_row)[t0 * N + idx] : make_float2(0.0f, 0.0f);
      else f.bc[q] = in ? bc_row[(t0 * N + idx) * 2 + 1] : 0.0f;
    }
  };

  float mu[NS], hf[NS], qd[NS];   // the adjoint; the state from zero and its pending decay
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    mu[s] = 0.0f;
    hf[s] = 0.0f;
    qd[s] = 1.0f;
  }
  float dsum = 0.0f;
  Fetch f;
  // the segment's stages, last to first; only the last (at the sequence's end)
  // can be partly outside it
  const int64_t swhole = t_end / ST;   // stages below swhole are whole
  if (se - 1 < swhole) fetch(std::true_type{}, se - 1, f);
  else fetch(std::false_type{}, se - 1, f);
  for (int64_t k = se - 1; k >= sb; --k) {
    const int64_t nj = t_end - k * ST;   // tokens of the stage inside the segment (ST or fewer)
#pragma unroll
    for (int i = 0; i < AS; ++i) {
      const float dl = (otok + i < nj) ? softplus_dt(span_elem<IO>(f.dt, i), bias2) : 0.0f;
      const float dyv = oact ? span_elem<IO>(f.dy, i) : 0.0f;   // padding tokens load as zero
      float gate = 1.0f;
      if (has_z) {
        const float zv = span_elem<IO>(f.z, i);
        gate = zv * sigmoid2(zv * kLog2e);
      }
      s_dr[otok + i][oc] = make_float2(dl, dyv * gate);
      if constexpr (FWD) s_dx[otok + i][oc] = dl * span_elem<IO>(f.x, i);
    }
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int idx = tid + q * THREADS;
      if (ST * N % THREADS == 0 || idx < ST * N) s_bc[idx / N][idx % N] = f.bc[q];
    }
    if (k > sb) fetch(std::true_type{}, k - 1, f);   // every stage before the last is whole
    __syncthreads();
#pragma unroll
    for (int j = ST - 1; j >= 0; --j) {
      const float2 o = s_dr[j][c];   // zero Delta, dr and Delta x past the segment's end
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const BCV bcv = s_bc[j][sg * NS + s];
        const float u2 = o.x * A2[s];
        const float E = __builtin_amdgcn_exp2f(u2);
        float Cv, Bv = 0.0f;
        if constexpr (FWD) {
          Bv = bcv.x;
          Cv = bcv.y;
        } else {
          Cv = bcv;
        }
        const float lam = fmaf(o.y, Cv, mu[s]);
        mu[s] = E * lam;
        if constexpr (FWD) {
          float in = s_dx[j][c] * Bv;
          if constexpr (ZOH) in *= zoh_phi(u2, E);
          hf[s] = fmaf(qd[s], in, hf[s]);
          qd[s] *= E;
        }
      }
      dsum += o.x;
    }
    __syncthreads();
  }
  if (act) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int64_t k = (ch * dm.nseg + seg) * N + sg * NS + s;
      if (seg > 0) p.adj_m[k] = mu[s];
      if constexpr (FWD) p.agg_h[k] = hf[s];
    }
    if (sg == 0) p.adj_s[ch * dm.nseg + seg] = dsum;
  }
}

template <int N, int G, int K, typename IO, bool ZOH, bool FWD>
hipError_t launch_segment_agg_t(const BwdDims& dm, const BwdPtrs& p, hipStream_t s) {
  const int64_t nwg = dm.cblocks * dm.batch * (dm.nseg - (FWD ? 0 : 1));
  const bool vec = dm.seqlen % IO::kPerSpan == 0;
  // rows of at least 1 MB (bf16, two lanes per channel): the row owners
  if constexpr (sizeof(typename IO::T) == 2 && G == 4 && K == 2) {
    if (vec && dm.seqlen * 2 >= (int64_t(1) << 20)) {
      hipLaunchKernelGGL((bwd_segment_agg_kernel<N, G, K, IO, ZOH, FWD, true, true>), dim3((unsigned)nwg),
                         dim3(64 * G), 0, s, dm, p);
      return hipGetLastError();
    }
  }
  if (vec)
    hipLaunchKernelGGL((bwd_segment_agg_kernel<N, G, K, IO, ZOH, FWD, true, false>), dim3((unsigned)nwg),
                       dim3(64 * G), 0, s, dm, p);
  else
    hipLaunchKernelGGL((bwd_segment_agg_kernel<N, G, K, IO, ZOH, FWD, false, false>), dim3((unsigned)nwg),
                       dim3(64 * G), 0, s, dm, p);
  return hipGetLastError();
}

// FWD: also the segments' state aggregates (no forward-saved checkpoints)
template <typename IO, bool ZOH, bool FWD>
hipError_t launch_segment_agg_n(const BwdDims& dm, const BwdPtrs& p, hipStream_t s) {
  switch (dm.dstate) {
    case 1: return launch_segment_agg_t<1, 1, 1, IO, ZOH, FWD>(dm, p, s);
    case 2: return launch_segment_agg_t<2, 2, 1, IO, ZOH, FWD>(dm, p, s);
    case 4: return launch_segment_agg_t<4, 4, 1, IO, ZOH, FWD>(dm, p, s);
    case 8: return launch_segment_agg_t<8, 4, 2, IO, ZOH, FWD>(dm, p, s);
    case 16: return launch_segment_agg_t<16, 4, 2, IO, ZOH, FWD>(dm, p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int N, int G, int K, typename IO, bool ZOH>
hipError_t launch_bwd_t(const BwdDims& dm, const BwdPtrs& p, hipStream_t s) {
  const int64_t nwg = dm.cblocks * dm.batch * dm.nseg;
  // Whole-piece operand loads for rows at least 1 MB long (bf16, first order):
  // there the workgroup's rows share their offset in the memory pages (the
  // million-token backward 58.0 -> 48.0 ms); at shorter rows they cost about
  // 0.5% (2.8B-shaped layer) and buy nothing.
  if constexpr (!ZOH && sizeof(typename IO::T) == 2 && G == 4 && K == 2) {
    if (dm.vec && dm.seqlen % 8 == 0 && dm.seqlen * 2 >= (int64_t(1) << 20)) {
      hipLaunchKernelGGL((scan_bwd_kernel<N, G, K, IO, ZOH, true, true>), dim3((unsigned)nwg), dim3(64 * G), 0, s,
                         dm, p);
      return hipGetLastError();
    }
  }
  if (dm.vec)
    hipLaunchKernelGGL((scan_bwd_kernel<N, G, K, IO, ZOH, true, false>), dim3((unsigned)nwg), dim3(64 * G), 0, s, dm,
                       p);
  else
    hipLaunchKernelGGL((scan_bwd_kernel<N, G, K, IO, ZOH, false, false>), dim3((unsigned)nwg), dim3(64 * G), 0, s,
                       dm, p);
  return hipGetLastError();
}

template <typename IO, bool ZOH>
hipError_t launch_bwd_n(const BwdDims& dm, const BwdPtrs& p, hipStream_t s) {
  switch (dm.dstate) {
    case 1: return launch_bwd_t<1, 1, 1, IO, ZOH>(dm, p, s);
    case 2: return launch_bwd_t<2, 2, 1, IO, ZOH>(dm, p, s);
    case 4: return launch_bwd_t<4, 4, 1, IO, ZOH>(dm, p, s);
    case 8: return launch_bwd_t<8, 4, 2, IO, ZOH>(dm, p, s);
    case 16: return launch_bwd_t<16, 4, 2, IO, ZOH>(dm, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bwd_detail
}  // namespace ssscan
