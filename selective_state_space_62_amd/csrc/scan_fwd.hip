// Full-sequence selective scan for gfx950.
//
// The recurrence (reader's notes on the Mamba paper, kurisu.si, "What they did",
// item "Selective SSM (S6)"): per channel, Delta_t = softplus(dt + dt_bias),
// Abar = exp(Delta A), h_t = Abar h_(t-1) + Delta B_t x_t, y_t = C_t . h_t (+ skip,
// gate).  The notes stress that the expanded state (one N-vector per channel and
// token) is never written to HBM; here it lives in VGPRs for the whole sequence.
//
// Mapping onto CDNA4:
//  * One workgroup = 64/K channels of one batch row and G waves; each channel
//    has K adjacent lanes (K = 1 or 2) in every wave.  The N state components are
//    split into G*K groups: lane k of a channel in wave w owns group w K + k.
//    K = 2 halves the channels per workgroup, so there are twice as many equal
//    workgroups (for the 2.8B-shaped layer 1280, exactly 5 per CU, where 640
//    leave half the CUs with one more than the rest).
//  * Tiles of T = G * 16B/elem tokens.  Each wave loads 16 bytes of x, dt, z per
//    channel for its own T/G tokens (16/K bytes per lane), computes Delta and
//    Delta*x once per (token, channel), and shares them through LDS.  The
//    tile's B and C (from a per-call fp32 re-layout, prep_bc_kernel) are staged in
//    LDS with one 16-byte load per thread and read back as same-address
//    (broadcast) LDS loads.  Everything the inner loop waits on is an in-order
//    LDS access, so it can be issued tokens ahead; scalar loads were tried for
//    B/C and stalled every token (they return out of order, so each use waits
//    for all outstanding scalar and LDS accesses).  All global loads of the next
//    tile are issued one tile ahead.
//  * Every lane runs its state components through all T tokens of the tile; the
//    K lanes of a channel add their readouts with one DPP add, and each wave
//    writes one partial readout per (token, channel) to LDS.  The owner of a
//    token sums the G partials in a fixed order (deterministic results), adds the
//    skip term, applies the gate and writes its span of y.
//  * The per-(token, state) work is exp2, two multiplies and two FMAs; transcendentals
//    are half-rate on gfx950 and do not co-issue with FMAs, so the kernel is bound
//    by VALU issue, not by HBM.
//  * Long sequences with few channels are cut into chunks: an aggregate pass
//    (AGG = true) gives each chunk's end state from a zero start and its sum of
//    Delta; combine_kernel runs the exclusive scan of (exp(A sum Delta), h_end)
//    pairs across chunks; the full pass then rescans every chunk from its true
//    initial state.  The combine (P1, h1) o (P2, h2) = (P1 P2, P2 h1 + h2) follows
//    from the linearity of the recurrence.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ssscan {
namespace {

using namespace dev;

// B and C (batch, N, L) in the I/O dtype -> (batch, L, N, 2) fp32, B_n and C_n
// adjacent.  One thread per (b, t): reads are coalesced along t, writes are 2N
// contiguous floats.
template <int N, typename IO>
__global__ __launch_bounds__(256) void prep_bc_kernel(const typename IO::T* __restrict__ B,
                                                      const typename IO::T* __restrict__ C,
                                                      float* __restrict__ bc, int64_t batch, int64_t L) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= batch * L) return;
  const int64_t b = i / L, t = i - b * L;
  float v[2 * N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    v[2 * n] = load_one<IO>(B, (b * N + n) * L + t);
    v[2 * n + 1] = load_one<IO>(C, (b * N + n) * L + t);
  }
  float* o = bc + i * (2 * N);
  if constexpr (N >= 2) {
#pragma unroll
    for (int k = 0; k < 2 * N; k += 4)
      *reinterpret_cast<float4*>(o + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  } else {
    *reinterpret_cast<float2*>(o) = make_float2(v[0], v[1]);
  }
}

// Workgroup index -> logical block, so that consecutive logical blocks (the
// channel blocks of one batch row, which share that row's B and C) land on the
// same XCD; workgroups are dealt to the 8 XCDs round-robin.
__device__ __forceinline__ int64_t xcd_logical_block(int64_t wg, int64_t nwg) {
  if ((nwg & 7) != 0) return wg;
  return (wg & 7) * (nwg >> 3) + (wg >> 3);
}

// B/C tile pieces: 16 bytes (two state components) for N >= 2, 8 bytes for N = 1.
template <int N>
struct BcPiece {
  using V = float4;
  static constexpr int kFloats = 4;
};
template <>
struct BcPiece<1> {
  using V = float2;
  static constexpr int kFloats = 2;
};

// At most 96 VGPRs (5 waves per SIMD): with 4 waves per workgroup and 28 KB of
// LDS, five workgroups fit on a CU at once, which the two-lanes-per-channel plan
// needs to keep every CU's share resident.
template <int N, int G, int K, typename IO, bool AGG>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(5, 10))) void scan_kernel(
    const ScanDims dm, const typename IO::T* __restrict__ x, const typename IO::T* __restrict__ dt,
    const typename IO::T* __restrict__ z, const float* __restrict__ bc, const float* __restrict__ A,
    const float* __restrict__ Dskip, const float* __restrict__ dt_bias, const float* __restrict__ h0,
    const float* __restrict__ h_in, typename IO::T* __restrict__ y, float* __restrict__ h_final,
    float* __restrict__ agg_h, float* __restrict__ agg_s) {
  constexpr int CPB = 64 / K;            // channels per workgroup (K adjacent lanes per channel)
  constexpr int SG = G * K;              // state groups (one per lane of a channel per wave)
  constexpr int NS = N / SG;             // state components per lane
  constexpr int TPW = IO::kPerSpan;      // tokens owned per wave per tile (16 bytes of a row)
  constexpr int SPAN = TPW / K;          // of which each lane of a channel owns SPAN
  constexpr int T = TPW * G;             // tile length
  constexpr int THREADS = 64 * G;
  constexpr int SW = SpanT<IO, SPAN>::kWords;
  using Piece = typename BcPiece<N>::V;
  constexpr int PF = BcPiece<N>::kFloats;
  constexpr int BC_PIECES = T * 2 * N / PF;                      // pieces of B/C per tile
  constexpr int BC_PER_THREAD = (BC_PIECES + THREADS - 1) / THREADS;
  constexpr int TOK_PIECES = 2 * N / PF;                         // pieces per token
  static_assert(NS >= 1 && N % SG == 0, "G * K must divide N");
  static_assert(K == 1 || K == 2, "one or two lanes per channel");
  constexpr bool SHARE_DD = (G * K) > 1;   // Delta is computed once and shared through LDS

  __shared__ float2 s_dd[SHARE_DD ? T : 1][CPB];              // (Delta, Delta*x) per token and channel
  __shared__ float s_part[(SHARE_DD && !AGG) ? T : 1][G][CPB];   // partial readouts per token, wave, channel
  __shared__ Piece s_bc[BC_PIECES];                           // the tile's B_n, C_n (token-major, n, B/C)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int c = lane / K;                 // channel within the block
  const int hk = lane % K;                // lane of the channel
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sg = w * K + hk;              // state group of this lane

  // logical block -> (chunk, batch row, channel block), channel block fastest
  const int64_t cblocks = (dm.dim + CPB - 1) / CPB;
  const int64_t nwg = cblocks * dm.batch * dm.num_chunks;
  int64_t lb = xcd_logical_block(blockIdx.x, nwg);
  const int64_t cb = lb % cblocks;
  lb /= cblocks;
  const int64_t b = lb % dm.batch;
  const int64_t chunk = lb / dm.batch;

  const int64_t d = cb * CPB + c;
  const bool act = d < dm.dim;
  const int64_t dc = act ? d : dm.dim - 1;   // clamped: inactive lanes compute on a valid row
  const int64_t L = dm.seqlen;
  const int64_t t0 = chunk * dm.chunk_len;
  const int64_t t1 = (t0 + dm.chunk_len < L) ? t0 + dm.chunk_len : L;
  const int64_t ch = b * dm.dim + dc;
  const int64_t row = ch * L;
  const bool vec = dm.vec != 0;
  const bool has_z = z != nullptr;

  float A2[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) A2[s] = A[dc * N + sg * NS + s] * kLog2e;
  const float bias2 = dt_bias ? dt_bias[dc] * kLog2e : 0.0f;
  const float skip = Dskip ? Dskip[dc] : 0.0f;

  float h[NS];
  {
    const float* hi = nullptr;
    if constexpr (!AGG) {
      if (h_in) hi = h_in + (ch * dm.num_chunks + chunk) * N + sg * NS;
      else if (h0) hi = h0 + ch * N + sg * NS;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) h[s] = hi ? hi[s] : 0.0f;
  }
  float dsum = 0.0f;   // AGG: sum of Delta over the chunk

  // B/C of this batch row, re-laid out (token, n, {B, C}); pieces never straddle tokens
  const Piece* __restrict__ bc_row = reinterpret_cast<const Piece*>(bc + b * L * (2 * N));
  Piece cbc[BC_PER_THREAD];
  // `whole`: every token of the tile lies inside the chunk (no per-piece check)
  auto load_bc_tile = [&](int64_t ts, bool whole) {
#pragma unroll
    for (int k = 0; k < BC_PER_THREAD; ++k) {
      const int piece = tid + k * THREADS;
      const int64_t tok = ts + piece / TOK_PIECES;
      if (piece < BC_PIECES && (whole || tok < t1)) cbc[k] = bc_row[ts * TOK_PIECES + piece];
      else cbc[k] = Piece{};
    }
  };
  // first token of the span this lane owns in the tile starting at ts
  auto own_first = [&](int64_t ts) { return ts + w * TPW + hk * SPAN; };
  auto own_valid = [&](int64_t first) {
    const int64_t v = t1 - first;
    return (int)(v < 0 ? 0 : (v < SPAN ? v : SPAN));
  };

  // raw spans of x, dt, z for this lane's tokens of the current tile (prefetched a tile ahead)
  uint32_t cx[SW], cdt[SW], cz[SW] = {};
  {
    const int64_t tf = own_first(t0);
    const int valid = own_valid(tf);
    load_span<IO, SPAN>(x, row + tf, valid, vec, cx);
    load_span<IO, SPAN>(dt, row + tf, valid, vec, cdt);
    if (has_z) load_span<IO, SPAN>(z, row + tf, valid, vec, cz);
    load_bc_tile(t0, t0 + T <= t1);
  }

  // One tile.  FULL (a compile-time tag) means all T tokens lie inside the chunk:
  // no per-token masks, no guards in the inner loop.
  auto tile = [&](auto full_tag, int64_t ts) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int64_t tf = own_first(ts);
    const int valid = FULL ? SPAN : own_valid(tf);

    // phase A: Delta and Delta*x for the owned tokens; stage the B/C tile
    float xv[SPAN], zv[SPAN], dl[SPAN], dx[SPAN];
#pragma unroll
    for (int i = 0; i < SPAN; ++i) {
      xv[i] = span_elem<IO>(cx, i);
      zv[i] = span_elem<IO>(cz, i);
      const float delta = softplus_dt(span_elem<IO>(cdt, i), bias2);
      if constexpr (FULL) dl[i] = delta;
      else dl[i] = (i < valid) ? delta : 0.0f;            // padding tokens leave the state alone
      dx[i] = dl[i] * xv[i];
    }
#pragma unroll
    for (int k = 0; k < BC_PER_THREAD; ++k)
      if (tid + k * THREADS < BC_PIECES) s_bc[tid + k * THREADS] = cbc[k];
    // prefetch the next tile: plain vector loads when it is whole and aligned
    // (every tile but the last), masked loads otherwise
    if (vec && ts + 2 * T <= t1) {
      const int64_t tn = tf + T;
      load_span<IO, SPAN>(x, row + tn, SPAN, true, cx);
      load_span<IO, SPAN>(dt, row + tn, SPAN, true, cdt);
      if (has_z) load_span<IO, SPAN>(z, row + tn, SPAN, true, cz);
      load_bc_tile(ts + T, true);
    } else if (ts + T < t1) {
      const int64_t tn = tf + T;
      const int validn = own_valid(tn);
      load_span<IO, SPAN>(x, row + tn, validn, vec, cx);
      load_span<IO, SPAN>(dt, row + tn, validn, vec, cdt);
      if (has_z) load_span<IO, SPAN>(z, row + tn, validn, vec, cz);
      load_bc_tile(ts + T, ts + 2 * T <= t1);
    }
    if constexpr (SHARE_DD) {
#pragma unroll
      for (int i = 0; i < SPAN; ++i) s_dd[w * TPW + hk * SPAN + i][c] = make_float2(dl[i], dx[i]);
    }
    __syncthreads();

    // phase B: this lane's state components through every token of the tile.
    // The LDS operands of token j + 1 are read before token j is computed.
    float yp[SHARE_DD ? 1 : T];
    struct Ops {
      float d, dx, bcv[2 * NS];
    };
    auto fetch = [&](int j, Ops& o) {
      if constexpr (SHARE_DD) {
        const float2 v = s_dd[j][c];
        o.d = v.x;
        o.dx = v.y;
      } else {
        o.d = dl[j];
        o.dx = dx[j];
      }
      const float* src = reinterpret_cast<const float*>(s_bc) + j * (2 * N) + 2 * sg * NS;
      if constexpr (NS == 1) {
        const float2 v = *reinterpret_cast<const float2*>(src);
        o.bcv[0] = v.x;
        o.bcv[1] = v.y;
      } else {
#pragma unroll
        for (int q = 0; q < 2 * NS; q += 4) {
          const float4 v = *reinterpret_cast<const float4*>(src + q);
          o.bcv[q] = v.x;
          o.bcv[q + 1] = v.y;
          o.bcv[q + 2] = v.z;
          o.bcv[q + 3] = v.w;
        }
      }
    };
    auto compute = [&](int j, const Ops& o) {
      float acc = 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float E = __builtin_amdgcn_exp2f(o.d * A2[s]);
        h[s] = fmaf(E, h[s], o.dx * o.bcv[2 * s]);
        if constexpr (!AGG) acc = (s == 0) ? o.bcv[1] * h[0] : fmaf(o.bcv[2 * s + 1], h[s], acc);
      }
      if constexpr (AGG) {
        dsum += o.d;
      } else {
        // both lanes of a channel end with the channel's sum over this wave's components
        if constexpr (K == 2) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0xB1, 0xf, 0xf, false);
        if constexpr (SHARE_DD) s_part[j][w][c] = acc;
        else yp[j] = acc;
      }
    };
    const int nj = FULL ? T : (int)(t1 - ts);
    Ops cur, nxt;
    fetch(0, cur);
#pragma unroll
    for (int j = 0; j < T; ++j) {
      if (FULL || j < nj) {
        if (j + 1 < T && (FULL || j + 1 < nj)) fetch(j + 1, nxt);
        compute(j, cur);
        cur = nxt;
      }
    }

    // phase C: the owner of each token sums the partial readouts, adds the skip
    // term, applies the gate and stores y
    if constexpr (SHARE_DD) __syncthreads();
    if constexpr (!AGG) {
      float yv[SPAN];
#pragma unroll
      for (int i = 0; i < SPAN; ++i) {
        float acc;
        if constexpr (SHARE_DD) {
          const int j = w * TPW + hk * SPAN + i;
          acc = s_part[j][0][c];
#pragma unroll
          for (int g = 1; g < G; ++g) acc += s_part[j][g][c];
        } else {
          acc = yp[i];
        }
        yv[i] = fmaf(skip, xv[i], acc);
      }
      if (has_z) {
#pragma unroll
        for (int i = 0; i < SPAN; ++i) yv[i] *= silu(zv[i]);
      }
      if (act && (FULL || valid > 0)) store_span<IO, SPAN>(y, row + tf, valid, vec, yv);
    }
  };

  for (int64_t ts = t0; ts < t1; ts += T) {
    if (ts + T <= t1) tile(std::true_type{}, ts);
    else tile(std::false_type{}, ts);
  }

  if (act) {
    if constexpr (AGG) {
      float* o = agg_h + (ch * dm.num_chunks + chunk) * N + sg * NS;
#pragma unroll
      for (int s = 0; s < NS; ++s) o[s] = h[s];
      if (sg == 0) agg_s[ch * dm.num_chunks + chunk] = dsum;
    } else if (h_final && chunk == dm.num_chunks - 1) {
#pragma unroll
      for (int s = 0; s < NS; ++s) h_final[ch * N + sg * NS + s] = h[s];
    }
  }
}

// Exclusive scan of the chunk aggregates, one lane per (b, d, n):
// h_in[c] = state entering chunk c; h <- exp(A * sum Delta_c) h + h_end_c.
__global__ __launch_bounds__(256) void combine_kernel(int64_t nstate, int64_t dim, int dstate, int num_chunks,
                                                      const float* __restrict__ A, const float* __restrict__ agg_h,
                                                      const float* __restrict__ agg_s, const float* __restrict__ h0,
                                                      float* __restrict__ h_in) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nstate) return;
  const int64_t ch = i / dstate;
  const int n = (int)(i - ch * dstate);
  const int64_t d = ch % dim;
  const float a2 = A[d * dstate + n] * dev::kLog2e;
  float h = h0 ? h0[i] : 0.0f;
  for (int c = 0; c < num_chunks; ++c) {
    const int64_t k = (ch * num_chunks + c) * dstate + n;
    h_in[k] = h;
    const float decay = __builtin_amdgcn_exp2f(a2 * agg_s[ch * num_chunks + c]);
    h = fmaf(decay, h, agg_h[k]);
  }
}

__global__ __launch_bounds__(256) void copy_state_kernel(int64_t count, const float* __restrict__ src,
                                                         float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) dst[i] = src ? src[i] : 0.0f;
}

template <int N, int G, int K, typename IO, bool AGG>
hipError_t launch_scan_t(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  using E = typename IO::T;
  const int64_t cblocks = (dm.dim + 64 / K - 1) / (64 / K);
  const int64_t nwg = cblocks * dm.batch * dm.num_chunks;
  hipLaunchKernelGGL((scan_kernel<N, G, K, IO, AGG>), dim3((unsigned)nwg), dim3(64 * G), 0, s, dm,
                     (const E*)p.x, (const E*)p.dt, (const E*)p.z, p.bc, p.A, p.Dskip, p.dt_bias, p.h0, p.h_in,
                     (E*)p.y, p.h_final, p.agg_h, p.agg_s);
  return hipGetLastError();
}

template <int N, int G, typename IO, bool AGG>
hipError_t launch_scan_k(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  if (dm.lanes == 1) return launch_scan_t<N, G, 1, IO, AGG>(dm, p, s);
  if constexpr (N >= 2 * G) {
    if (dm.lanes == 2) return launch_scan_t<N, G, 2, IO, AGG>(dm, p, s);
  }
  return hipErrorInvalidValue;
}

template <int N, typename IO, bool AGG>
hipError_t launch_scan_g(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  switch (dm.groups) {
    case 1: return launch_scan_k<N, 1, IO, AGG>(dm, p, s);
    case 2: if constexpr (N >= 2) return launch_scan_k<N, 2, IO, AGG>(dm, p, s); else break;
    case 4: if constexpr (N >= 4) return launch_scan_k<N, 4, IO, AGG>(dm, p, s); else break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename IO, bool AGG>
hipError_t launch_scan_n(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  switch (dm.dstate) {
    case 1: return launch_scan_g<1, IO, AGG>(dm, p, s);
    case 2: return launch_scan_g<2, IO, AGG>(dm, p, s);
    case 4: return launch_scan_g<4, IO, AGG>(dm, p, s);
    case 8: return launch_scan_g<8, IO, AGG>(dm, p, s);
    case 16: return launch_scan_g<16, IO, AGG>(dm, p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename IO>
hipError_t launch_prep_t(const ScanDims& dm, const void* B, const void* C, float* bc, hipStream_t s) {
  using E = typename IO::T;
  const int64_t n = dm.batch * dm.seqlen;
  const dim3 grid((unsigned)((n + 255) / 256));
  switch (dm.dstate) {
    case 1: hipLaunchKernelGGL((prep_bc_kernel<1, IO>), grid, dim3(256), 0, s, (const E*)B, (const E*)C, bc, dm.batch, dm.seqlen); break;
    case 2: hipLaunchKernelGGL((prep_bc_kernel<2, IO>), grid, dim3(256), 0, s, (const E*)B, (const E*)C, bc, dm.batch, dm.seqlen); break;
    case 4: hipLaunchKernelGGL((prep_bc_kernel<4, IO>), grid, dim3(256), 0, s, (const E*)B, (const E*)C, bc, dm.batch, dm.seqlen); break;
    case 8: hipLaunchKernelGGL((prep_bc_kernel<8, IO>), grid, dim3(256), 0, s, (const E*)B, (const E*)C, bc, dm.batch, dm.seqlen); break;
    case 16: hipLaunchKernelGGL((prep_bc_kernel<16, IO>), grid, dim3(256), 0, s, (const E*)B, (const E*)C, bc, dm.batch, dm.seqlen); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep_bc(const ScanDims& dm, const void* B, const void* C, float* bc, hipStream_t s) {
  return dm.io == kIoBf16 ? launch_prep_t<BF16>(dm, B, C, bc, s) : launch_prep_t<F32>(dm, B, C, bc, s);
}

hipError_t launch_scan(const ScanDims& dm, const ScanPtrs& p, bool aggregate, hipStream_t s) {
  if (dm.io == kIoBf16)
    return aggregate ? launch_scan_n<BF16, true>(dm, p, s) : launch_scan_n<BF16, false>(dm, p, s);
  return aggregate ? launch_scan_n<F32, true>(dm, p, s) : launch_scan_n<F32, false>(dm, p, s);
}

hipError_t launch_combine(const ScanDims& dm, const float* A, const float* agg_h, const float* agg_s,
                          const float* h0, float* h_in, hipStream_t s) {
  const int64_t nstate = dm.batch * dm.dim * dm.dstate;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((nstate + 255) / 256)), dim3(256), 0, s, nstate, dm.dim,
                     dm.dstate, dm.num_chunks, A, agg_h, agg_s, h0, h_in);
  return hipGetLastError();
}

hipError_t launch_copy_state(int64_t count, const float* src, float* dst, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, count, src, dst);
  return hipGetLastError();
}

}  // namespace ssscan
