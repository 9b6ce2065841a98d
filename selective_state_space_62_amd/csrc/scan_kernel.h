// The scan kernel template and its launch dispatch, shared by the translation
// units that instantiate it (one per I/O dtype and discretisation, compiled in
// parallel).  See scan_fwd.hip for the design.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ssscan {
namespace scan_detail {

using namespace dev;

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

// At most 96 VGPRs (5 waves per SIMD) for the plans with two or four lanes per
// channel and up to 2 state components per lane: with 4 waves per workgroup and
// 28 KB of LDS, five workgroups fit on a CU at once, which the two-lanes-per-
// channel plan needs to keep every CU's share resident.  One-lane plans (each
// lane owns 8 or 4 tokens of the per-token work) and plans with more components
// per lane get no occupancy target.
// CKPT_K (full pass only): also store the state entering every backward-pass
// chunk, for a training step's backward.  It is a separate instantiation so
// that the plain scan keeps its registers.
template <int N, int G, int K, typename IO, bool AGG, bool ZOH, bool CKPT_K>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(K >= 2 && N / (G * K) <= 2 ? 5 : 1, 10))) void scan_kernel(
    const ScanDims dm, const typename IO::T* __restrict__ x, const typename IO::T* __restrict__ dt,
    const typename IO::T* __restrict__ z, const float* __restrict__ bc, const float* __restrict__ A,
    const float* __restrict__ Dskip, const float* __restrict__ dt_bias, const float* __restrict__ h0,
    const float* __restrict__ h_in, typename IO::T* __restrict__ y, float* __restrict__ h_final,
    float* __restrict__ agg_h, float* __restrict__ agg_s, float* __restrict__ ckpt) {
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
  static_assert(K == 1 || K == 2 || K == 4, "one, two or four lanes per channel");
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
  const int64_t dt_row = dm.dt_row ? b * L : row;   // dt per (row, token) is shared by the row's channels
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
  // checkpoints for the backward pass: the state entering every ck_len-token chunk
  float* __restrict__ ck_row = nullptr;
  if constexpr (CKPT_K) {
    if (ckpt && act) ck_row = ckpt + (b * dm.ck_count * dm.dim + dc) * N + sg * NS;   // (batch, chunk, dim, N)
  }
  constexpr int CKL = bwd_chunk_tokens(N);   // checkpoint interval (a power of 2)
  if constexpr (CKPT_K) {
    if (ck_row && (t0 % CKL) == 0) {
#pragma unroll
      for (int s = 0; s < NS; ++s) ck_row[(t0 / CKL) * dm.dim * N + s] = h[s];
    }
  }

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
    load_span<IO, SPAN>(dt, dt_row + tf, valid, vec, cdt);
    if (has_z) load_span<IO, SPAN>(z, row + tf, valid, vec, cz);
    load_bc_tile(t0, t0 + T <= t1);
  }

  // One tile.  FULL (a compile-time tag) means all T tokens lie inside the chunk:
  // no per-token masks, no guards in the inner loop.
  auto tile = [&](auto full_tag, auto ck_tag, int64_t ts) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr bool CKPT = decltype(ck_tag)::value && CKPT_K;
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
      load_span<IO, SPAN>(dt, dt_row + tn, SPAN, true, cdt);
      if (has_z) load_span<IO, SPAN>(z, row + tn, SPAN, true, cz);
      load_bc_tile(ts + T, true);
    } else if (ts + T < t1) {
      const int64_t tn = tf + T;
      const int validn = own_valid(tn);
      load_span<IO, SPAN>(x, row + tn, validn, vec, cx);
      load_span<IO, SPAN>(dt, dt_row + tn, validn, vec, cdt);
      if (has_z) load_span<IO, SPAN>(z, row + tn, validn, vec, cz);
      load_bc_tile(ts + T, ts + 2 * T <= t1);
    }
    if constexpr (SHARE_DD) {
#pragma unroll
      for (int i = 0; i < SPAN; ++i) s_dd[w * TPW + hk * SPAN + i][c] = make_float2(dl[i], dx[i]);
    }
    __syncthreads();
    // Phase B runs at a raised wave priority and phases C and A at the
    // default, so a SIMD's issue favours the waves sweeping the state over
    // those of other workgroups in their short owner phases (5-6% faster at
    // the 2.8B shape than one priority throughout).
    __builtin_amdgcn_s_setprio(2);

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
        const float u2 = o.d * A2[s];
        const float E = __builtin_amdgcn_exp2f(u2);
        float in = o.dx * o.bcv[2 * s];                 // first order: Bbar x = Delta B x
        if constexpr (ZOH) in *= zoh_phi(u2, E);        // zero-order hold: (e^u - 1)/u Delta B x
        h[s] = fmaf(E, h[s], in);
        if constexpr (!AGG) acc = (s == 0) ? o.bcv[1] * h[0] : fmaf(o.bcv[2 * s + 1], h[s], acc);
      }
      if constexpr (AGG) {
        dsum += o.d;
      } else {
        // both lanes of a channel end with the channel's sum over this wave's components
        // the K lanes of a channel (adjacent in a quad) end with the channel's sum
        if constexpr (K >= 2) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0xB1, 0xf, 0xf, false);   // [1,0,3,2]
        if constexpr (K == 4) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0x4E, 0xf, 0xf, false);   // [2,3,0,1]
        if constexpr (SHARE_DD) s_part[j][w][c] = acc;
        else yp[j] = acc;
      }
    };
    const int nj = FULL ? T : (int)(t1 - ts);
    constexpr int NMID = (T > CKL) ? T / CKL - 1 : 1;   // checkpoint positions inside the tile
    float hmid[NMID][NS];
    Ops cur, nxt;
    fetch(0, cur);
#pragma unroll
    for (int j = 0; j < T; ++j) {
      if (FULL || j < nj) {
        if (j + 1 < T && (FULL || j + 1 < nj)) fetch(j + 1, nxt);
        compute(j, cur);
        cur = nxt;
        if constexpr (CKPT && T > CKL) {
          // the state after token ts + j enters checkpoint chunk (ts + j + 1) / CKL;
          // tiles start at multiples of T, so inside a tile the positions are
          // fixed: keep a copy (no branch here), stored after the tile
          if ((j + 1) % CKL == 0 && j + 1 < T) {
#pragma unroll
            for (int s = 0; s < NS; ++s) hmid[(j + 1) / CKL - 1][s] = h[s];
          }
        }
      }
    }

    if constexpr (CKPT) {
      if (ck_row) {
        if constexpr (T > CKL) {
#pragma unroll
          for (int m = 0; m < NMID; ++m) {
            const int64_t tn = ts + (m + 1) * CKL;
            if ((FULL || (m + 1) * CKL <= nj) && tn < L) {
#pragma unroll
              for (int s = 0; s < NS; ++s) ck_row[(tn / CKL) * dm.dim * N + s] = hmid[m][s];
            }
          }
        }
        const int64_t te = ts + nj;   // the state after the tile's last token
        if (te % CKL == 0 && te < L) {
#pragma unroll
          for (int s = 0; s < NS; ++s) ck_row[(te / CKL) * dm.dim * N + s] = h[s];
        }
      }
    }

    // phase C: the owner of each token sums the partial readouts, adds the skip
    // term, applies the gate and stores y
    if constexpr (SHARE_DD) __syncthreads();
    __builtin_amdgcn_s_setprio(0);
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
    if (ts + T <= t1) tile(std::true_type{}, std::integral_constant<bool, CKPT_K>{}, ts);
    else tile(std::false_type{}, std::integral_constant<bool, CKPT_K>{}, ts);
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

template <int N, int G, int K, typename IO, bool AGG, bool ZOH>
hipError_t launch_scan_t(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  using E = typename IO::T;
  const int64_t cblocks = (dm.dim + 64 / K - 1) / (64 / K);
  const int64_t nwg = cblocks * dm.batch * dm.num_chunks;
  if constexpr (!AGG) {
    if (p.ckpt) {
      hipLaunchKernelGGL((scan_kernel<N, G, K, IO, false, ZOH, true>), dim3((unsigned)nwg), dim3(64 * G), 0, s,
                         dm, (const E*)p.x, (const E*)p.dt, (const E*)p.z, p.bc, p.A, p.Dskip, p.dt_bias, p.h0,
                         p.h_in, (E*)p.y, p.h_final, p.agg_h, p.agg_s, p.ckpt);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((scan_kernel<N, G, K, IO, AGG, ZOH, false>), dim3((unsigned)nwg), dim3(64 * G), 0, s, dm,
                     (const E*)p.x, (const E*)p.dt, (const E*)p.z, p.bc, p.A, p.Dskip, p.dt_bias, p.h0, p.h_in,
                     (E*)p.y, p.h_final, p.agg_h, p.agg_s, nullptr);
  return hipGetLastError();
}

template <int N, int G, typename IO, bool AGG, bool ZOH>
hipError_t launch_scan_k(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  if (dm.lanes == 1) return launch_scan_t<N, G, 1, IO, AGG, ZOH>(dm, p, s);
  if constexpr (N >= 2 * G) {
    if (dm.lanes == 2) return launch_scan_t<N, G, 2, IO, AGG, ZOH>(dm, p, s);
  }
  if constexpr (N >= 4 * G && G == 4) {
    if (dm.lanes == 4) return launch_scan_t<N, G, 4, IO, AGG, ZOH>(dm, p, s);
  }
  return hipErrorInvalidValue;
}

template <int N, typename IO, bool AGG, bool ZOH>
hipError_t launch_scan_g(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  switch (dm.groups) {
    case 1: return launch_scan_k<N, 1, IO, AGG, ZOH>(dm, p, s);
    case 2: if constexpr (N >= 2) return launch_scan_k<N, 2, IO, AGG, ZOH>(dm, p, s); else break;
    case 4: if constexpr (N >= 4) return launch_scan_k<N, 4, IO, AGG, ZOH>(dm, p, s); else break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename IO, bool AGG, bool ZOH>
hipError_t launch_scan_n(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  switch (dm.dstate) {
    case 1: return launch_scan_g<1, IO, AGG, ZOH>(dm, p, s);
    case 2: return launch_scan_g<2, IO, AGG, ZOH>(dm, p, s);
    case 4: return launch_scan_g<4, IO, AGG, ZOH>(dm, p, s);
    case 8: return launch_scan_g<8, IO, AGG, ZOH>(dm, p, s);
    case 16: return launch_scan_g<16, IO, AGG, ZOH>(dm, p, s);
    default: return hipErrorInvalidValue;
  }
}

// Entry used by the instantiating translation units.
template <typename IO, bool ZOH>
hipError_t launch_scan_impl(const ScanDims& dm, const ScanPtrs& p, bool aggregate, hipStream_t s) {
  return aggregate ? launch_scan_n<IO, true, ZOH>(dm, p, s) : launch_scan_n<IO, false, ZOH>(dm, p, s);
}

}  // namespace scan_detail
}  // namespace ssscan
