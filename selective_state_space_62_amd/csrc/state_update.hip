// One-token decode step (ss_state_update) for gfx950.
//
// Generation needs a single state update per token (tellworld.net summary of the
// Mamba paper, section "Architecture"); the update is the scan's recurrence for
// one token (reader's notes, kurisu.si, "What they did": Delta from a softplus,
// Abar = exp(Delta A)), with the fp32 state read from and written back to HBM.
//
// The step moves about 136 bytes per (b, d) at N = 16 (64 B of state in, 64 B
// out, 8 B of x, dt, z, y) against ~100 VALU instructions per lane, so it is
// bound by the state's read-modify-write traffic.  Lanes map to (channel, group
// of 4 state components): each lane moves one 16-byte piece of the state and a
// wave covers 1 KB of contiguous state, so every load and store is fully
// coalesced.  The readout of the N components is summed across the channel's
// lanes with DPP quad permutes in a fixed order.  A (dim, N) is re-read per
// batch row from L2.  The state is streamed with non-temporal loads and stores
// (it is touched once per step).  All of an item's loads are issued together,
// and no lane divides: a grid of up to DECODE_BLOCKS workgroups strides over
// (batch row, 64-item piece) pairs advanced by a host-computed quotient and
// remainder.  A wave advances the same piece of two batch rows: A, dt_bias and
// Dskip are read once for both and twice as many independent loads are in
// flight per wave (30.98 -> 29.53 us at the 256 x 5120 x 16 decode shape; four
// rows per wave 29.93 us, eight 33.2 us).  At that shape every wave then has a
// single pair of items: more, short-lived waves measured faster than fewer,
// longer-lived ones.
#include "device_common.h"
#include "internal.h"

#ifndef DECODE_BLOCKS
#define DECODE_BLOCKS 16384
#endif

namespace ssscan {
namespace {

using namespace dev;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Load Q consecutive elements of a (batch, N) row of B or C as floats, with one
// 8- or 16-byte vector load when Q == 4 (the row offsets are multiples of Q).
template <typename IO, int Q>
__device__ __forceinline__ void load_q(const typename IO::T* __restrict__ p, float (&v)[Q]) {
  if constexpr (Q == 4 && IO::kPerSpan == 8) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xffff0000u);
  } else if constexpr (Q == 4 && IO::kPerSpan == 4) {
    const float4 w = *reinterpret_cast<const float4*>(p);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) v[q] = load_one<IO>(p, q);
  }
}

// One lane's operands for one item: Q state components with their A, B and C
// values, and the channel's x, dt, z, dt_bias and Dskip.
template <int Q>
struct Item {
  float st[Q], a2[Q], bq[Q], cq[Q];
  float xv, dtv, zl, bl, sl;
  int64_t ch;
  int j;
  bool act;
};

template <int N, typename IO>
struct Operands {
  int64_t dim, row_items;
  bool dt_row;   // dt is (batch): one value per row, shared by its channels
  float* __restrict__ state;
  const typename IO::T* __restrict__ x;
  const typename IO::T* __restrict__ dt;
  const typename IO::T* __restrict__ z;
  const typename IO::T* __restrict__ B;
  const typename IO::T* __restrict__ C;
  const float* __restrict__ A;
  const float* __restrict__ Dskip;
  const float* __restrict__ dt_bias;
  typename IO::T* __restrict__ y;
};

// Issue every load of item (row b, piece) for this lane.  Optional operands are
// read unconditionally from an always-valid stand-in (x for z, A for the
// per-channel vectors) and selected later, so all loads are in flight at once
// instead of one wait per branch.
template <int N, typename IO, int Q, int K>
__device__ __forceinline__ Item<Q> fetch(const Operands<N, IO>& o, int64_t b, uint32_t piece, int lane) {
  Item<Q> r;
  const int64_t it = (int64_t)piece * 64 + lane;
  r.act = it < o.row_items;
  const int64_t itc = r.act ? it : o.row_items - 1;   // padding lanes work on a valid item, store nothing
  const int64_t d = itc / K;
  r.j = (int)(itc - d * K);
  r.ch = b * o.dim + d;
  const float* sp = o.state + r.ch * N + r.j * Q;
  if constexpr (Q == 4) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp));
    r.st[0] = v[0]; r.st[1] = v[1]; r.st[2] = v[2]; r.st[3] = v[3];
    const float4 av = *reinterpret_cast<const float4*>(o.A + d * N + r.j * Q);
    r.a2[0] = av.x; r.a2[1] = av.y; r.a2[2] = av.z; r.a2[3] = av.w;
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      r.st[q] = sp[q];
      r.a2[q] = o.A[d * N + r.j * Q + q];
    }
  }
  load_q<IO, Q>(o.B + b * N + r.j * Q, r.bq);
  load_q<IO, Q>(o.C + b * N + r.j * Q, r.cq);
  r.xv = load_one<IO>(o.x, r.ch);
  r.dtv = load_one<IO>(o.dt, o.dt_row ? b : r.ch);
  r.zl = load_one<IO>(o.z ? o.z : o.x, r.ch);
  r.bl = (o.dt_bias ? o.dt_bias : o.A)[d];
  r.sl = (o.Dskip ? o.Dskip : o.A)[d];
  return r;
}

// Advance one item by one token and store the new state and the output.
template <int N, typename IO, int Q, int K, bool ZOH>
__device__ __forceinline__ void finish(const Operands<N, IO>& o, Item<Q>& r) {
  float zv = o.z ? r.zl : 0.0f;
  const float bias2 = o.dt_bias ? r.bl * kLog2e : 0.0f;
  float skip = o.Dskip ? r.sl : 0.0f;
  const float delta = softplus_dt(r.dtv, bias2);
  const float dx = delta * r.xv;
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const float u2 = delta * (r.a2[q] * kLog2e);
    const float E = __builtin_amdgcn_exp2f(u2);
    float in = dx * r.bq[q];                   // first order: Bbar x = Delta B x
    if constexpr (ZOH) in *= zoh_phi(u2, E);   // zero-order hold: (e^u - 1)/u Delta B x
    r.st[q] = fmaf(E, r.st[q], in);
    acc = fmaf(r.cq[q], r.st[q], acc);
  }
  // sum the channel's K partial readouts (lanes are adjacent inside one quad)
  if constexpr (K >= 2) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0xB1, 0xf, 0xf, false);  // [1,0,3,2]
  if constexpr (K == 4) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0x4E, 0xf, 0xf, false);  // [2,3,0,1]
  // every lane forms the output; the empty asm pins z and Dskip here, so the
  // compiler cannot sink their loads into the store branch behind a second wait
  // for memory.  The channel's first lane stores the output.
  __asm__ volatile("" : "+v"(zv), "+v"(skip));
  float out = fmaf(skip, r.xv, acc);
  if (o.z) out *= silu(zv);
  if (r.act) {
    float* sp = o.state + r.ch * N + r.j * Q;
    if constexpr (Q == 4) {
      const f32x4 v = {r.st[0], r.st[1], r.st[2], r.st[3]};
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(sp));
    } else {
#pragma unroll
      for (int q = 0; q < Q; ++q) sp[q] = r.st[q];
    }
    if (r.j == 0) store_one<IO>(o.y, r.ch, out);
  }
}

// Work decomposition: lane items are (channel, group of Q state components),
// K = N / Q items per channel, laid out row by row (one row per batch entry,
// dim * K items, padded to whole waves of 64).  Each wave owns one 64-item
// piece of a pair of rows per iteration and strides over (row pair, piece) by
// the grid's wave count; the (row, piece) pair is advanced with a quotient and remainder the
// host precomputes, so no lane divides.  Row and piece are wave-uniform, so all
// K lanes of a channel are active together for the DPP sum.
template <int N, typename IO, bool ZOH>
__global__ __launch_bounds__(256) void state_update_kernel(int64_t batch, uint32_t pieces_per_row,
                                                           uint32_t stride_rows, uint32_t stride_pieces,
                                                           Operands<N, IO> o) {
  constexpr int Q = N < 4 ? N : 4;   // state components per lane
  constexpr int K = N / Q;           // lanes per channel (1, 2 or 4), adjacent within a quad
  const int lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  int64_t b = wave / pieces_per_row;
  uint32_t piece = wave - (uint32_t)b * pieces_per_row;
  // advance (b, piece) by the grid's wave count: stride_rows rows and stride_pieces pieces
  auto advance = [&](int64_t& bb, uint32_t& pp) {
    bb += stride_rows;
    pp += stride_pieces;
    if (pp >= pieces_per_row) {
      pp -= pieces_per_row;
      ++bb;
    }
  };
  // b counts pairs of batch rows: a wave advances the same channels of two rows
  // (A, dt_bias and Dskip are loaded once for both, and both rows' loads are in
  // flight together); an odd batch's last row is a pair of one
  const int64_t pairs = (batch + 1) / 2;
  for (; b < pairs; advance(b, piece)) {
    const int64_t r = 2 * b;
    Item<Q> i0 = fetch<N, IO, Q, K>(o, r, piece, lane);
    if (r + 1 < batch) {
      Item<Q> i1 = fetch<N, IO, Q, K>(o, r + 1, piece, lane);
      finish<N, IO, Q, K, ZOH>(o, i0);
      finish<N, IO, Q, K, ZOH>(o, i1);
    } else {
      finish<N, IO, Q, K, ZOH>(o, i0);
    }
  }
}

template <int N, typename IO, bool ZOH>
hipError_t launch_t(int64_t batch, int64_t dim, bool dt_row, float* state, const void* x, const void* dt, const void* z,
                    const void* B, const void* C, const float* A, const float* Dskip, const float* dt_bias, void* y,
                    hipStream_t s) {
  using E = typename IO::T;
  constexpr int K = N < 4 ? 1 : N / 4;
  constexpr int64_t kWavesPerBlock = 4;
  const int64_t pieces = (dim * K + 63) / 64;
  const int64_t total_waves = (batch + 1) / 2 * pieces;   // waves over (row pair, piece)
  // wave indices and pieces are 32-bit in the kernel
  if (pieces >= (int64_t(1) << 31) || total_waves >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  // a bounded grid (DECODE_BLOCKS workgroups); the grid-stride loop covers the rest
  int64_t blocks = (total_waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > DECODE_BLOCKS) blocks = DECODE_BLOCKS;
  const int64_t grid_waves = blocks * kWavesPerBlock;
  const uint32_t stride_rows = (uint32_t)(grid_waves / pieces);
  const uint32_t stride_pieces = (uint32_t)(grid_waves % pieces);
  const Operands<N, IO> o{dim, dim * K, dt_row, state, (const E*)x, (const E*)dt, (const E*)z,
                          (const E*)B, (const E*)C, A, Dskip, dt_bias, (E*)y};
  hipLaunchKernelGGL((state_update_kernel<N, IO, ZOH>), dim3((unsigned)blocks),
                     dim3(64 * kWavesPerBlock), 0, s, batch, (uint32_t)pieces, stride_rows, stride_pieces, o);
  return hipGetLastError();
}

template <typename IO, bool ZOH>
hipError_t launch_n(int64_t batch, int64_t dim, bool dt_row, int dstate, float* state, const void* x, const void* dt,
                    const void* z,
                    const void* B, const void* C, const float* A, const float* Dskip, const float* dt_bias, void* y,
                    hipStream_t s) {
  switch (dstate) {
    case 1: return launch_t<1, IO, ZOH>(batch, dim, dt_row, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 2: return launch_t<2, IO, ZOH>(batch, dim, dt_row, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 4: return launch_t<4, IO, ZOH>(batch, dim, dt_row, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 8: return launch_t<8, IO, ZOH>(batch, dim, dt_row, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 16: return launch_t<16, IO, ZOH>(batch, dim, dt_row, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_state_update(int64_t batch, int64_t dim, int dstate, int io, bool zoh, bool dt_row, float* state,
                               const void* x, const void* dt, const void* z, const void* B, const void* C,
                               const float* A, const float* Dskip, const float* dt_bias, void* y, hipStream_t s) {
  if (io == kIoBf16) {
    return zoh ? launch_n<BF16, true>(batch, dim, dt_row, dstate, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s)
               : launch_n<BF16, false>(batch, dim, dt_row, dstate, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
  }
  return zoh ? launch_n<F32, true>(batch, dim, dt_row, dstate, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s)
             : launch_n<F32, false>(batch, dim, dt_row, dstate, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
}

}  // namespace ssscan
