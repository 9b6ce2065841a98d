// One-token decode step (ss_state_update) for gfx950.
//
// Generation needs a single state update per token (tellworld.net summary of the
// Mamba paper, section "Architecture"); the update is the scan's recurrence for
// one token (reader's notes, kurisu.si, "What they did": Delta from a softplus,
// Abar = exp(Delta A)), with the fp32 state read from and written back to HBM.
//
// The step moves about 136 bytes per (b, d) at N = 16 (64 B of state in, 64 B
// out, 8 B of x, dt, z, y) against ~120 VALU slots, so it is bound by the state's
// read-modify-write traffic.  Lanes map to (channel, group of 4 state
// components): each lane moves one 16-byte piece of the state and a wave covers
// 1 KB of contiguous state, so every load and store is fully coalesced.  The
// readout of the N components is summed across the channel's lanes with DPP
// quad permutes in a fixed order.  A (dim, N) is re-read per batch row from L2.
// The state is streamed with non-temporal loads and stores (it is touched once
// per step), and a bounded grid of workgroups strides over the items, which
// kept more bytes in flight than one short-lived workgroup per 64 channels.
#include "device_common.h"
#include "internal.h"

#ifndef DECODE_UNROLL
#define DECODE_UNROLL 1
#endif
#ifndef DECODE_BLOCKS
#define DECODE_BLOCKS 2048
#endif

namespace ssscan {
namespace {

using namespace dev;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Load Q consecutive elements of a (batch, N) row of B or C as floats (one
// vector load when Q * sizeof(element) is 8 or 16 bytes).
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

// Grid-stride over waves: each wave handles U x 64 consecutive (channel,
// component group) items per iteration, all U state loads issued before any
// arithmetic (more bytes in flight per wave); the loop bound is wave-uniform, so
// every lane of a channel is active for the DPP sum.
template <int N, typename IO, int U, bool ZOH>
__global__ __launch_bounds__(256) void state_update_kernel(
    int64_t nch, int64_t dim, float* __restrict__ state, const typename IO::T* __restrict__ x,
    const typename IO::T* __restrict__ dt, const typename IO::T* __restrict__ z,
    const typename IO::T* __restrict__ B, const typename IO::T* __restrict__ C, const float* __restrict__ A,
    const float* __restrict__ Dskip, const float* __restrict__ dt_bias, typename IO::T* __restrict__ y) {
  constexpr int Q = N < 4 ? N : 4;   // state components per lane
  constexpr int K = N / Q;           // lanes per channel (1, 2 or 4), adjacent within a quad
  const int64_t items = nch * K;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~63)) * U;
  const int64_t wstride = (int64_t)gridDim.x * blockDim.x * U;
  for (int64_t wb = wave0; wb < items; wb += wstride) {
    bool act[U];
    int64_t ch[U], b[U], d[U];
    int j[U];
    float st[U][Q], a2[U][Q], bq[U][Q], cq[U][Q], xv[U], dtv[U], zv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t it = wb + u * 64 + lane;
      act[u] = it < items;
      const int64_t itc = act[u] ? it : items - 1;   // inactive lanes work on a valid item, store nothing
      ch[u] = itc / K;
      j[u] = (int)(itc - ch[u] * K);
      b[u] = ch[u] / dim;
      d[u] = ch[u] - b[u] * dim;
      const float* sp = state + ch[u] * N + j[u] * Q;
      if constexpr (Q == 4) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp));
        st[u][0] = v[0]; st[u][1] = v[1]; st[u][2] = v[2]; st[u][3] = v[3];
      } else {
#pragma unroll
        for (int q = 0; q < Q; ++q) st[u][q] = sp[q];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (Q == 4) {
        const float4 av = *reinterpret_cast<const float4*>(A + d[u] * N + j[u] * Q);
        a2[u][0] = av.x; a2[u][1] = av.y; a2[u][2] = av.z; a2[u][3] = av.w;
      } else {
#pragma unroll
        for (int q = 0; q < Q; ++q) a2[u][q] = A[d[u] * N + j[u] * Q + q];
      }
      load_q<IO, Q>(B + b[u] * N + j[u] * Q, bq[u]);
      load_q<IO, Q>(C + b[u] * N + j[u] * Q, cq[u]);
      xv[u] = load_one<IO>(x, ch[u]);
      dtv[u] = load_one<IO>(dt, ch[u]);
      zv[u] = z ? load_one<IO>(z, ch[u]) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float bias2 = dt_bias ? dt_bias[d[u]] * kLog2e : 0.0f;
      const float skip = Dskip ? Dskip[d[u]] : 0.0f;
      const float delta = softplus_dt(dtv[u], bias2);
      const float dx = delta * xv[u];
      float acc = 0.0f;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float u2 = delta * (a2[u][q] * kLog2e);
        const float E = __builtin_amdgcn_exp2f(u2);
        float in = dx * bq[u][q];                  // first order: Bbar x = Delta B x
        if constexpr (ZOH) in *= zoh_phi(u2, E);   // zero-order hold: (e^u - 1)/u Delta B x
        st[u][q] = fmaf(E, st[u][q], in);
        acc = fmaf(cq[u][q], st[u][q], acc);
      }
      // sum the channel's K partial readouts (lanes are adjacent inside one quad)
      if constexpr (K >= 2) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0xB1, 0xf, 0xf, false);  // [1,0,3,2]
      if constexpr (K == 4) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0x4E, 0xf, 0xf, false);  // [2,3,0,1]
      if (act[u]) {
        float* sp = state + ch[u] * N + j[u] * Q;
        if constexpr (Q == 4) {
          const f32x4 v = {st[u][0], st[u][1], st[u][2], st[u][3]};
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(sp));
        } else {
#pragma unroll
          for (int q = 0; q < Q; ++q) sp[q] = st[u][q];
        }
        if (j[u] == 0) {
          float out = fmaf(skip, xv[u], acc);
          if (z) out *= silu(zv[u]);
          store_one<IO>(y, ch[u], out);
        }
      }
    }
  }
}

template <int N, typename IO, bool ZOH>
hipError_t launch_t(int64_t nch, int64_t dim, float* state, const void* x, const void* dt, const void* z,
                    const void* B, const void* C, const float* A, const float* Dskip, const float* dt_bias, void* y,
                    hipStream_t s) {
  using E = typename IO::T;
  constexpr int K = N < 4 ? 1 : N / 4;
  constexpr int U = DECODE_UNROLL;
  const int64_t threads = (nch * K + U - 1) / U;
  int64_t blocks = (threads + 255) / 256;
  // a bounded grid (DECODE_BLOCKS workgroups); the grid-stride loop covers the rest
  const int64_t cap = DECODE_BLOCKS;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((state_update_kernel<N, IO, U, ZOH>), dim3((unsigned)blocks), dim3(256), 0, s, nch, dim, state,
                     (const E*)x, (const E*)dt, (const E*)z, (const E*)B, (const E*)C, A, Dskip, dt_bias, (E*)y);
  return hipGetLastError();
}

template <typename IO, bool ZOH>
hipError_t launch_n(int64_t nch, int64_t dim, int dstate, float* state, const void* x, const void* dt, const void* z,
                    const void* B, const void* C, const float* A, const float* Dskip, const float* dt_bias, void* y,
                    hipStream_t s) {
  switch (dstate) {
    case 1: return launch_t<1, IO, ZOH>(nch, dim, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 2: return launch_t<2, IO, ZOH>(nch, dim, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 4: return launch_t<4, IO, ZOH>(nch, dim, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 8: return launch_t<8, IO, ZOH>(nch, dim, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 16: return launch_t<16, IO, ZOH>(nch, dim, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_state_update(int64_t batch, int64_t dim, int dstate, int io, bool zoh, float* state,
                               const void* x, const void* dt, const void* z, const void* B, const void* C,
                               const float* A, const float* Dskip, const float* dt_bias, void* y, hipStream_t s) {
  const int64_t nch = batch * dim;
  if (io == kIoBf16) {
    return zoh ? launch_n<BF16, true>(nch, dim, dstate, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s)
               : launch_n<BF16, false>(nch, dim, dstate, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
  }
  return zoh ? launch_n<F32, true>(nch, dim, dstate, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s)
             : launch_n<F32, false>(nch, dim, dstate, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
}

}  // namespace ssscan
