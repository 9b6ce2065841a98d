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
#include "device_common.h"
#include "internal.h"

namespace ssscan {
namespace {

using namespace dev;

template <int N, typename IO>
__global__ __launch_bounds__(256) void state_update_kernel(
    int64_t nch, int64_t dim, float* __restrict__ state, const typename IO::T* __restrict__ x,
    const typename IO::T* __restrict__ dt, const typename IO::T* __restrict__ z,
    const typename IO::T* __restrict__ B, const typename IO::T* __restrict__ C, const float* __restrict__ A,
    const float* __restrict__ Dskip, const float* __restrict__ dt_bias, typename IO::T* __restrict__ y) {
  constexpr int Q = N < 4 ? N : 4;   // state components per lane
  constexpr int K = N / Q;           // lanes per channel (1, 2 or 4), adjacent within a quad
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t chr = gid / K;
  const int j = (int)(gid - chr * K);
  const bool act = chr < nch;
  const int64_t ch = act ? chr : nch - 1;   // inactive lanes work on a valid channel, store nothing
  const int64_t b = ch / dim;
  const int64_t d = ch - b * dim;

  float st[Q], a2[Q], bq[Q], cq[Q];
  float* sp = state + ch * N + j * Q;
  if constexpr (Q == 4) {
    const float4 v = *reinterpret_cast<const float4*>(sp);
    st[0] = v.x; st[1] = v.y; st[2] = v.z; st[3] = v.w;
    const float4 av = *reinterpret_cast<const float4*>(A + d * N + j * Q);
    a2[0] = av.x; a2[1] = av.y; a2[2] = av.z; a2[3] = av.w;
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      st[q] = sp[q];
      a2[q] = A[d * N + j * Q + q];
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    a2[q] *= kLog2e;
    bq[q] = load_one<IO>(B, b * N + j * Q + q);
    cq[q] = load_one<IO>(C, b * N + j * Q + q);
  }
  const float xv = load_one<IO>(x, ch);
  const float delta = softplus_dt(load_one<IO>(dt, ch), dt_bias ? dt_bias[d] * kLog2e : 0.0f);
  const float dx = delta * xv;
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const float E = __builtin_amdgcn_exp2f(delta * a2[q]);
    st[q] = fmaf(E, st[q], dx * bq[q]);
    acc = fmaf(cq[q], st[q], acc);
  }
  // sum the channel's K partial readouts (lanes are adjacent inside one quad)
  if constexpr (K >= 2) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
  if constexpr (K == 4) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]

  if (act) {
    if constexpr (Q == 4) {
      *reinterpret_cast<float4*>(sp) = make_float4(st[0], st[1], st[2], st[3]);
    } else {
#pragma unroll
      for (int q = 0; q < Q; ++q) sp[q] = st[q];
    }
    if (j == 0) {
      float out = fmaf(Dskip ? Dskip[d] : 0.0f, xv, acc);
      if (z) out *= silu(load_one<IO>(z, ch));
      store_one<IO>(y, ch, out);
    }
  }
}

template <int N, typename IO>
hipError_t launch_t(int64_t nch, int64_t dim, float* state, const void* x, const void* dt, const void* z,
                    const void* B, const void* C, const float* A, const float* Dskip, const float* dt_bias, void* y,
                    hipStream_t s) {
  using E = typename IO::T;
  constexpr int K = N < 4 ? 1 : N / 4;
  const int64_t threads = nch * K;
  hipLaunchKernelGGL((state_update_kernel<N, IO>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, nch,
                     dim, state, (const E*)x, (const E*)dt, (const E*)z, (const E*)B, (const E*)C, A, Dskip,
                     dt_bias, (E*)y);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_n(int64_t nch, int64_t dim, int dstate, float* state, const void* x, const void* dt, const void* z,
                    const void* B, const void* C, const float* A, const float* Dskip, const float* dt_bias, void* y,
                    hipStream_t s) {
  switch (dstate) {
    case 1: return launch_t<1, IO>(nch, dim, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 2: return launch_t<2, IO>(nch, dim, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 4: return launch_t<4, IO>(nch, dim, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 8: return launch_t<8, IO>(nch, dim, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    case 16: return launch_t<16, IO>(nch, dim, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_state_update(int64_t batch, int64_t dim, int dstate, int io, float* state, const void* x,
                               const void* dt, const void* z, const void* B, const void* C, const float* A,
                               const float* Dskip, const float* dt_bias, void* y, hipStream_t s) {
  const int64_t nch = batch * dim;
  if (io == kIoBf16) return launch_n<BF16>(nch, dim, dstate, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
  return launch_n<F32>(nch, dim, dstate, state, x, dt, z, B, C, A, Dskip, dt_bias, y, s);
}

}  // namespace ssscan
