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
//    has K adjacent lanes (K = 1, 2 or 4) in every wave.  The N state components
//    are split into G*K groups: lane k of a channel in wave w owns group w K + k.
//    K = 2 halves the channels per workgroup, so there are twice as many equal
//    workgroups (for the 2.8B-shaped layer 1280, exactly 5 per CU, where 640
//    leave half the CUs with one more than the rest); K = 4 (one component per
//    lane) doubles them again for layers with too few channels to fill the chip.
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
//    K lanes of a channel add their readouts with DPP adds (one for K = 2, two
//    for K = 4), and each wave
//    writes one partial readout per (token, channel) to LDS.  The owner of a
//    token sums the G partials in a fixed order (deterministic results), adds the
//    skip term, applies the gate and writes its span of y.
//  * The per-(token, state) work is exp2, two multiplies and two FMAs; transcendentals
//    are half-rate on gfx950 and do not co-issue with FMAs, so the kernel is bound
//    by VALU issue, not by HBM.
//  * The input term is first order (Bbar x = Delta B x) or, in the zero-order-hold
//    entry points, phi(Delta A) Delta B x with phi(u) = (e^u - 1)/u: the
//    discretisation under which the notes' Theorem 1 (selection is gating) holds
//    exactly.  The kernels are instantiated per I/O dtype and discretisation in
//    scan_{bf16,f32}_{euler,zoh}.hip from scan_kernel.h.
//  * dt may hold one value per (batch row, token), shared by the row's channels
//    (the broadcast Delta of the notes); the kernel then reads it by row.
//  * For a training step the forward can also store the state entering every
//    backward chunk (a separate instantiation, CKPT_K, so the plain scan keeps
//    its registers); the backward then skips its own checkpoint sweep.
//  * Long sequences with few channels are cut into chunks: an aggregate pass
//    (AGG = true) gives each chunk's end state from a zero start and its sum of
//    Delta; combine_kernel runs the exclusive scan of (exp(A sum Delta), h_end)
//    pairs across chunks; the full pass then rescans every chunk from its true
//    initial state.  The combine (P1, h1) o (P2, h2) = (P1 P2, P2 h1 + h2) follows
//    from the linearity of the recurrence.
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

// Exclusive scan of the chunk aggregates: h_in[c] = the state entering chunk
// c.  A chunk's pair (P, H) = (exp(A * sum Delta_c), its end state from a zero
// start) acts on a state as h -> P h + H; composing an earlier pair with a later
// one gives (P1 P2, P2 H1 + H2), an associative operation, so the scan runs in
// parallel.  One wave takes one (b, d): lane l owns state component n = l % N
// and the l / N-th of R = 64 / N contiguous groups of chunks.  Each lane folds
// its group into one pair (the decay from the group's summed Delta), the waves'
// R groups are scanned across lanes N apart with cross-lane shifts
// (ds_bpermute), and each lane then walks its group from the state entering
// it, writing h_in.  The loads and stores of one chunk are N adjacent floats.
template <int N>
__global__ __launch_bounds__(256) void combine_kernel(int64_t nch, int64_t dim, int num_chunks,
                                                      const float* __restrict__ A, const float* __restrict__ agg_h,
                                                      const float* __restrict__ agg_s, const float* __restrict__ h0,
                                                      float* __restrict__ h_in) {
  constexpr int R = 64 / N;   // groups of chunks per (b, d)
  const int64_t ch = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;   // (b, d) of this wave
  if (ch >= nch) return;
  const int lane = threadIdx.x & 63;
  const int n = lane % N;
  const int g = lane / N;
  const int64_t d = ch % dim;
  const float a2 = A[d * N + n] * dev::kLog2e;
  const int per = (num_chunks + R - 1) / R;
  const int c0 = g * per < num_chunks ? g * per : num_chunks;
  const int c1 = c0 + per < num_chunks ? c0 + per : num_chunks;
  const float* __restrict__ hs = agg_h + ch * (int64_t)num_chunks * N + n;
  const float* __restrict__ ss = agg_s + ch * (int64_t)num_chunks;

  // this lane's group as one pair: H from a zero start, S = the group's sum of Delta
  float H = 0.0f, S = 0.0f;
  for (int c = c0; c < c1; ++c) {
    const float sc = ss[c];
    H = fmaf(__builtin_amdgcn_exp2f(a2 * sc), H, hs[(int64_t)c * N]);
    S += sc;
  }
  float P = __builtin_amdgcn_exp2f(a2 * S);
  // inclusive scan over the R groups (lanes N apart): Hillis-Steele doubling
#pragma unroll
  for (int off = N; off < 64; off *= 2) {
    const float Pp = __shfl_up(P, off, 64);
    const float Hp = __shfl_up(H, off, 64);
    if (lane >= off) {
      H = fmaf(P, Hp, H);   // (Pp, Hp) then (P, H)
      P = Pp * P;
    }
  }
  // exclusive: the groups before this one
  float Pe = __shfl_up(P, N, 64), He = __shfl_up(H, N, 64);
  if (g == 0) {
    Pe = 1.0f;
    He = 0.0f;
  }
  float h = fmaf(Pe, h0 ? h0[ch * N + n] : 0.0f, He);
  float* __restrict__ out = h_in + ch * (int64_t)num_chunks * N + n;
  for (int c = c0; c < c1; ++c) {
    out[(int64_t)c * N] = h;
    h = fmaf(__builtin_amdgcn_exp2f(a2 * ss[c]), h, hs[(int64_t)c * N]);
  }
}

// A shard's aggregate from its chunks' aggregates, one lane per (b, d, n):
// h = state after the last chunk from a zero start, and (n == 0) the sum of Delta.
__global__ __launch_bounds__(256) void shard_reduce_kernel(int64_t nstate, int64_t dim, int dstate, int num_chunks,
                                                           const float* __restrict__ A,
                                                           const float* __restrict__ agg_h,
                                                           const float* __restrict__ agg_s, float* __restrict__ h_end,
                                                           float* __restrict__ dsum) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nstate) return;
  const int64_t ch = i / dstate;
  const int n = (int)(i - ch * dstate);
  const int64_t d = ch % dim;
  const float a2 = A[d * dstate + n] * dev::kLog2e;
  float h = 0.0f, s = 0.0f;
  for (int c = 0; c < num_chunks; ++c) {
    const float sc = agg_s[ch * num_chunks + c];
    h = fmaf(__builtin_amdgcn_exp2f(a2 * sc), h, agg_h[(ch * num_chunks + c) * dstate + n]);
    s += sc;
  }
  h_end[i] = h;
  if (n == 0) dsum[ch] = s;
}

// The state entering each of a sequence's shards, one lane per (b, d, n):
// h_in[0] = h0, h_in[s + 1] = exp(A dsum[s]) h_in[s] + h_end[s]; h_final = the
// state after the last shard.  Shard-major layouts: dsum (nshards, batch, dim),
// h_end and h_in (nshards, batch, dim, N).
__global__ __launch_bounds__(256) void shard_combine_kernel(int64_t nstate, int64_t dim, int dstate,
                                                            int64_t nshards, const float* __restrict__ A,
                                                            const float* __restrict__ dsum,
                                                            const float* __restrict__ h_end,
                                                            const float* __restrict__ h0, float* __restrict__ h_in,
                                                            float* __restrict__ h_final) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nstate) return;
  const int64_t ch = i / dstate;
  const int n = (int)(i - ch * dstate);
  const int64_t d = ch % dim;
  const int64_t nch = nstate / dstate;
  const float a2 = A[d * dstate + n] * dev::kLog2e;
  float h = h0 ? h0[i] : 0.0f;
  for (int64_t s = 0; s < nshards; ++s) {
    if (h_in) h_in[s * nstate + i] = h;
    h = fmaf(__builtin_amdgcn_exp2f(a2 * dsum[s * nch + ch]), h, h_end[s * nstate + i]);
  }
  if (h_final) h_final[i] = h;
}

__global__ __launch_bounds__(256) void copy_state_kernel(int64_t count, const float* __restrict__ src,
                                                         float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) dst[i] = src ? src[i] : 0.0f;
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

hipError_t launch_scan(const ScanDims& dm, const ScanPtrs& p, bool aggregate, bool zoh, hipStream_t s) {
  if (dm.io == kIoBf16)
    return zoh ? launch_scan_bf16_zoh(dm, p, aggregate, s) : launch_scan_bf16_euler(dm, p, aggregate, s);
  return zoh ? launch_scan_f32_zoh(dm, p, aggregate, s) : launch_scan_f32_euler(dm, p, aggregate, s);
}

hipError_t launch_combine(const ScanDims& dm, const float* A, const float* agg_h, const float* agg_s,
                          const float* h0, float* h_in, hipStream_t s) {
  const int64_t nch = dm.batch * dm.dim;
  const dim3 grid((unsigned)((nch + 3) / 4));   // four waves per workgroup, one (b, d) per wave
  switch (dm.dstate) {
    case 1: hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(256), 0, s, nch, dm.dim, dm.num_chunks, A, agg_h, agg_s, h0, h_in); break;
    case 2: hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(256), 0, s, nch, dm.dim, dm.num_chunks, A, agg_h, agg_s, h0, h_in); break;
    case 4: hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(256), 0, s, nch, dm.dim, dm.num_chunks, A, agg_h, agg_s, h0, h_in); break;
    case 8: hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, s, nch, dm.dim, dm.num_chunks, A, agg_h, agg_s, h0, h_in); break;
    case 16: hipLaunchKernelGGL(combine_kernel<16>, grid, dim3(256), 0, s, nch, dm.dim, dm.num_chunks, A, agg_h, agg_s, h0, h_in); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_shard_reduce(const ScanDims& dm, const float* A, const float* agg_h, const float* agg_s,
                               float* h_end, float* dsum, hipStream_t s) {
  const int64_t nstate = dm.batch * dm.dim * dm.dstate;
  hipLaunchKernelGGL(shard_reduce_kernel, dim3((unsigned)((nstate + 255) / 256)), dim3(256), 0, s, nstate, dm.dim,
                     dm.dstate, dm.num_chunks, A, agg_h, agg_s, h_end, dsum);
  return hipGetLastError();
}

hipError_t launch_shard_combine(int64_t batch, int64_t dim, int dstate, int64_t nshards, const float* A,
                                const float* dsum, const float* h_end, const float* h0, float* h_in, float* h_final,
                                hipStream_t s) {
  const int64_t nstate = batch * dim * dstate;
  hipLaunchKernelGGL(shard_combine_kernel, dim3((unsigned)((nstate + 255) / 256)), dim3(256), 0, s, nstate, dim,
                     dstate, nshards, A, dsum, h_end, h0, h_in, h_final);
  return hipGetLastError();
}

hipError_t launch_copy_state(int64_t count, const float* src, float* dst, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, count, src, dst);
  return hipGetLastError();
}

}  // namespace ssscan
