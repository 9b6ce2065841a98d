// Backward pass of the selective scan (ss_scan_bwd): the first-order
// instantiation of the main kernel (scan_bwd_kernel.h), the reduce kernels that
// finish the cross-block sums, and the launch sequence.
#include "scan_bwd_kernel.h"

namespace ssscan {
namespace {

using namespace dev;

// dB[b, n, t], dC[b, n, t] and, for a per-row dt, ddt[b, t]: the channel
// blocks' partials, in block order.  Partials are (batch, block, chunk, output,
// chunk token) with bwd_part_outputs(N) outputs per chunk of ck tokens.  One
// thread per (b, chunk, output, chunk token) of the nred outputs reduced, in
// that order, so a wave reads a contiguous run of each block's chunk and
// writes runs of ck tokens.
template <typename IO>
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ part, int64_t batch,
                                                            int64_t cblocks, int64_t L, int64_t nck, int ck, int N,
                                                            int nred, typename IO::T* __restrict__ dB,
                                                            typename IO::T* __restrict__ dC,
                                                            typename IO::T* __restrict__ ddt_row) {
  const int64_t npart = bwd_part_outputs(N);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= batch * nck * nred * ck) return;
  const int j = (int)(i % ck);
  const int64_t o = (i / ck) % nred;
  const int64_t k = (i / (ck * nred)) % nck;
  const int64_t b = i / (ck * nred * nck);
  const int64_t t = k * ck + j;
  if (t >= L) return;   // padding tokens of the last chunk
  const int64_t blk = nck * npart * ck;   // one block's partials
  const float* src = part + b * cblocks * blk + (k * npart + o) * ck + j;
  // eight loads in flight per thread (a single chain of dependent load-add
  // pairs left each thread waiting on one load at a time); the sum keeps the
  // block order
  float acc = 0.0f;
  int64_t q = 0;
  for (; q + 8 <= cblocks; q += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + (q + u) * blk);   // read once
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; q < cblocks; ++q) acc += src[q * blk];
  if (o == 2 * N) store_one<IO>(ddt_row, b * L + t, acc);
  else store_one<IO>(o < N ? dB : dC, (b * N + o % N) * L + t, acc);
}

// dA, dDskip and dt_bias's gradient: sums over the (segment, batch row) rows of
// the partials, in row order.
__global__ __launch_bounds__(256) void bwd_reduce_param_kernel(const float* __restrict__ dA_p,
                                                               const float* __restrict__ dD_p,
                                                               const float* __restrict__ dbias_p, int64_t rows,
                                                               int64_t dim, int N, float* __restrict__ dA,
                                                               float* __restrict__ dD, float* __restrict__ dbias) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t na = dim * N;
  if (i < na) {
    if (dA) {
      float acc = 0.0f;
      for (int64_t b = 0; b < rows; ++b) acc += dA_p[b * na + i];
      dA[i] = acc;
    }
  } else if (i < na + dim) {
    const int64_t dd = i - na;
    float a0 = 0.0f, a1 = 0.0f;
    for (int64_t b = 0; b < rows; ++b) {
      a0 += dD_p[b * dim + dd];
      a1 += dbias_p[b * dim + dd];
    }
    if (dD) dD[dd] = a0;
    if (dbias) dbias[dd] = a1;
  }
}

// The adjoint carried into every segment of a split sequence, one lane per
// (b, d, n), from the last segment back: lam_seg[nseg-1] = dh_final (or zero),
// lam_seg[s-1] = exp(A sum Delta_s) lam_seg[s] + M_s.  The decay factor is the
// product of the segment's Abar, as in the forward's combine.
__global__ __launch_bounds__(256) void bwd_adjoint_combine_kernel(int64_t nstate, int64_t dim, int dstate, int nseg,
                                                                  const float* __restrict__ A,
                                                                  const float* __restrict__ dh_final,
                                                                  const float* __restrict__ adj_m,
                                                                  const float* __restrict__ adj_s,
                                                                  float* __restrict__ lam_seg) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nstate) return;
  const int64_t ch = i / dstate;
  const int n = (int)(i - ch * dstate);
  const int64_t d = ch % dim;
  const float a2 = A[d * dstate + n] * kLog2e;
  float mu = dh_final ? dh_final[i] : 0.0f;
  for (int sgi = nseg - 1; sgi >= 0; --sgi) {
    const int64_t k = (ch * nseg + sgi) * dstate + n;
    lam_seg[k] = mu;
    if (sgi > 0) mu = fmaf(__builtin_amdgcn_exp2f(a2 * adj_s[ch * nseg + sgi]), mu, adj_m[k]);
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace

int bwd_lanes_per_channel(int dstate) { return dstate >= 8 ? 2 : 1; }
int bwd_chunk_len(int dstate) { return bwd_chunk_tokens(dstate); }

hipError_t launch_scan_bwd(const BwdDims& dm, const BwdPtrs& p, hipStream_t s) {
  hipError_t e = dm.zoh ? launch_scan_bwd_zoh_main(dm, p, s)
                : (dm.io == kIoBf16) ? bwd_detail::launch_bwd_n<BF16, false>(dm, p, s)
                                     : bwd_detail::launch_bwd_n<F32, false>(dm, p, s);
  if (e != hipSuccess) return e;
  const int nred = 2 * dm.dstate + (dm.dt_row ? 1 : 0);   // outputs to reduce
  const int ck = bwd_chunk_tokens(dm.dstate);
  const int64_t nck = (dm.seqlen + ck - 1) / ck;
  const int64_t nbc = dm.batch * nck * nred * ck;
  if (nbc > 0) {
    const unsigned blocks = (unsigned)((nbc + 255) / 256);
    if (dm.io == kIoBf16)
      hipLaunchKernelGGL((bwd_reduce_bc_kernel<BF16>), dim3(blocks), dim3(256), 0, s, p.part, dm.batch, dm.cblocks,
                         dm.seqlen, nck, ck, dm.dstate, nred, static_cast<uint16_t*>(p.dB),
                         static_cast<uint16_t*>(p.dC), static_cast<uint16_t*>(p.ddt));
    else
      hipLaunchKernelGGL((bwd_reduce_bc_kernel<F32>), dim3(blocks), dim3(256), 0, s, p.part, dm.batch, dm.cblocks,
                         dm.seqlen, nck, ck, dm.dstate, nred, static_cast<float*>(p.dB), static_cast<float*>(p.dC),
                         static_cast<float*>(p.ddt));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t npar = dm.dim * dm.dstate + dm.dim;
  hipLaunchKernelGGL(bwd_reduce_param_kernel, dim3((unsigned)((npar + 255) / 256)), dim3(256), 0, s, p.dA_p, p.dD_p,
                     p.dbias_p, dm.batch * dm.nseg, dm.dim, dm.dstate, p.dA, p.dDskip, p.ddt_bias);
  return hipGetLastError();
}

hipError_t launch_bwd_segment_agg(const BwdDims& dm, const BwdPtrs& p, bool states, hipStream_t s) {
  using namespace bwd_detail;
  if (dm.nseg < 2) return hipSuccess;
  const bool bf = dm.io == kIoBf16;
  if (!states) return bf ? launch_segment_agg_n<BF16, false, false>(dm, p, s) : launch_segment_agg_n<F32, false, false>(dm, p, s);
  if (dm.zoh) return bf ? launch_segment_agg_n<BF16, true, true>(dm, p, s) : launch_segment_agg_n<F32, true, true>(dm, p, s);
  return bf ? launch_segment_agg_n<BF16, false, true>(dm, p, s) : launch_segment_agg_n<F32, false, true>(dm, p, s);
}

hipError_t launch_bwd_adjoint_combine(const BwdDims& dm, const float* A, const float* dh_final, const float* adj_m,
                                      const float* adj_s, float* lam_seg, hipStream_t s) {
  const int64_t nstate = dm.batch * dm.dim * dm.dstate;
  hipLaunchKernelGGL(bwd_adjoint_combine_kernel, dim3((unsigned)((nstate + 255) / 256)), dim3(256), 0, s, nstate,
                     dm.dim, dm.dstate, dm.nseg, A, dh_final, adj_m, adj_s, lam_seg);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* dst, int64_t n, hipStream_t s) {
  if (n <= 0 || !dst) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, n);
  return hipGetLastError();
}

}  // namespace ssscan
