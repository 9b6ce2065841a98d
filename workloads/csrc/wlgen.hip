// Device-side generator of the seeded synthetic workloads (input generation only;
// nothing here computes any step of the selective scan).
//
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
// 1, 2, 3", SC'11), written from its published definition: ten rounds of
//   (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
// with the key bumped by (0x9E3779B9, 0xBB67AE85) between rounds.
// Element i of a stream comes from the block with counter
// (i/8 mod 2^32, i/8 >> 32, stream, step); the block's four 32-bit words give
// eight 16-bit draws, low half first.  A draw j becomes table[j], a 65536-entry
// table built on the host (inverse normal CDF at (j + 0.5)/65536, rounded to the
// output dtype), so device and host produce bit-identical inputs.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(M0, c[0]), lo0 = M0 * c[0];
    const uint32_t hi1 = __umulhi(M1, c[2]), lo1 = M1 * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

template <typename E>
__global__ __launch_bounds__(256) void fill_kernel(const E* __restrict__ table, uint32_t key0, uint32_t key1,
                                                   uint32_t stream, uint32_t step, uint64_t start, uint64_t count,
                                                   E* __restrict__ out) {
  const uint64_t blk = (start >> 3) + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t e0 = blk << 3;
  if (e0 >= start + count) return;
  uint32_t c[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), stream, step};
  philox4x32_10(c, key0, key1);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint64_t e = e0 + k;
    if (e >= start && e < start + count) {
      const uint32_t j = (c[k >> 1] >> ((k & 1) * 16)) & 0xffffu;
      out[e - start] = table[j];
    }
  }
}

// Raw Philox outputs for known-answer checks: one block per thread.
__global__ void philox_kernel(const uint32_t* __restrict__ ctr, const uint32_t* __restrict__ key, uint32_t* out,
                              int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t c[4] = {ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]};
  philox4x32_10(c, key[2 * i], key[2 * i + 1]);
  for (int k = 0; k < 4; ++k) out[4 * i + k] = c[k];
}

}  // namespace

extern "C" {

// Fill out[0, count) with elements [start, start + count) of one stream.
// elem_bytes: 4 (fp32 table) or 2 (bf16 table).  Returns a hipError_t code.
int wl_fill(const void* table, int elem_bytes, uint32_t key0, uint32_t key1, uint32_t stream, uint32_t step,
            uint64_t start, uint64_t count, void* out, void* hip_stream) {
  if (count == 0) return 0;
  const uint64_t blocks = ((start + count + 7) >> 3) - (start >> 3);
  const uint64_t grid = (blocks + 255) / 256;
  if (grid > 0x7fffffffull) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(fill_kernel<uint32_t>, dim3((unsigned)grid), dim3(256), 0, s, (const uint32_t*)table, key0,
                       key1, stream, step, start, count, (uint32_t*)out);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(fill_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, s, (const uint16_t*)table, key0,
                       key1, stream, step, start, count, (uint16_t*)out);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int wl_philox(const uint32_t* ctr, const uint32_t* key, uint32_t* out, int n, void* hip_stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(philox_kernel, dim3((n + 255) / 256), dim3(256), 0, reinterpret_cast<hipStream_t>(hip_stream),
                     ctr, key, out, n);
  return (int)hipGetLastError();
}

}  // extern "C"
