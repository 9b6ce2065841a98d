// Device-side helpers shared by the scan and decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ssscan {
namespace dev {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

// I/O element types.  Both load 16 bytes per lane per span.
struct F32 {
  using T = float;
  static constexpr int kPerSpan = 4;
};
struct BF16 {
  using T = uint16_t;
  static constexpr int kPerSpan = 8;
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float v) {
  const __bf16 b = (__bf16)v;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 v = {lo, hi};
  const b2 r = __builtin_convertvector(v, b2);
  return __builtin_bit_cast(uint32_t, r);
}

// A span is SPAN consecutive elements of one row, loaded or stored with one
// vector access of SPAN * sizeof(element) bytes (16, 8 or 4) and held as 32-bit
// words.
template <typename IO, int SPAN>
struct SpanT {
  static constexpr int kBytes = SPAN * (int)sizeof(typename IO::T);
  static constexpr int kWords = kBytes / 4;
  static_assert(kBytes == 16 || kBytes == 8 || kBytes == 4, "span must be 4, 8 or 16 bytes");
};

// Element i of a span held as 32-bit words.
template <typename IO, int W>
__device__ __forceinline__ float span_elem(const uint32_t (&w)[W], int i) {
  if constexpr (IO::kPerSpan == 4) {
    return __uint_as_float(w[i]);
  } else {
    return (i & 1) ? __uint_as_float(w[i >> 1] & 0xffff0000u) : __uint_as_float(w[i >> 1] << 16);
  }
}

// Load elements [idx, idx + SPAN) of `base`; elements at or beyond `valid`
// (counted from idx) read as zero.  `vec` allows one vector load when the whole
// span is valid (the caller guarantees the alignment then).
template <typename IO, int SPAN>
__device__ __forceinline__ void load_span(const typename IO::T* __restrict__ base, int64_t idx, int valid,
                                          bool vec, uint32_t (&w)[SpanT<IO, SPAN>::kWords]) {
  constexpr int B = SpanT<IO, SPAN>::kBytes;
  if (vec && valid >= SPAN) {
    if constexpr (B == 16) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + idx);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (B == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(base + idx);
      w[0] = v.x; w[1] = v.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(base + idx);
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < SpanT<IO, SPAN>::kWords; ++k) w[k] = 0u;
  if constexpr (IO::kPerSpan == 4) {
#pragma unroll
    for (int i = 0; i < SPAN; ++i)
      if (i < valid) w[i] = __float_as_uint(base[idx + i]);
  } else {
#pragma unroll
    for (int i = 0; i < SPAN; ++i)
      if (i < valid) w[i >> 1] |= (uint32_t)base[idx + i] << ((i & 1) * 16);
  }
}

// Store the first `valid` of SPAN values at base[idx...].
template <typename IO, int SPAN>
__device__ __forceinline__ void store_span(typename IO::T* __restrict__ base, int64_t idx, int valid, bool vec,
                                           const float (&v)[SPAN]) {
  constexpr int B = SpanT<IO, SPAN>::kBytes;
  if (vec && valid >= SPAN) {
    uint32_t o[SpanT<IO, SPAN>::kWords];
    if constexpr (IO::kPerSpan == 4) {
#pragma unroll
      for (int i = 0; i < SPAN; ++i) o[i] = __float_as_uint(v[i]);
    } else {
#pragma unroll
      for (int i = 0; i < SPAN; i += 2) o[i >> 1] = pack_bf16x2(v[i], v[i + 1]);
    }
    if constexpr (B == 16) {
      *reinterpret_cast<uint4*>(base + idx) = make_uint4(o[0], o[1], o[2], o[3]);
    } else if constexpr (B == 8) {
      *reinterpret_cast<uint2*>(base + idx) = make_uint2(o[0], o[1]);
    } else {
      *reinterpret_cast<uint32_t*>(base + idx) = o[0];
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < SPAN; ++i) {
    if (i < valid) {
      if constexpr (IO::kPerSpan == 4) base[idx + i] = v[i];
      else base[idx + i] = (uint16_t)float_to_bf16_bits(v[i]);
    }
  }
}

// Buffer-resource forms of the span load and store, for whole aligned spans:
// the workgroup's rows are one buffer (base and size in scalar registers), the
// lane's row and token offset a 32-bit register offset fixed for the whole
// sequence, and the tile's token offset a scalar offset, so advancing a tile
// costs no vector instructions.  Raw buffer resource word 3 for gfx9-class parts.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferWord3);
}

template <typename IO, int SPAN>
__device__ __forceinline__ void buf_load_span(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              uint32_t (&w)[SpanT<IO, SPAN>::kWords]) {
  constexpr int B = SpanT<IO, SPAN>::kBytes;
  if constexpr (B == 16) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (B == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    w[0] = v[0]; w[1] = v[1];
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  }
}

template <typename IO, int SPAN>
__device__ __forceinline__ void buf_store_span(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                               const float (&v)[SPAN]) {
  constexpr int B = SpanT<IO, SPAN>::kBytes;
  uint32_t o[SpanT<IO, SPAN>::kWords];
  if constexpr (IO::kPerSpan == 4) {
#pragma unroll
    for (int i = 0; i < SPAN; ++i) o[i] = __float_as_uint(v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < SPAN; i += 2) o[i >> 1] = pack_bf16x2(v[i], v[i + 1]);
  }
  if constexpr (B == 16) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 d = {o[0], o[1], o[2], o[3]};
    __builtin_amdgcn_raw_buffer_store_b128(d, r, voff, soff, 0);
  } else if constexpr (B == 8) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    const u2 d = {o[0], o[1]};
    __builtin_amdgcn_raw_buffer_store_b64(d, r, voff, soff, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(o[0], r, voff, soff, 0);
  }
}

template <typename IO>
__device__ __forceinline__ float load_one(const typename IO::T* __restrict__ base, int64_t idx) {
  if constexpr (IO::kPerSpan == 4) return base[idx];
  else return bf16_bits_to_float(base[idx]);
}

template <typename IO>
__device__ __forceinline__ void store_one(typename IO::T* __restrict__ base, int64_t idx, float v) {
  if constexpr (IO::kPerSpan == 4) base[idx] = v;
  else base[idx] = (uint16_t)float_to_bf16_bits(v);
}

// Delta = softplus(dt + dt_bias), given bias2 = dt_bias * log2(e).
// softplus(v) = max(v, 0) + log1p(e^-|v|).  With v2 = v log2(e) and e = 2^-|v2|,
// u = 1 + e is rounded; c = (u - 1) - e is that rounding error exactly, so
// log1p(e) = ln(u) - c/u ~= ln2 * log2(u) - c (u is in [1, 2]; the dropped
// c (1 - 1/u) is below 2^-24 e).  Uses the hardware exp2 and log2.
__device__ __forceinline__ float softplus_dt(float dt, float bias2) {
  const float v2 = fmaf(dt, kLog2e, bias2);
  const float e = __builtin_amdgcn_exp2f(-fabsf(v2));
  const float u = 1.0f + e;
  const float c = (u - 1.0f) - e;
  const float l = __builtin_amdgcn_logf(u);
  return fmaf(fmaxf(v2, 0.0f) + l, kLn2, -c);
}

// phi(u) = (e^u - 1)/u, phi(0) = 1, for the zero-order-hold input term
// Bbar x = (e^(Delta A) - 1)/A B x = phi(Delta A) Delta B x (no division by A,
// so A = 0 gives Delta B x).  Takes u2 = u log2(e) and E = 2^u2 = e^u, which the
// caller already has.  |u| < 1/4: degree-5 Taylor polynomial (the next term is
// below 5e-8 relative); otherwise (E - 1)/u, where E - 1 cancels no digits.
__device__ __forceinline__ float zoh_phi(float u2, float E) {
  const float u = u2 * kLn2;
  float p = fmaf(u, 1.0f / 720.0f, 1.0f / 120.0f);
  p = fmaf(p, u, 1.0f / 24.0f);
  p = fmaf(p, u, 1.0f / 6.0f);
  p = fmaf(p, u, 0.5f);
  p = fmaf(p, u, 1.0f);
  const float q = (E - 1.0f) * __builtin_amdgcn_rcpf(u);
  return fabsf(u) < 0.25f ? p : q;
}

// The zero-order-hold input coefficient itself, c = (e^u - 1)/A = Delta phi(u)
// with u = Delta A, for a caller that holds u2 = u log2(e), E = e^u, Delta and
// inv_a = 1/A (A != 0).  For |u| >= 1/20 it is E inv_a - inv_a, one fma and no
// reciprocal per element: E carries its own rounding, about 7e-8 absolute below
// 1 (1.4e-7 above), so c is within 1.4e-6 relative there (2.9e-6 for A > 0).
// Below that the relative error of E - 1 grows like 7e-8/|u| (E cannot hold
// the low bits of a small u: at |u| = 1e-4 it is 7e-4), so there c = Delta (1 +
// u/2 + u^2/6 + u^3/24), the Taylor polynomial of phi in u2, whose first
// dropped term is below 5.3e-8 relative.  Both are formed and one selected,
// without a branch; A = 0 (u = 0) gives c = Delta.
__device__ __forceinline__ float zoh_coef(float u2, float E, float delta, float inv_a) {
  float p = fmaf(u2, 0.0138760274f, 0.0800755024f);   // ln2^3/24, ln2^2/6
  p = fmaf(p, u2, 0.346573591f);                      // ln2/2
  const float small = fmaf(delta * u2, p, delta);
  const float large = fmaf(E, inv_a, -inv_a);
  return fabsf(u2) < 0.0721347556f ? small : large;   // |u| < 1/20
}

// silu(z) = z / (1 + e^-z).  For z below about -88 the exponential overflows to
// +inf and the result is -0, the correctly rounded limit.
__device__ __forceinline__ float silu(float z) {
  const float s = __builtin_amdgcn_exp2f(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + s);
}

}  // namespace dev
}  // namespace ssscan
