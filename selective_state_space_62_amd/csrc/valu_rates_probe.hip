// Issue-rate probe for the gfx950 vector ALU (measurement tooling, not part of
// the scan library's ABI).
//
// The scan's roofline needs constants that no data sheet states: how many
// hardware exponentials (v_exp_f32) the chip retires per second, how many fp32
// multiplies and fused multiply-adds (unpacked), what a DPP cross-lane add
// costs, and whether transcendentals overlap with the other VALU work.  Each
// mode below keeps CH independent dependency chains per lane and does nothing
// else in its loop; the launch shape sets the waves per SIMD (one wave per SIMD
// per 256-thread workgroup and 256 workgroups).
//   0  exp2 only                      a = 2^(-a)              (converges near 0.64)
//   1  fma only, literal operand      b = 0.999 b + 0.0005    (converges to 0.5)
//   2  both in every wave             one exp2 and one fma per chain step
//   3  both, in separate waves        even waves exp2, odd waves fma
//   4  fma only, one chain            the dependent-issue latency
//   5  fma only, three VGPR operands  b = b * p + q
//   6  mul only                       b = b * p
//   7  DPP add only                   b = b + (b of the neighbour lane)
//   8  exp2 and four fmas             the scan's ratio of transcendentals to the rest
//   9  the scan's state step          per step: d, dx updated (2 ops); per component
//                                     E = 2^(d A), h = E h + dx B, acc = C h + acc (5 ops)
//  10  exp2 and four fmas, in bursts  per round 8 exp2 back to back, then 32 fmas
//  11  rcp only
//  12  log2 and an add                a = log2(a + 1.5)
//  13  the scan's work split by kind  even waves: a = 2^(-a p) (mul, exp2); odd waves:
//                                     three fmas/muls per step (no transcendental)
//  14  the same work in every wave    a = 2^(-a p) and the three ops, interleaved
//  15  long bursts                    per round 8 exp2 back to back, then 128 fmas
//  16  sparse exponentials            per round 8 exp2, each followed by 16 fmas
//  17  one exp2 before the loop       then fmas only (as mode 5)
// Rates are lane-operations per second over all CUs: a mode's operations per
// lane per launch, times the lanes, over the average launch time.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kRounds = 16;   // chain steps per loop iteration

template <int MODE, int CH>
__global__ __launch_bounds__(256) void rate_kernel(float* __restrict__ out, int iters) {
  float a[CH], b[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    a[i] = 0.5f + 0.01f * i + 1e-7f * threadIdx.x;
    b[i] = 0.25f + 0.01f * i + 1e-7f * threadIdx.x;
  }
  // per-lane operands the compiler cannot fold into literals
  const float p = 0.999f + 1e-9f * (float)(threadIdx.x & 7);
  const float q = 0.0005f + 1e-9f * (float)(threadIdx.x & 3);
  float A[CH], Bc[CH];   // mode 9: per-lane decay rates and input weights
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    A[i] = -1.0f - 0.25f * i - 1e-7f * threadIdx.x;
    Bc[i] = 0.3f + 0.1f * i;
  }
  float d = 0.05f, dx = 0.01f;
  if constexpr (MODE == 17) {
    a[0] = __builtin_amdgcn_exp2f(-a[0]);
    asm volatile("" : "+v"(a[0]));
  }
  // wave-uniform, so mode 3 branches once per launch, not per step
  const bool exp_wave = (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1) == 0;
  if constexpr (MODE == 13 || MODE == 14) {
    float c[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) c[i] = 0.1f * i;
    auto step_e = [&](int i) { a[i] = __builtin_amdgcn_exp2f(-(a[i] * p)); };
    auto step_s = [&](int i) {
      b[i] = fmaf(b[i], p, q);
      c[i] = fmaf(c[i], p, b[i]);
      b[i] = b[i] * p;
    };
    if (MODE == 14) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
#pragma unroll
          for (int i = 0; i < CH; ++i) {
            step_e(i);
            step_s(i);
          }
        }
      }
    } else if (exp_wave) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
#pragma unroll
          for (int i = 0; i < CH; ++i) step_e(i);
        }
      }
    } else {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
#pragma unroll
          for (int i = 0; i < CH; ++i) step_s(i);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) b[i] += c[i];
  } else if (MODE == 3 && !exp_wave) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
#pragma unroll
        for (int i = 0; i < CH; ++i) b[i] = fmaf(b[i], 0.999f, 0.0005f);
      }
    }
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          if constexpr (MODE == 0 || MODE == 2 || MODE == 3) a[i] = __builtin_amdgcn_exp2f(-a[i]);
          if constexpr (MODE == 1 || MODE == 2 || MODE == 4) b[i] = fmaf(b[i], 0.999f, 0.0005f);
          if constexpr (MODE == 5 || MODE == 17) b[i] = fmaf(b[i], p, q);
          if constexpr (MODE == 6) b[i] = b[i] * p;
          if constexpr (MODE == 7) b[i] += __builtin_amdgcn_update_dpp(0.0f, b[i], 0xB1, 0xf, 0xf, false);
          if constexpr (MODE == 8) {
            a[i] = __builtin_amdgcn_exp2f(-a[i]);
            b[i] = fmaf(b[i], p, q);
            b[i] = fmaf(b[i], p, q);
            b[i] = fmaf(b[i], p, q);
            b[i] = fmaf(b[i], p, q);
          }
          if constexpr (MODE == 11) a[i] = __builtin_amdgcn_rcpf(a[i]);   // alternates between a0 and 1/a0
          if constexpr (MODE == 12) a[i] = __builtin_amdgcn_logf(a[i] + 1.5f);
          if constexpr (MODE == 9) {
            // a: state h, b: readout partial; the step's Delta is carried in d
            const float E = __builtin_amdgcn_exp2f(d * A[i]);
            a[i] = fmaf(E, a[i], dx * Bc[i]);
            b[i] = fmaf(Bc[i] + 0.5f, a[i], b[i]);
          }
        }
        if constexpr (MODE == 9) {
          d = fmaf(d, p, q);   // the next step's Delta and Delta x
          dx = d * q;
        }
        if constexpr (MODE == 15) {
#pragma unroll
          for (int i = 0; i < CH; ++i) a[i] = __builtin_amdgcn_exp2f(-a[i]);
#pragma unroll
          for (int k = 0; k < 16; ++k) {
#pragma unroll
            for (int i = 0; i < CH; ++i) b[i] = fmaf(b[i], p, q);
          }
        }
        if constexpr (MODE == 16) {
#pragma unroll
          for (int i = 0; i < CH; ++i) {
            a[i] = __builtin_amdgcn_exp2f(-a[i]);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
#pragma unroll
              for (int j = 0; j < CH; ++j) b[j] = fmaf(b[j], p, q);
            }
          }
        }
        if constexpr (MODE == 10) {
#pragma unroll
          for (int i = 0; i < CH; ++i) a[i] = __builtin_amdgcn_exp2f(-a[i]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int i = 0; i < CH; ++i) b[i] = fmaf(b[i], p, q);
          }
        }
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) s += a[i] + b[i];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Operations one lane performs per loop round (all chains) in each mode (a wave
// of mode 3 does one per chain).
constexpr int kModes = 18;
// mode 13: an average lane does (2 + 3) / 2 ops per chain step
constexpr double kOpsPerRound[kModes] = {8, 8, 16, 8, 1, 8, 8, 8, 40, 2 + 4 * 5, 40, 8, 16, 20, 40, 136, 136, 8};

template <int MODE, int CH>
hipError_t launch(int workgroups, int iters, float* out) {
  hipLaunchKernelGGL((rate_kernel<MODE, CH>), dim3(workgroups), dim3(256), 0, 0, out, iters);
  return hipGetLastError();
}

hipError_t launch_mode(int mode, int workgroups, int iters, float* out) {
  switch (mode) {
    case 0: return launch<0, 8>(workgroups, iters, out);
    case 1: return launch<1, 8>(workgroups, iters, out);
    case 2: return launch<2, 8>(workgroups, iters, out);
    case 3: return launch<3, 8>(workgroups, iters, out);
    case 4: return launch<4, 1>(workgroups, iters, out);
    case 5: return launch<5, 8>(workgroups, iters, out);
    case 6: return launch<6, 8>(workgroups, iters, out);
    case 7: return launch<7, 8>(workgroups, iters, out);
    case 8: return launch<8, 8>(workgroups, iters, out);
    case 9: return launch<9, 4>(workgroups, iters, out);
    case 10: return launch<10, 8>(workgroups, iters, out);
    case 11: return launch<11, 8>(workgroups, iters, out);
    case 12: return launch<12, 8>(workgroups, iters, out);
    case 13: return launch<13, 8>(workgroups, iters, out);
    case 14: return launch<14, 8>(workgroups, iters, out);
    case 15: return launch<15, 8>(workgroups, iters, out);
    case 16: return launch<16, 8>(workgroups, iters, out);
    case 17: return launch<17, 8>(workgroups, iters, out);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

extern "C" {

// Number of probe modes.
int ss_probe_valu_modes(void) { return kModes; }

// Runs one mode on the current device: one untimed launch, then `reps` timed
// launches of `workgroups` workgroups of 256 threads with `iters` loop
// iterations per lane.  Writes the average launch time in milliseconds to
// *ms_out and the operations one lane performs per launch to *ops_out.
// Returns 0, or the HIP error code.
int ss_probe_valu_mode(int mode, int workgroups, int iters, int reps, double* ms_out, double* ops_out) {
  if (mode < 0 || mode >= kModes || workgroups < 1 || iters < 1 || reps < 1 || !ms_out || !ops_out)
    return (int)hipErrorInvalidValue;
  float* out = nullptr;
  hipError_t e = hipMalloc(&out, (size_t)workgroups * 256 * sizeof(float));
  if (e != hipSuccess) return (int)e;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if ((e = hipEventCreate(&e0)) == hipSuccess && (e = hipEventCreate(&e1)) == hipSuccess &&
      (e = launch_mode(mode, workgroups, iters, out)) == hipSuccess && (e = hipEventRecord(e0, 0)) == hipSuccess) {
    for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch_mode(mode, workgroups, iters, out);
    if (e == hipSuccess && (e = hipEventRecord(e1, 0)) == hipSuccess && (e = hipEventSynchronize(e1)) == hipSuccess) {
      float ms = 0.0f;
      if ((e = hipEventElapsedTime(&ms, e0, e1)) == hipSuccess) {
        *ms_out = (double)ms / reps;
        *ops_out = (double)iters * kRounds * kOpsPerRound[mode];
      }
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(out);
  return (int)e;
}

}  // extern "C"
