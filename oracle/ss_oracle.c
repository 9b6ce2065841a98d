/*
 * CPU oracle for the selective state-space (S6) scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing but the tests, the smoke check of the
 * graft entry point and the benchmark's cpu_baseline leg may load or call this
 * library.  It shares no source, header or helper with the GPU library, and the
 * GPU library never calls it.
 *
 * What it computes — the definition written out, in double precision, one
 * channel at a time and one token at a time, with no blocking or reordering.
 * Sources (page title, then section):
 *  - "Mamba: linear-time sequence modeling with selective state spaces",
 *    reader's notes at kurisu.si, section "What they did", item "Selective SSM
 *    (S6)": the SSM parameters Delta, B and C are computed from the input; Delta
 *    is the softplus of a parameter plus a projection of the input; A stays an
 *    input-independent parameter entering through Abar = exp(Delta*A); because the
 *    system varies in time it is evaluated as a recurrent scan.
 *  - same notes, "Architecture": the recurrent state holds D x N numbers per
 *    sequence (N = 16 in the language models), built from the input.
 *  - "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" summary
 *    at tellworld.net, section "Architecture": generating a token costs a single
 *    state update (the decode entry point below).
 *  - The state space model itself is the classical linear one named on the
 *    tellworld.net page ("Selective state spaces"): h_t = Abar_t h_{t-1} + Bbar_t x_t,
 *    y_t = C_t . h_t.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - Bbar: the pages give only Abar.  Default is the first-order (Euler) form
 *    Bbar x = Delta * B * x.  With zoh != 0 the zero-order-hold form
 *    Bbar x = (exp(Delta*A) - 1)/A * B * x (Delta*B*x when A = 0) is used; it is
 *    the form under which the notes' Theorem 1 (selection = gating) holds.
 *  - skip and gate: y_t = (C_t . h_t + Dskip * x_t) * silu(z_t), silu(z) = z/(1+e^-z),
 *    with the gate applied to the whole sum; z == NULL means no gate.  The gate is
 *    the gated-MLP branch of the Mamba block ("Architecture" in the notes).
 *  - dt_bias is the softplus "parameter": Delta = softplus(dt + dt_bias).
 *
 * Layouts (row-major, last index fastest):
 *   x, dt, z, y      (batch, dim, seqlen)      decode: (batch, dim)
 *   B, C             (batch, dstate, seqlen)   decode: (batch, dstate)
 *   A                (dim, dstate)
 *   Dskip, dt_bias   (dim)                     NULL means all zeros
 *   h0, h_final      (batch, dim, dstate)      NULL h0 means zeros
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SS_ORACLE_VERSION 1

int ss_oracle_version(void) { return SS_ORACLE_VERSION; }

int ss_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* softplus(v) = log(1 + e^v), in the form that neither overflows nor loses
 * the small-argument digits: max(v, 0) + log1p(e^-|v|). */
static double softplus(double v) { return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v))); }

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z) */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* The discretised input term for one state component. */
static double bbar_x(double delta, double a, double abar, double b, double x, int zoh) {
  if (!zoh) return delta * b * x;
  if (a == 0.0) return delta * b * x;
  /* (Abar - 1)/A, with Abar - 1 taken as expm1(Delta*A) to keep its digits */
  (void)abar;
  return expm1(delta * a) / a * b * x;
}

/*
 * Full-sequence scan.  For every (b, d): h = h0[b, d, :] (or 0); for t = 0..L-1:
 *   Delta = softplus(dt[b,d,t] + dt_bias[d])
 *   for n: Abar = exp(Delta * A[d,n]); h[n] = Abar * h[n] + Bbar x
 *   y[b,d,t] = (sum_n C[b,n,t] h[n] + Dskip[d] x[b,d,t]) * silu(z[b,d,t])
 * and h_final[b, d, :] = h.  Returns 0, or -1 on invalid arguments.
 */
int ss_oracle_scan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                   const double* x, const double* dt, const double* z,
                   const double* B, const double* C, const double* A,
                   const double* Dskip, const double* dt_bias, const double* h0,
                   int zoh, double* y, double* h_final, int nthreads) {
  if (batch < 0 || dim < 0 || dstate < 1 || dstate > 64 || seqlen < 0) return -1;
  if (batch * dim * seqlen > 0 && (!x || !dt || !B || !C || !A || !y)) return -1;
  const int64_t nch = batch * dim;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int64_t b = ch / dim, d = ch % dim;
    double h[64];
    for (int64_t n = 0; n < dstate; ++n) h[n] = h0 ? h0[ch * dstate + n] : 0.0;
    const double skip = Dskip ? Dskip[d] : 0.0;
    const double bias = dt_bias ? dt_bias[d] : 0.0;
    const double* xr = x + ch * seqlen;
    const double* dtr = dt + ch * seqlen;
    const double* zr = z ? z + ch * seqlen : NULL;
    double* yr = y + ch * seqlen;
    for (int64_t t = 0; t < seqlen; ++t) {
      const double delta = softplus(dtr[t] + bias);
      double acc = 0.0;
      for (int64_t n = 0; n < dstate; ++n) {
        const double a = A[d * dstate + n];
        const double abar = exp(delta * a);
        const double bt = B[(b * dstate + n) * seqlen + t];
        const double ct = C[(b * dstate + n) * seqlen + t];
        h[n] = abar * h[n] + bbar_x(delta, a, abar, bt, xr[t], zoh);
        acc += ct * h[n];
      }
      double out = acc + skip * xr[t];
      if (zr) out *= silu(zr[t]);
      yr[t] = out;
    }
    if (h_final)
      for (int64_t n = 0; n < dstate; ++n) h_final[ch * dstate + n] = h[n];
  }
  return 0;
}

/*
 * One decode step: the same update for a single token per (b, d), with the
 * state read from and written back to `state` (batch, dim, dstate).
 * Written out on its own (not by calling the scan) so that "T decode steps equal
 * a scan over T tokens" is a real check.
 */
int ss_oracle_state_update(int64_t batch, int64_t dim, int64_t dstate, double* state,
                           const double* x, const double* dt, const double* z,
                           const double* B, const double* C, const double* A,
                           const double* Dskip, const double* dt_bias, int zoh,
                           double* y, int nthreads) {
  if (batch < 0 || dim < 0 || dstate < 1 || dstate > 64) return -1;
  if (batch * dim > 0 && (!state || !x || !dt || !B || !C || !A || !y)) return -1;
  const int64_t nch = batch * dim;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int64_t b = ch / dim, d = ch % dim;
    double* s = state + ch * dstate;
    const double v = dt[ch] + (dt_bias ? dt_bias[d] : 0.0);
    const double delta = (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));
    double acc = 0.0;
    for (int64_t n = 0; n < dstate; ++n) {
      const double a = A[d * dstate + n];
      const double abar = exp(delta * a);
      double in;
      if (zoh && a != 0.0) in = expm1(delta * a) / a * B[b * dstate + n] * x[ch];
      else in = delta * B[b * dstate + n] * x[ch];
      s[n] = abar * s[n] + in;
      acc += C[b * dstate + n] * s[n];
    }
    double out = acc + (Dskip ? Dskip[d] : 0.0) * x[ch];
    if (z) out *= z[ch] / (1.0 + exp(-z[ch]));
    y[ch] = out;
  }
  return 0;
}
