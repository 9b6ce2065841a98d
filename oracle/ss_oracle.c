/*
 * CPU oracle for the selective state-space (S6) scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing but the tests, the smoke check in
 * __graft_entry__.py and the benchmark's cpu_baseline leg may load or call this
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
#include <stdlib.h>
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

/* ------------------------------------------------------------------------- */
/* Backward pass (reverse-mode gradients of the scan).                        */
/*
 * Training runs the scan forward and backward; the pages' fused kernel
 * recomputes the expanded state in the backward pass rather than storing it
 * (reader's notes, kurisu.si, "What they did", Selective SSM item).  What is
 * differentiated here is exactly ss_oracle_scan above: the gradients follow from
 * the chain rule applied to its steps in reverse token order, with the whole
 * forward state of one channel kept in memory (the oracle has no reason to
 * recompute).
 *
 * Given dy (batch, dim, L) = dLoss/dy and dh_final (batch, dim, N) (NULL = 0):
 *   for each (b, d), with lam[n] = dLoss/dh_t[n] carried backwards from
 *   lam = dh_final, for t = L-1 .. 0:
 *     g = silu(z_t) (1 without a gate); r_t = C_t . h_t + Dskip x_t;  y_t = r_t g
 *     dr = dy_t g;   dz_t = dy_t r_t silu'(z_t)
 *     lam[n] += dr C[b,n,t];         dC[b,n,t] += dr h_t[n]     (summed over d)
 *     dDskip[d] += dr x_t;           dx_t = dr Dskip
 *     h_t[n] = Abar h_{t-1}[n] + c(Delta, A) B x_t, Abar = exp(Delta A):
 *       dAbar = lam[n] h_{t-1}[n]:  dDelta += dAbar Abar A;  dA[d,n] += dAbar Abar Delta
 *       input term (c = Delta for Euler, c = phi = (Abar - 1)/A for ZOH):
 *         dDelta += lam[n] B x dc/dDelta;   dA[d,n] += lam[n] B x dc/dA
 *         dB[b,n,t] += lam[n] c x_t (summed over d);  dx_t += lam[n] c B[b,n,t]
 *       lam[n] *= Abar  (dLoss/dh_{t-1} through the recurrence)
 *     Delta = softplus(v), v = dt_t + dt_bias[d]:  dv = dDelta sigmoid(v)
 *     ddt_t = dv;  ddt_bias[d] += dv
 *   dh0[b,d,n] = lam[n] after the loop.
 * Cross-channel sums (dB, dC over d) and cross-row sums (dA, dDskip, ddt_bias
 * over b and t) are accumulated in double.  Returns 0, -1 on invalid
 * arguments, -2 if memory runs out.
 */
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))) */
static double dsilu(double z) {
  const double s = sigmoid(z);
  return s * (1.0 + z * (1.0 - s));
}

/* The input coefficient c(Delta, A) and its partial derivatives.
 * Euler: c = Delta, dc/dDelta = 1, dc/dA = 0.
 * ZOH:   c = phi = (e^{Delta A} - 1)/A (Delta when A = 0), dphi/dDelta = e^{Delta A},
 *        dphi/dA = (Delta e^{Delta A} - phi)/A = Delta^2 psi(Delta A) with
 *        psi(u) = (u e^u - e^u + 1)/u^2 = sum_{m>=2} (m-1) u^(m-2) / m!
 *        = 1/2 + u/3 + u^2/8 + u^3/30 + ...; the series is used for |u| < 1e-3
 *        (first dropped term u^4/144 < 1e-14), the closed form otherwise. */
static void input_coef(double delta, double a, int zoh, double* c, double* dc_ddelta, double* dc_da) {
  if (!zoh) {
    *c = delta;
    *dc_ddelta = 1.0;
    *dc_da = 0.0;
    return;
  }
  const double u = delta * a;
  const double eu = exp(u);
  *c = (a == 0.0) ? delta : expm1(u) / a;
  *dc_ddelta = eu;
  double psi;
  if (fabs(u) < 1e-3) psi = 0.5 + u * (1.0 / 3.0 + u * (1.0 / 8.0 + u * (1.0 / 30.0)));
  else psi = (u * eu - expm1(u)) / (u * u);
  *dc_da = delta * delta * psi;
}

int ss_oracle_scan_bwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                       const double* x, const double* dt, const double* z,
                       const double* B, const double* C, const double* A,
                       const double* Dskip, const double* dt_bias, const double* h0, int zoh,
                       const double* dy, const double* dh_final,
                       double* dx, double* ddt, double* dz, double* dB, double* dC,
                       double* dA, double* dDskip, double* ddt_bias, double* dh0, int nthreads) {
  if (batch < 0 || dim < 0 || dstate < 1 || dstate > 64 || seqlen < 0) return -1;
  if (!dA || !dDskip || !ddt_bias || !dh0 || !A) return -1;
  if (batch * dim * seqlen > 0 && (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC)) return -1;
  if (z && !dz && batch * dim * seqlen > 0) return -1;
  const int64_t N = dstate, L = seqlen;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
  nthreads = 1;
#endif
  for (int64_t i = 0; i < dim * N; ++i) dA[i] = 0.0;
  for (int64_t i = 0; i < dim; ++i) dDskip[i] = ddt_bias[i] = 0.0;
  for (int64_t i = 0; i < batch * N * L; ++i) dB[i] = dC[i] = 0.0;
  /* per thread: dB/dC partial sums for one batch row, and one channel's forward */
  const int64_t per = 2 * N * L + (L + 1) * N + 2 * L;
  double* work = (double*)calloc((size_t)(nthreads * per > 0 ? nthreads * per : 1), sizeof(double));
  if (!work) return -2;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t i = 0; i < nthreads * per; ++i) work[i] = 0.0;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t d = 0; d < dim; ++d) {
#ifdef _OPENMP
      double* wk = work + omp_get_thread_num() * per;
#else
      double* wk = work;
#endif
      double* pdB = wk;              /* (N, L) */
      double* pdC = wk + N * L;      /* (N, L) */
      double* hs = wk + 2 * N * L;   /* (L + 1, N): hs[(t + 1) N + n] = h_t[n], hs[n] = h0 */
      double* dl = hs + (L + 1) * N; /* (L) Delta_t */
      double* rr = dl + L;           /* (L) r_t, the readout before the gate */
      const int64_t ch = b * dim + d;
      const double skip = Dskip ? Dskip[d] : 0.0;
      const double bias = dt_bias ? dt_bias[d] : 0.0;
      const double* xr = x + ch * L;
      const double* dtr = dt + ch * L;
      const double* zr = z ? z + ch * L : NULL;
      /* forward, keeping every state */
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[ch * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const double delta = softplus(dtr[t] + bias);
        dl[t] = delta;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double a = A[d * N + n];
          double c, dcd, dca;
          input_coef(delta, a, zoh, &c, &dcd, &dca);
          const double h = exp(delta * a) * hs[t * N + n] + c * B[(b * N + n) * L + t] * xr[t];
          hs[(t + 1) * N + n] = h;
          acc += C[(b * N + n) * L + t] * h;
        }
        rr[t] = acc + skip * xr[t];
      }
      /* backward */
      double lam[64];
      for (int64_t n = 0; n < N; ++n) lam[n] = dh_final ? dh_final[ch * N + n] : 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const double g = zr ? silu(zr[t]) : 1.0;
        const double dr = dy[ch * L + t] * g;
        if (zr) dz[ch * L + t] = dy[ch * L + t] * rr[t] * dsilu(zr[t]);
        dDskip[d] += dr * xr[t];
        double dxv = dr * skip;
        double ddelta = 0.0;
        const double delta = dl[t];
        for (int64_t n = 0; n < N; ++n) {
          lam[n] += dr * C[(b * N + n) * L + t];
          pdC[n * L + t] += dr * hs[(t + 1) * N + n];
        }
        for (int64_t n = 0; n < N; ++n) {
          const double a = A[d * N + n];
          const double abar = exp(delta * a);
          const double bt = B[(b * N + n) * L + t];
          double c, dcd, dca;
          input_coef(delta, a, zoh, &c, &dcd, &dca);
          const double dabar = lam[n] * hs[t * N + n];
          ddelta += dabar * abar * a + lam[n] * bt * xr[t] * dcd;
          dA[d * N + n] += dabar * abar * delta + lam[n] * bt * xr[t] * dca;
          pdB[n * L + t] += lam[n] * c * xr[t];
          dxv += lam[n] * c * bt;
          lam[n] *= abar;
        }
        const double dv = ddelta * sigmoid(dtr[t] + bias);
        ddt[ch * L + t] = dv;
        ddt_bias[d] += dv;
        dx[ch * L + t] = dxv;
      }
      for (int64_t n = 0; n < N; ++n) dh0[ch * N + n] = lam[n];
    }
    /* the threads' partial sums, in thread order */
    for (int k = 0; k < nthreads; ++k) {
      const double* wk = work + k * per;
      for (int64_t i = 0; i < N * L; ++i) {
        dB[b * N * L + i] += wk[i];
        dC[b * N * L + i] += wk[N * L + i];
      }
    }
  }
  free(work);
  return 0;
}
