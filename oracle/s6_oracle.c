/*
 * s6_oracle.c -- plain, slow fp64 CPU oracle for the selective SSM scan (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this file's library.  It shares no code, header,
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes.  Sources: the page "【LLM】Mamba和State Space Models详解"
 * (a Chinese translation of a visual guide to Mamba), sections as cited:
 *
 *   continuous SSM: h'(t) = A h(t) + B x(t), y(t) = C h(t) + D x(t)      (§2.2)
 *   discretisation by zero-order hold with a learnable step Delta; the
 *     continuous A is what is stored, it is discretised on the fly         (§2.3)
 *     The formula image is missing from the page.  Reading taken here:
 *     dA = exp(Delta*A[d,n]) and dBx = Delta*B[n]*x.
 *   recurrent form: the token's input term is added to A times the previous
 *     state, and the output is read from the UPDATED state                 (§2.4)
 *   selection: Delta, B and C get a batch and a length axis (one value per
 *     token); A stays input-independent                                    (§3.2)
 *   the scan: every state is the previous state times A plus the current
 *     input times B, evaluated here as a plain loop over time              (§3.3)
 *   D is a skip connection from x to y                                     (§2.2)
 *   optional gate y <- y * SiLU(z), SiLU(z) = z / (1 + exp(-z)), applied
 *     after the skip term.  The pages do not show the gate; this is the plain
 *     reading of the gated Mamba output.
 *
 * Layouts (row-major, last index fastest):
 *   x, delta, z, y, m : (Bsz, D, L)      Bm, Cm : (Bsz, N, L)
 *   A : (D, N)        Dskip : (D)        h0, h_last, H_last : (Bsz, D, N)
 *   decode step: x, delta, z, y, m : (Bsz, D); Bm, Cm : (Bsz, N)
 *
 Step bias and discretisation options (oracle_scan_ex, oracle_step_ex):
 *   delta_bias (D), nullable: the step is delta + delta_bias[d].
 *   ORACLE_DELTA_SOFTPLUS (bit flag): the step is softplus(delta + bias),
 *     softplus(v) = ln(1 + e^v).  The pages make Delta learnable and
 *     input-dependent (§3.2) but do not say how it is kept positive; a
 *     per-channel bias and softplus are the plain reading of the Mamba layer
 *     this guide describes.
 *   ORACLE_ZOH_EXACT  the input coefficient is the zero-order-hold integral
 *     of exp(s A) over s in [0, Delta], i.e. (exp(Delta A) - 1) / A (its
 *     limit at A = 0 is Delta), in place of Delta: the hold the pages name
 *     in §2.3, applied to B as well as to A.
 *
 * Besides y the oracle returns the magnitude m: the same recurrence run on
 * absolute values (|dA| H + |dBx|, then sum_n |C| H + |D x|, times |gate|).
 * m bounds |y| and is the scale of the componentwise error metric of the
 * parity tests.
 *
 * Every (batch, channel) pair is independent; the OpenMP loop over pairs does
 * not change any result (there is no reduction across pairs).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

enum { ORACLE_DELTA_SOFTPLUS = 1, ORACLE_ZOH_EXACT = 2 };

/* softplus(v) = ln(1 + e^v), written as max(v, 0) + ln(1 + e^-|v|) so that
 * no exponential overflows (the two forms are equal for every v). */
static double softplus(double v) { return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v))); }

/* The step Delta of channel d for a stored delta value. */
static double step_of(double raw, const double* dbias, int64_t d, int flags) {
  double v = dbias ? raw + dbias[d] : raw;
  return (flags & ORACLE_DELTA_SOFTPLUS) ? softplus(v) : v;
}

/* Zero-order-hold input coefficient: integral of exp(s a) ds over [0, dt],
 * (exp(dt a) - 1) / a, which is dt when a = 0. */
static double zoh_coef(double dt, double a) { return a != 0.0 ? expm1(dt * a) / a : dt; }

/* One token of one (batch, channel) pair, all N states.
 * h, H   : the N states and their magnitudes, updated in place.
 * Ad     : A[d, 0..N-1].
 * Bt, Ct : B and C of this token; state n is at Bt[n * bstride].
 * Returns the token's output before the gate; *mag gets its magnitude. */
static double step_channel(int64_t N, double* h, double* H, const double* Ad, double dt, double xt,
                           const double* Bt, const double* Ct, int64_t bstride, double dskip,
                           int zoh, double* mag) {
  double acc = 0.0, macc = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    double a = exp(dt * Ad[n]);         /* zero-order-hold state transition */
    double bx = (zoh ? zoh_coef(dt, Ad[n]) : dt) * Bt[n * bstride] * xt; /* input term */
    h[n] = a * h[n] + bx;               /* update first ... */
    H[n] = fabs(a) * H[n] + fabs(bx);
    acc += Ct[n * bstride] * h[n];      /* ... then read the output from the new state */
    macc += fabs(Ct[n * bstride]) * H[n];
  }
  double skip = dskip * xt;
  *mag = macc + fabs(skip);
  return acc + skip;
}

/* Whole sequence.  Dskip, z and h0 may be NULL (no skip, no gate, zero
 * initial state).  m, h_last and H_last may be NULL (not written).
 * dbias (D) may be NULL (no bias); flags: ORACLE_* above.
 * N must not exceed 256. */
void oracle_scan_ex(int64_t Bsz, int64_t D, int64_t L, int64_t N, const double* x,
                    const double* delta, const double* dbias, int flags, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip, const double* z,
                    const double* h0, double* y, double* m, double* h_last, double* H_last) {
  const int zoh = (flags & ORACLE_ZOH_EXACT) != 0;
  int64_t pairs = Bsz * D;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < pairs; ++p) {
    int64_t b = p / D, d = p % D;
    double h[256], H[256];
    for (int64_t n = 0; n < N; ++n) {
      h[n] = h0 ? h0[p * N + n] : 0.0;
      H[n] = fabs(h[n]);
    }
    const double* Bb = Bm + b * N * L;
    const double* Cb = Cm + b * N * L;
    double dsk = Dskip ? Dskip[d] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      double mag;
      double dt = step_of(delta[p * L + t], dbias, d, flags);
      double yt = step_channel(N, h, H, A + d * N, dt, x[p * L + t], Bb + t, Cb + t,
                               L, dsk, zoh, &mag);
      if (z) {
        double g = silu(z[p * L + t]);
        yt *= g;
        mag *= fabs(g);
      }
      y[p * L + t] = yt;
      if (m) m[p * L + t] = mag;
    }
    for (int64_t n = 0; n < N; ++n) {
      if (h_last) h_last[p * N + n] = h[n];
      if (H_last) H_last[p * N + n] = H[n];
    }
  }
}

void oracle_scan(int64_t Bsz, int64_t D, int64_t L, int64_t N, const double* x, const double* delta,
                 const double* A, const double* Bm, const double* Cm, const double* Dskip,
                 const double* z, const double* h0, double* y, double* m, double* h_last,
                 double* H_last) {
  oracle_scan_ex(Bsz, D, L, N, x, delta, NULL, 0, A, Bm, Cm, Dskip, z, h0, y, m, h_last, H_last);
}

/* One decode token for every (batch, channel) pair: h and its magnitude H are
 * updated in place, y and m receive the token's output.  Same arithmetic as
 * one iteration of the time loop above. */
void oracle_step_ex(int64_t Bsz, int64_t D, int64_t N, double* h, double* H, const double* x,
                    const double* delta, const double* dbias, int flags, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip, const double* z,
                    double* y, double* m) {
  const int zoh = (flags & ORACLE_ZOH_EXACT) != 0;
  int64_t pairs = Bsz * D;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; ++p) {
    int64_t b = p / D, d = p % D;
    double dsk = Dskip ? Dskip[d] : 0.0;
    double mag;
    double dt = step_of(delta[p], dbias, d, flags);
    double yt = step_channel(N, h + p * N, H + p * N, A + d * N, dt, x[p], Bm + b * N,
                             Cm + b * N, 1, dsk, zoh, &mag);
    if (z) {
      double g = silu(z[p]);
      yt *= g;
      mag *= fabs(g);
    }
    y[p] = yt;
    if (m) m[p] = mag;
  }
}

void oracle_step(int64_t Bsz, int64_t D, int64_t N, double* h, double* H, const double* x,
                 const double* delta, const double* A, const double* Bm, const double* Cm,
                 const double* Dskip, const double* z, double* y, double* m) {
  oracle_step_ex(Bsz, D, N, h, H, x, delta, NULL, 0, A, Bm, Cm, Dskip, z, y, m);
}
