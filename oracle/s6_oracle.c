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

/* One token of one (batch, channel) pair, all N states.
 * h, H   : the N states and their magnitudes, updated in place.
 * Ad     : A[d, 0..N-1].
 * Bt, Ct : B and C of this token; state n is at Bt[n * bstride].
 * Returns the token's output before the gate; *mag gets its magnitude. */
static double step_channel(int64_t N, double* h, double* H, const double* Ad, double dt, double xt,
                           const double* Bt, const double* Ct, int64_t bstride, double dskip,
                           double* mag) {
  double acc = 0.0, macc = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    double a = exp(dt * Ad[n]);         /* zero-order-hold state transition */
    double bx = dt * Bt[n * bstride] * xt; /* input term */
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
 * N must not exceed 256. */
void oracle_scan(int64_t Bsz, int64_t D, int64_t L, int64_t N, const double* x, const double* delta,
                 const double* A, const double* Bm, const double* Cm, const double* Dskip,
                 const double* z, const double* h0, double* y, double* m, double* h_last,
                 double* H_last) {
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
      double yt = step_channel(N, h, H, A + d * N, delta[p * L + t], x[p * L + t], Bb + t, Cb + t,
                               L, dsk, &mag);
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

/* One decode token for every (batch, channel) pair: h and its magnitude H are
 * updated in place, y and m receive the token's output.  Same arithmetic as
 * one iteration of the time loop above. */
void oracle_step(int64_t Bsz, int64_t D, int64_t N, double* h, double* H, const double* x,
                 const double* delta, const double* A, const double* Bm, const double* Cm,
                 const double* Dskip, const double* z, double* y, double* m) {
  int64_t pairs = Bsz * D;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; ++p) {
    int64_t b = p / D, d = p % D;
    double dsk = Dskip ? Dskip[d] : 0.0;
    double mag;
    double yt = step_channel(N, h + p * N, H + p * N, A + d * N, delta[p], x[p], Bm + b * N,
                             Cm + b * N, 1, dsk, &mag);
    if (z) {
      double g = silu(z[p]);
      yt *= g;
      mag *= fabs(g);
    }
    y[p] = yt;
    if (m) m[p] = mag;
  }
}
