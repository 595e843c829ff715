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
 * Step bias and discretisation options (oracle_scan_ex, oracle_step_ex):
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
#include <stdlib.h>
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
 * xm     : the magnitude taken for the input x_t in H and *mag: |x_t| for a
 *          plain input, the convolution front's magnitude for its output.
 * Returns the token's output before the gate; *mag gets its magnitude. */
static double step_channel(int64_t N, double* h, double* H, const double* Ad, double dt, double xt,
                           const double* Bt, const double* Ct, int64_t bstride, double dskip,
                           int zoh, double xm, double* mag) {
  double acc = 0.0, macc = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    double a = exp(dt * Ad[n]);         /* zero-order-hold state transition */
    double cb = (zoh ? zoh_coef(dt, Ad[n]) : dt) * Bt[n * bstride];
    double bx = cb * xt;                /* input term */
    h[n] = a * h[n] + bx;               /* update first ... */
    H[n] = fabs(a) * H[n] + fabs(cb) * xm;
    acc += Ct[n * bstride] * h[n];      /* ... then read the output from the new state */
    macc += fabs(Ct[n * bstride]) * H[n];
  }
  double skip = dskip * xt;
  *mag = macc + fabs(dskip) * xm;
  return acc + skip;
}

/* Whole sequence.  Dskip, z and h0 may be NULL (no skip, no gate, zero
 * initial state).  m, h_last and H_last may be NULL (not written).
 * dbias (D) may be NULL (no bias); flags: ORACLE_* above.
 * xmag (Bsz, D, L) may be NULL: the magnitudes taken for x (|x| when NULL;
 * oracle_conv_silu's xm when x is the convolution front's output).
 * N must not exceed 256. */
void oracle_scan_xm(int64_t Bsz, int64_t D, int64_t L, int64_t N, const double* x,
                    const double* xmag, const double* delta, const double* dbias, int flags,
                    const double* A, const double* Bm, const double* Cm, const double* Dskip,
                    const double* z, const double* h0, double* y, double* m, double* h_last,
                    double* H_last) {
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
      double xm = xmag ? xmag[p * L + t] : fabs(x[p * L + t]);
      double yt = step_channel(N, h, H, A + d * N, dt, x[p * L + t], Bb + t, Cb + t,
                               L, dsk, zoh, xm, &mag);
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

void oracle_scan_ex(int64_t Bsz, int64_t D, int64_t L, int64_t N, const double* x,
                    const double* delta, const double* dbias, int flags, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip, const double* z,
                    const double* h0, double* y, double* m, double* h_last, double* H_last) {
  oracle_scan_xm(Bsz, D, L, N, x, NULL, delta, dbias, flags, A, Bm, Cm, Dskip, z, h0, y, m,
                 h_last, H_last);
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
void oracle_step_xm(int64_t Bsz, int64_t D, int64_t N, double* h, double* H, const double* x,
                    const double* xmag, const double* delta, const double* dbias, int flags,
                    const double* A, const double* Bm, const double* Cm, const double* Dskip,
                    const double* z, double* y, double* m) {
  const int zoh = (flags & ORACLE_ZOH_EXACT) != 0;
  int64_t pairs = Bsz * D;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; ++p) {
    int64_t b = p / D, d = p % D;
    double dsk = Dskip ? Dskip[d] : 0.0;
    double mag;
    double dt = step_of(delta[p], dbias, d, flags);
    double xm = xmag ? xmag[p] : fabs(x[p]);
    double yt = step_channel(N, h + p * N, H + p * N, A + d * N, dt, x[p], Bm + b * N,
                             Cm + b * N, 1, dsk, zoh, xm, &mag);
    if (z) {
      double g = silu(z[p]);
      yt *= g;
      mag *= fabs(g);
    }
    y[p] = yt;
    if (m) m[p] = mag;
  }
}

void oracle_step_ex(int64_t Bsz, int64_t D, int64_t N, double* h, double* H, const double* x,
                    const double* delta, const double* dbias, int flags, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip, const double* z,
                    double* y, double* m) {
  oracle_step_xm(Bsz, D, N, h, H, x, NULL, delta, dbias, flags, A, Bm, Cm, Dskip, z, y, m);
}

void oracle_step(int64_t Bsz, int64_t D, int64_t N, double* h, double* H, const double* x,
                 const double* delta, const double* A, const double* Bm, const double* Cm,
                 const double* Dskip, const double* z, double* y, double* m) {
  oracle_step_ex(Bsz, D, N, h, H, x, delta, NULL, 0, A, Bm, Cm, Dskip, z, y, m);
}

/* ------------------------------------------------------ convolution front --
 * The guide's Mamba block (§3.5 "Mamba Block") applies a convolution to the
 * expanded input before the selective SSM, so that tokens are not handled
 * independently.  The pages give neither its width nor its activation.
 * Reading: per channel d a causal filter of width K with weights w[d, k]
 * and a bias, followed by SiLU, the input the scan then takes as x:
 *   xc_t = bias[d] + sum_{k=0}^{K-1} w[d, k] x_{t-K+1+k},   x'_t = SiLU(xc_t),
 * where x_s for s < 0 is state[b, d, K-1+s] (the K-1 inputs before the
 * sequence, oldest first) or 0 when state is NULL.  bias may be NULL (0).
 * Layouts: x, xo, xm (Bsz, D, L); w (D, K); bias (D); state (Bsz, D, K-1).
 * xm receives the magnitude the error metric takes for x'_t:
 *   |x'_t| + |SiLU'(xc_t)| (|bias[d]| + sum_k |w[d, k] x_{t-K+1+k}|),
 * |x'| plus the first-order effect of a rounding of each term of the
 * convolution's sum, SiLU'(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z).
 * Returns -1 when K < 1, else 0. */
/* Input of the filter at token s of pair p: x itself, or before token 0 the
 * state (oldest first), or 0 without one. */
static double conv_input(int64_t p, int64_t s, int64_t L, int64_t K, const double* x,
                         const double* state) {
  return s >= 0 ? x[p * L + s] : (state ? state[p * (K - 1) + (K - 1) + s] : 0.0);
}

/* The filter's output xc_t of pair p (channel d) before SiLU; *mag receives
 * |bias| + sum_k |w x|. */
static double conv_pre(int64_t p, int64_t d, int64_t t, int64_t L, int64_t K, const double* x,
                       const double* w, const double* bias, const double* state, double* mag) {
  double b0 = bias ? bias[d] : 0.0;
  double acc = b0, m = fabs(b0);
  for (int64_t k = 0; k < K; ++k) {
    int64_t s = t - (K - 1) + k;  /* token of tap k */
    double xs = conv_input(p, s, L, K, x, state);
    acc += w[d * K + k] * xs;
    m += fabs(w[d * K + k] * xs);
  }
  *mag = m;
  return acc;
}

int oracle_conv_silu(int64_t Bsz, int64_t D, int64_t L, int64_t K, const double* x,
                     const double* w, const double* bias, const double* state, double* xo,
                     double* xm) {
  if (K < 1) return -1;
  int64_t pairs = Bsz * D;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; ++p) {
    int64_t d = p % D;
    for (int64_t t = 0; t < L; ++t) {
      double mag;
      double acc = conv_pre(p, d, t, L, K, x, w, bias, state, &mag);
      double sg = 1.0 / (1.0 + exp(-acc));
      xo[p * L + t] = acc * sg;
      if (xm) xm[p * L + t] = fabs(acc * sg) + fabs(sg * (1.0 + acc * (1.0 - sg))) * mag;
    }
  }
  return 0;
}

/* Gradients through the convolution front, given the gradient dxo of the
 * loss with respect to its output x' (the scan backward's dx when the scan
 * ran on x') and that gradient's magnitude mdxo.  With xc_t the filter's
 * output before SiLU and dxc_t = dxo_t SiLU'(xc_t):
 *   dx_s      = sum_k w[d,k] dxc_{s+K-1-k}          (tokens s = 0 .. L-1)
 *   dstate_s  = the same sum for s = -(K-1) .. -1   (at [b, d, K-1+s])
 *   dw[d,k]   = sum_{b,t} dxc_t x_{t-K+1+k}         dbias[d] = sum_{b,t} dxc_t
 * where x_s for s < 0 comes from state (or is 0), and terms with
 * s+K-1-k >= L are absent.  SiLU'(z) = s (1 + z (1 - s)); SiLU''(z) =
 * s (1 - s) (2 + z (1 - 2 s)).  Magnitudes: mdxc_t = mdxo_t |SiLU'(xc_t)| +
 * |dxo_t| |SiLU''(xc_t)| (|bias| + sum_k |w x|) (the second term: a
 * rounding of the filter's sum moves SiLU'), then the same sums over
 * absolute values.  dstate, dbias and every magnitude output are nullable;
 * dw and dbias are summed over rows in order b = 0 .. Bsz-1.  Returns -1
 * when K < 1, -3 when out of memory. */
int oracle_conv_silu_bwd(int64_t Bsz, int64_t D, int64_t L, int64_t K, const double* x,
                         const double* w, const double* bias, const double* state,
                         const double* dxo, const double* mdxo, double* dx, double* dw,
                         double* dbias, double* dstate, double* mdx, double* mdw, double* mdbias,
                         double* mdstate) {
  if (K < 1) return -1;
  const int64_t pairs = Bsz * D;
  double* dxc = (double*)malloc((size_t)(pairs * L) * sizeof(double));
  double* mdxc = (double*)malloc((size_t)(pairs * L) * sizeof(double));
  if (!dxc || !mdxc) {
    free(dxc);
    free(mdxc);
    return -3;
  }
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; ++p) {
    const int64_t d = p % D;
    for (int64_t t = 0; t < L; ++t) {
      double mag;
      const double acc = conv_pre(p, d, t, L, K, x, w, bias, state, &mag);
      const double sg = 1.0 / (1.0 + exp(-acc));
      const double d1 = sg * (1.0 + acc * (1.0 - sg));
      const double d2 = sg * (1.0 - sg) * (2.0 + acc * (1.0 - 2.0 * sg));
      dxc[p * L + t] = dxo[p * L + t] * d1;
      mdxc[p * L + t] = (mdxo ? mdxo[p * L + t] : fabs(dxo[p * L + t])) * fabs(d1) +
                        fabs(dxo[p * L + t]) * fabs(d2) * mag;
    }
    /* token s (s >= -(K-1)) feeds outputs t = s + K - 1 - k through tap k */
    for (int64_t s = -(K - 1); s < L; ++s) {
      double g = 0.0, mg = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t t = s + K - 1 - k;
        if (t < 0 || t >= L) continue;
        g += w[d * K + k] * dxc[p * L + t];
        mg += fabs(w[d * K + k]) * mdxc[p * L + t];
      }
      if (s >= 0) {
        dx[p * L + s] = g;
        if (mdx) mdx[p * L + s] = mg;
      } else {
        if (dstate) dstate[p * (K - 1) + (K - 1) + s] = g;
        if (mdstate) mdstate[p * (K - 1) + (K - 1) + s] = mg;
      }
    }
  }
  for (int64_t d = 0; d < D; ++d) {
    for (int64_t k = 0; k <= K; ++k) { /* k == K: the bias */
      double g = 0.0, mg = 0.0;
      for (int64_t b = 0; b < Bsz; ++b) {
        const int64_t p = b * D + d;
        for (int64_t t = 0; t < L; ++t) {
          double xs = 1.0;
          if (k < K) xs = conv_input(p, t + k - (K - 1), L, K, x, state);
          g += dxc[p * L + t] * xs;
          mg += mdxc[p * L + t] * fabs(xs);
        }
      }
      if (k < K) {
        dw[d * K + k] = g;
        if (mdw) mdw[d * K + k] = mg;
      } else {
        if (dbias) dbias[d] = g;
        if (mdbias) mdbias[d] = mg;
      }
    }
  }
  free(dxc);
  free(mdxc);
  return 0;
}

/* ---------------------------------------------------------------- backward --
 * Gradients of the scan for the loss  <dy, y> + <dh_last, h_last>  (reverse
 * mode; plain step, no options).  The state is recomputed from the inputs
 * (the pages' guide, §3.4, notes that the fused scan recomputes the states in
 * the backward pass instead of storing them).  With a_t[n] = exp(Delta_t
 * A[n]), g_t = SiLU(z_t) (1 without a gate), yc_t = sum_n C_t[n] h_t[n] +
 * D x_t (the output before the gate) and dyc_t = dy_t g_t:
 *
 *   lambda_t[n] = dL/dh_t[n] = dyc_t C_t[n] + a_{t+1}[n] lambda_{t+1}[n],
 *                 lambda_{L-1}[n] = dyc_{L-1} C_{L-1}[n] + dh_last[n]
 *   dx_t     = dyc_t D + sum_n lambda_t[n] Delta_t B_t[n]
 *   ddelta_t = sum_n lambda_t[n] (A[n] a_t[n] h_{t-1}[n] + B_t[n] x_t)
 *   dA[d,n]  = sum_{b,t} lambda_t[n] Delta_t a_t[n] h_{t-1}[n]
 *   dB[b,n,t] = sum_d lambda_t[n] Delta_t x_t      dC[b,n,t] = sum_d dyc_t h_t[n]
 *   dD[d]    = sum_{b,t} dyc_t x_t                 dh0[n] = a_0[n] lambda_0[n]
 *   dz_t     = dy_t yc_t SiLU'(z_t),  SiLU'(z) = s (1 + z (1 - s)), s = 1/(1+e^-z)
 * with h_{-1} = h0 (or 0).  Each output also gets its magnitude: the same
 * sums over the absolute values of every factor (states and adjoints
 * replaced by their magnitude recurrences), the scale of the componentwise
 * error metric.
 *
 * Order of evaluation: batch rows in parallel; within a row the channels in
 * order d = 0 .. D-1, so dB and dC are summed over d in a fixed order; dA and
 * dD are summed over rows b = 0 .. Bsz-1 after the parallel loop.
 * Nullable: Dskip, z, h0, dh_last (inputs); dDskip, dz, dh0 (outputs); every
 * magnitude output.  Work memory: 4 L N doubles per batch row.
 *
 * oracle_scan_bwd_ex also takes the options of oracle_scan_ex.  The step is
 * Delta = v or softplus(v), v = delta + bias[d], so ddelta above becomes the
 * gradient of the stored delta, ddelta * dDelta/dv with dsoftplus/dv =
 * 1/(1 + e^-v), and dbias[d] = sum over b, t of that (ddbias, nullable).
 * With ORACLE_ZOH_EXACT the input term is c(Delta, A[n]) B x with the hold's
 * coefficient c = (e^{Delta A} - 1) / A in place of Delta, so in the sums
 * above Delta B (dx) and Delta x (dB) take c, the input part of ddelta takes
 * dc/dDelta = e^{Delta A} = a, and dA gains lambda B x dc/dA. */
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* dc/dA of the hold's coefficient c(dt, a) = (e^{dt a} - 1) / a:
 * (dt a e^{dt a} - (e^{dt a} - 1)) / a^2 = dt^2 q(dt a) with
 * q(u) = (u e^u - (e^u - 1)) / u^2 = sum_{k>=0} (k+1) u^k / (k+2)!, q(0) = 1/2.
 * The difference cancels for small |u|, so there the series (7 terms: the
 * next one is below 1e-18 for |u| < 1e-2) is summed instead. */
static double zoh_dcoef_da(double dt, double a) {
  const double u = dt * a;
  double q;
  if (fabs(u) < 1e-2)
    q = 1.0 / 2 + u * (1.0 / 3 + u * (1.0 / 8 + u * (1.0 / 30 + u * (1.0 / 144 + u * (1.0 / 840 + u / 5760)))));
  else
    q = (u * exp(u) - expm1(u)) / (u * u);
  return dt * dt * q;
}

int oracle_scan_bwd_xm(int64_t Bsz, int64_t D, int64_t L, int64_t N, const double* x,
                       const double* xmag, const double* delta, const double* dbias, int flags,
                       const double* A,
                       const double* Bm, const double* Cm, const double* Dskip, const double* z,
                       const double* h0, const double* dy, const double* dh_last, double* dx,
                       double* ddelta, double* dA, double* dBm, double* dCm, double* dDskip,
                       double* dz, double* dh0, double* ddbias, double* mdx, double* mddelta,
                       double* mdA, double* mdB, double* mdC, double* mdD, double* mdz, double* mdh0,
                       double* mddbias) {
  if (flags & ~(ORACLE_DELTA_SOFTPLUS | ORACLE_ZOH_EXACT)) return -2;
  const int sp = (flags & ORACLE_DELTA_SOFTPLUS) != 0;
  const int zoh = (flags & ORACLE_ZOH_EXACT) != 0;
  double* dA_b = (double*)calloc((size_t)(Bsz * D * N), sizeof(double));
  double* mdA_b = (double*)calloc((size_t)(Bsz * D * N), sizeof(double));
  double* dD_b = (double*)calloc((size_t)(Bsz * D), sizeof(double));
  double* mdD_b = (double*)calloc((size_t)(Bsz * D), sizeof(double));
  double* db_b = (double*)calloc((size_t)(Bsz * D), sizeof(double));
  double* mdb_b = (double*)calloc((size_t)(Bsz * D), sizeof(double));
  int fail = !dA_b || !mdA_b || !dD_b || !mdD_b || !db_b || !mdb_b;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < Bsz; ++b) {
    if (fail) continue;
    /* states h_t and magnitudes H_t, t = -1 .. L-1 (row t+1) */
    double* hs = (double*)malloc((size_t)((L + 1) * N) * sizeof(double));
    double* Hs = (double*)malloc((size_t)((L + 1) * N) * sizeof(double));
    double lam[256], Lam[256];
    if (!hs || !Hs) {
      free(hs);
      free(Hs);
#pragma omp atomic write
      fail = 1;
      continue;
    }
    const double* Bb = Bm + b * N * L;
    const double* Cb = Cm + b * N * L;
    for (int64_t i = 0; i < N * L; ++i) {
      dBm[b * N * L + i] = 0.0;
      dCm[b * N * L + i] = 0.0;
      if (mdB) mdB[b * N * L + i] = 0.0;
      if (mdC) mdC[b * N * L + i] = 0.0;
    }
    for (int64_t d = 0; d < D; ++d) {
      const int64_t p = b * D + d;
      const double* Ad = A + d * N;
      const double dsk = Dskip ? Dskip[d] : 0.0;
      /* forward: the states of every token */
      for (int64_t n = 0; n < N; ++n) {
        hs[n] = h0 ? h0[p * N + n] : 0.0;
        Hs[n] = fabs(hs[n]);
      }
      for (int64_t t = 0; t < L; ++t) {
        const double dt = step_of(delta[p * L + t], dbias, d, flags), xt = x[p * L + t];
        const double xm = xmag ? xmag[p * L + t] : fabs(xt);
        for (int64_t n = 0; n < N; ++n) {
          const double a = exp(dt * Ad[n]);
          const double cb = (zoh ? zoh_coef(dt, Ad[n]) : dt) * Bb[n * L + t];
          hs[(t + 1) * N + n] = a * hs[t * N + n] + cb * xt;
          Hs[(t + 1) * N + n] = a * Hs[t * N + n] + fabs(cb) * xm;
        }
      }
      /* reverse: adjoints from the last token back */
      for (int64_t n = 0; n < N; ++n) {
        lam[n] = dh_last ? dh_last[p * N + n] : 0.0; /* a_{t+1} lambda_{t+1} carried in */
        Lam[n] = fabs(lam[n]);
      }
      for (int64_t t = L - 1; t >= 0; --t) {
        const double dt = step_of(delta[p * L + t], dbias, d, flags), xt = x[p * L + t];
        const double xm = xmag ? xmag[p * L + t] : fabs(xt);
        const double g = z ? silu(z[p * L + t]) : 1.0;
        const double dyc = dy[p * L + t] * g;
        double gx = 0.0, mgx = 0.0, gd = 0.0, mgd = 0.0, yc = 0.0, myc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double a = exp(dt * Ad[n]);
          const double Bt = Bb[n * L + t], Ct = Cb[n * L + t];
          const double l = dyc * Ct + lam[n]; /* lambda_t */
          const double ml = fabs(dyc * Ct) + Lam[n];
          const double hp = hs[t * N + n], Hp = Hs[t * N + n]; /* h_{t-1} */
          const double ht = hs[(t + 1) * N + n], Ht = Hs[(t + 1) * N + n];
          /* the input coefficient and its derivatives in the step and in A */
          const double cf = zoh ? zoh_coef(dt, Ad[n]) : dt;
          const double cfd = zoh ? a : 1.0;
          const double cfa = zoh ? zoh_dcoef_da(dt, Ad[n]) : 0.0;
          gx += l * cf * Bt;
          mgx += ml * fabs(cf * Bt);
          gd += l * (Ad[n] * a * hp + cfd * Bt * xt);
          mgd += ml * (fabs(Ad[n] * a) * Hp + fabs(cfd * Bt) * xm);
          dA_b[p * N + n] += l * dt * a * hp + l * cfa * Bt * xt;
          mdA_b[p * N + n] += ml * fabs(dt * a) * Hp + ml * fabs(cfa * Bt) * xm;
          dBm[b * N * L + n * L + t] += l * cf * xt;
          dCm[b * N * L + n * L + t] += dyc * ht;
          if (mdB) mdB[b * N * L + n * L + t] += ml * fabs(cf) * xm;
          if (mdC) mdC[b * N * L + n * L + t] += fabs(dyc) * Ht;
          yc += Ct * ht;
          myc += fabs(Ct) * Ht;
          lam[n] = a * l; /* carried to token t - 1 */
          Lam[n] = a * ml;
        }
        yc += dsk * xt;
        myc += fabs(dsk) * xm;
        /* chain rule through the step: dDelta/d(stored delta) */
        const double v = dbias ? delta[p * L + t] + dbias[d] : delta[p * L + t];
        const double js = sp ? sigmoid(v) : 1.0;
        dx[p * L + t] = dyc * dsk + gx;
        ddelta[p * L + t] = gd * js;
        if (mdx) mdx[p * L + t] = fabs(dyc * dsk) + mgx;
        if (mddelta) mddelta[p * L + t] = mgd * js;
        db_b[p] += gd * js;
        mdb_b[p] += mgd * js;
        dD_b[p] += dyc * xt;
        mdD_b[p] += fabs(dyc) * xm;
        if (dz) {
          double zz = z ? z[p * L + t] : 0.0;
          double s = sigmoid(zz);
          double dsilu = s * (1.0 + zz * (1.0 - s));
          dz[p * L + t] = z ? dy[p * L + t] * yc * dsilu : 0.0;
          /* magnitude of SiLU'(z) = s + z s (1 - s): the sum of its two terms' absolute values */
          double mdsilu = s + fabs(zz) * s * (1.0 - s);
          if (mdz) mdz[p * L + t] = z ? fabs(dy[p * L + t]) * mdsilu * myc : 0.0;
        }
      }
      for (int64_t n = 0; n < N; ++n) {
        if (dh0) dh0[p * N + n] = lam[n];
        if (mdh0) mdh0[p * N + n] = Lam[n];
      }
    }
    free(hs);
    free(Hs);
  }
  if (!fail) {
    for (int64_t i = 0; i < D * N; ++i) {
      double s = 0.0, ms = 0.0;
      for (int64_t b = 0; b < Bsz; ++b) {
        s += dA_b[b * D * N + i];
        ms += mdA_b[b * D * N + i];
      }
      dA[i] = s;
      if (mdA) mdA[i] = ms;
    }
    for (int64_t d = 0; d < D; ++d) {
      double s = 0.0, ms = 0.0, sb = 0.0, msb = 0.0;
      for (int64_t b = 0; b < Bsz; ++b) {
        s += dD_b[b * D + d];
        ms += mdD_b[b * D + d];
        sb += db_b[b * D + d];
        msb += mdb_b[b * D + d];
      }
      if (dDskip) dDskip[d] = s;
      if (mdD) mdD[d] = ms;
      if (ddbias) ddbias[d] = sb;
      if (mddbias) mddbias[d] = msb;
    }
  }
  free(dA_b);
  free(mdA_b);
  free(dD_b);
  free(mdD_b);
  free(db_b);
  free(mdb_b);
  return fail ? -1 : 0;
}

int oracle_scan_bwd_ex(int64_t Bsz, int64_t D, int64_t L, int64_t N, const double* x,
                       const double* delta, const double* dbias, int flags, const double* A,
                       const double* Bm, const double* Cm, const double* Dskip, const double* z,
                       const double* h0, const double* dy, const double* dh_last, double* dx,
                       double* ddelta, double* dA, double* dBm, double* dCm, double* dDskip,
                       double* dz, double* dh0, double* ddbias, double* mdx, double* mddelta,
                       double* mdA, double* mdB, double* mdC, double* mdD, double* mdz, double* mdh0,
                       double* mddbias) {
  return oracle_scan_bwd_xm(Bsz, D, L, N, x, NULL, delta, dbias, flags, A, Bm, Cm, Dskip, z, h0, dy,
                            dh_last, dx, ddelta, dA, dBm, dCm, dDskip, dz, dh0, ddbias, mdx, mddelta,
                            mdA, mdB, mdC, mdD, mdz, mdh0, mddbias);
}

int oracle_scan_bwd(int64_t Bsz, int64_t D, int64_t L, int64_t N, const double* x,
                    const double* delta, const double* A, const double* Bm, const double* Cm,
                    const double* Dskip, const double* z, const double* h0, const double* dy,
                    const double* dh_last, double* dx, double* ddelta, double* dA, double* dBm,
                    double* dCm, double* dDskip, double* dz, double* dh0, double* mdx,
                    double* mddelta, double* mdA, double* mdB, double* mdC, double* mdD,
                    double* mdz, double* mdh0) {
  return oracle_scan_bwd_ex(Bsz, D, L, N, x, delta, NULL, 0, A, Bm, Cm, Dskip, z, h0, dy, dh_last, dx,
                            ddelta, dA, dBm, dCm, dDskip, dz, dh0, NULL, mdx, mddelta, mdA, mdB, mdC,
                            mdD, mdz, mdh0, NULL);
}
