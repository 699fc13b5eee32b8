/*
 * mamba_oracle.c -- plain fp64 CPU reference of Mamba's selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this file;
 * only the test-suite, the smoke check and the benchmark's CPU-baseline leg use it.  It shares
 * no code, header, table or constant with the GPU library.
 *
 * What it computes (sources, by page title and section):
 *  - "Mamba" (elemedex dex entry), section "How it works": the discrete SSM is the linear
 *    recurrence h_t = Abar*h_{t-1} + Bbar*x_t with readout y_t = C*h_t, and Delta, B and C are
 *    functions of the current token (selection).
 *  - "State Spaces, Selectively -- Mamba" (papermap explainer), chapter 02 "The Discretized View":
 *    a step size Delta turns h'(t) = A h(t) + B x(t) into the discrete recurrence, with Abar and
 *    Bbar derived from (Delta, A, B); a large Delta lets the current token dominate the state.
 *  - "Mamba remembers by forgetting, read closely" (interactiveml.org), the scalar equation:
 *    zero-order hold with A = -1 gives h_t = exp(-Delta_t) h_{t-1} + (1 - exp(-Delta_t)) x_t,
 *    starting from a zero state.
 *  - The per-element rules that the pages leave open are taken as: Delta = softplus(raw + bias)
 *    (bias added first, softplus only when requested), Abar = exp(Delta*A[d,n]),
 *    Bbar*x = Delta*B[b,n,t]*u[b,d,t], readout after the update, an optional skip D[d]*u added
 *    before the gate, and the output gate y*silu(z) ("Mamba" (visual-learn), "Simplifications and
 *    limits": the block ends in an output gate; "Mamba" (elemedex) "How it works": a
 *    multiplicative gate).
 *
 * The recurrence is evaluated strictly sequentially in t for every channel, in double precision,
 * with no scan, blocking or reordering: the pages state that composing affine updates in any
 * grouping reaches the same result ("Mamba remembers by forgetting", the composition equation),
 * so the sequential loop is the plain definition.  OpenMP parallelism is over independent
 * (batch, channel) pairs only; the t and n loops stay in order.
 *
 * Layouts (dense, row-major): u, delta, z, out: (batch, dim, seqlen); B, C: (batch, dstate,
 * seqlen); A: (dim, dstate); D, delta_bias: (dim); last_state: (batch, dim, dstate).
 * NULL for D, z, delta_bias or last_state means: no skip, no gate, zero bias, not written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(x) = log(1 + e^x), in the overflow-free form max(x,0) + log1p(e^-|x|). */
static double sp(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

double ref_softplus_f64(double x) { return sp(x); }
double ref_silu_f64(double z) { return silu(z); }

void ref_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int ref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* One token of the selective SSM for one channel: updates h[0..N-1] in place and returns y.
 * x = u[b,d,t], draw = raw Delta, bn/cn = B[b,:,t]/C[b,:,t] with element stride bstride. */
static double one_step(double* h, const double* Arow, int64_t N, double x, double draw, double bias,
                       int softplus_flag, const double* Bp, const double* Cp, int64_t bstride,
                       int has_D, double Dd, int has_z, double zz) {
  double dt = draw + bias;
  if (softplus_flag) dt = sp(dt);
  double y = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    double abar = exp(dt * Arow[n]);
    double bx = dt * Bp[n * bstride] * x;
    h[n] = abar * h[n] + bx;
    y += Cp[n * bstride] * h[n];
  }
  if (has_D) y += Dd * x;
  if (has_z) y *= silu(zz);
  return y;
}

/* Whole-sequence forward from a zero state. */
void ref_scan_fwd_f64(const double* u, const double* delta, const double* A, const double* B,
                      const double* C, const double* D, const double* z, const double* delta_bias,
                      int softplus_flag, int64_t batch, int64_t dim, int64_t dstate,
                      int64_t seqlen, double* out, double* last_state) {
  const int64_t nch = batch * dim;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int64_t b = ch / dim, d = ch % dim;
    double* h = (double*)calloc((size_t)dstate, sizeof(double));
    const double bias = delta_bias ? delta_bias[d] : 0.0;
    const double* Arow = A + d * dstate;
    const int64_t row = (b * dim + d) * seqlen;
    for (int64_t t = 0; t < seqlen; ++t) {
      out[row + t] = one_step(h, Arow, dstate, u[row + t], delta[row + t], bias, softplus_flag,
                              B + b * dstate * seqlen + t, C + b * dstate * seqlen + t, seqlen,
                              D != NULL, D ? D[d] : 0.0, z != NULL, z ? z[row + t] : 0.0);
    }
    if (last_state) memcpy(last_state + (b * dim + d) * dstate, h, (size_t)dstate * sizeof(double));
    free(h);
  }
}

/* One generation step: state (batch, dim, dstate) is read and written in place; u, delta, z, out
 * are (batch, dim); B, C are (batch, dstate). */
void ref_state_update_f64(double* state, const double* u, const double* delta, const double* A,
                          const double* B, const double* C, const double* D, const double* z,
                          const double* delta_bias, int softplus_flag, int64_t batch, int64_t dim,
                          int64_t dstate, double* out) {
  const int64_t nch = batch * dim;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int64_t b = ch / dim, d = ch % dim;
    out[ch] = one_step(state + ch * dstate, A + d * dstate, dstate, u[ch], delta[ch],
                       delta_bias ? delta_bias[d] : 0.0, softplus_flag, B + b * dstate,
                       C + b * dstate, 1, D != NULL, D ? D[d] : 0.0, z != NULL, z ? z[ch] : 0.0);
  }
}

/* Scalar affine recurrence h_t = a_t*h_{t-1} + b_t from h_{-1} = h0 (the update
 * "multiply by a, then add b" of "Mamba" (visual-learn), "Training without stepping token by
 * token"). Writes every h_t. */
void ref_affine_scan_f64(const double* a, const double* b, int64_t n, double h0, double* h) {
  double s = h0;
  for (int64_t t = 0; t < n; ++t) {
    s = a[t] * s + b[t];
    h[t] = s;
  }
}

/*
 * Gradients of the whole-sequence forward (the backward pass that "activation recomputation"
 * refers to in "State Spaces, Selectively -- Mamba" (papermap), chapter 01/02), written out as the
 * adjoint of the recurrence above.  For loss = sum(out * dout) + sum(last_state * dlast):
 *
 *   with s = sigmoid(z):  dy_t = dout_t * z_t * s       (dy_t = dout_t without a gate)
 *                         dz_t = dout_t * ypre_t * s * (1 + z_t * (1 - s)),  ypre_t = sum_n C h_t + D u_t
 *   lam_t[n] = dy_t * C[n,t] + Abar_{t+1}[n] * lam_{t+1}[n],   lam_{L-1} carry = dlast
 *   h_t = Abar_t h_{t-1} + Delta_t B_t u_t  gives
 *     dDelta_t  = sum_n lam_t (Abar_t A_n h_{t-1} + B_t u_t);  dDelta_raw = dDelta * softplus'(raw + bias)
 *     dA[d,n]  += lam_t Abar_t Delta_t h_{t-1}
 *     dB[b,n,t] += lam_t Delta_t u_t          (summed over channels d)
 *     dC[b,n,t] += dy_t h_t                   (summed over channels d)
 *     du_t      = dy_t D + sum_n lam_t Delta_t B_t
 *     dD[d]    += dy_t u_t;   ddelta_bias[d] += dDelta_raw_t
 *
 * Every h_t of a channel is stored by a plain forward loop (no recomputation scheme).  Parallel
 * over channels d (each thread owns whole rows of dA, dD, ddelta_bias); dB and dC are summed into
 * one buffer per thread, added in thread order at the end.  dlast may be NULL (zero); dz is written
 * only when z is given; dD and ddelta_bias are always written (the gradient for a zero skip or
 * bias when D or delta_bias is NULL).
 */
void ref_scan_bwd_f64(const double* u, const double* delta, const double* A, const double* B,
                      const double* C, const double* D, const double* z, const double* delta_bias,
                      int softplus_flag, const double* dout, const double* dlast, int64_t batch,
                      int64_t dim, int64_t N, int64_t L, double* du, double* ddelta, double* dA,
                      double* dB, double* dC, double* dD, double* dz, double* ddelta_bias) {
  const int64_t nbc = batch * N * L;
  int nthreads = 1;
#ifdef _OPENMP
  nthreads = omp_get_max_threads();
#endif
  double* pB = (double*)calloc((size_t)nthreads * (size_t)nbc, sizeof(double));
  double* pC = (double*)calloc((size_t)nthreads * (size_t)nbc, sizeof(double));
#pragma omp parallel num_threads(nthreads)
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* myB = pB + (size_t)tid * (size_t)nbc;
    double* myC = pC + (size_t)tid * (size_t)nbc;
    double* H = (double*)malloc((size_t)L * (size_t)N * sizeof(double));
    double* dtv = (double*)malloc((size_t)L * sizeof(double));
    double* sig = (double*)malloc((size_t)L * sizeof(double));
    double* ypre = (double*)malloc((size_t)L * sizeof(double));
    double* lam = (double*)malloc((size_t)N * sizeof(double));
    double* gA = (double*)malloc((size_t)N * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t d = 0; d < dim; ++d) {
      const double* Arow = A + d * N;
      const double bias = delta_bias ? delta_bias[d] : 0.0;
      const double Dd = D ? D[d] : 0.0;
      for (int64_t n = 0; n < N; ++n) gA[n] = 0.0;
      double gD = 0.0, gbias = 0.0;
      for (int64_t b = 0; b < batch; ++b) {
        const int64_t row = (b * dim + d) * L;
        const double* Bb = B + b * N * L;
        const double* Cb = C + b * N * L;
        /* forward, keeping every state */
        for (int64_t t = 0; t < L; ++t) {
          const double raw = delta[row + t] + bias;
          dtv[t] = softplus_flag ? sp(raw) : raw;
          sig[t] = softplus_flag ? 1.0 / (1.0 + exp(-raw)) : 1.0;
          double y = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            const double hp = t > 0 ? H[(t - 1) * N + n] : 0.0;
            const double h = exp(dtv[t] * Arow[n]) * hp + dtv[t] * Bb[n * L + t] * u[row + t];
            H[t * N + n] = h;
            y += Cb[n * L + t] * h;
          }
          ypre[t] = y + Dd * u[row + t];
        }
        /* reverse: adjoint recurrence */
        for (int64_t n = 0; n < N; ++n) lam[n] = dlast ? dlast[(b * dim + d) * N + n] : 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
          const double x = u[row + t], dt = dtv[t];
          double dy = dout[row + t];
          if (z) {
            const double zz = z[row + t];
            const double s = 1.0 / (1.0 + exp(-zz));
            dz[row + t] = dout[row + t] * ypre[t] * s * (1.0 + zz * (1.0 - s));
            dy = dout[row + t] * zz * s;
          }
          gD += dy * x;
          double gu = dy * Dd, gdt = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            const double l = dy * Cb[n * L + t] + lam[n];
            const double hp = t > 0 ? H[(t - 1) * N + n] : 0.0;
            const double a_t = exp(dt * Arow[n]);
            gdt += l * (a_t * Arow[n] * hp + Bb[n * L + t] * x);
            gA[n] += l * a_t * dt * hp;
            myB[(b * N + n) * L + t] += l * dt * x;
            gu += l * dt * Bb[n * L + t];
            myC[(b * N + n) * L + t] += dy * H[t * N + n];
            lam[n] = l * a_t;
          }
          const double graw = gdt * sig[t];
          du[row + t] = gu;
          ddelta[row + t] = graw;
          gbias += graw;
        }
      }
      for (int64_t n = 0; n < N; ++n) dA[d * N + n] = gA[n];
      dD[d] = gD;
      ddelta_bias[d] = gbias;
    }
    free(H);
    free(dtv);
    free(sig);
    free(ypre);
    free(lam);
    free(gA);
  }
  for (int64_t i = 0; i < nbc; ++i) {
    double sb = 0.0, sc = 0.0;
    for (int t = 0; t < nthreads; ++t) {
      sb += pB[(size_t)t * (size_t)nbc + i];
      sc += pC[(size_t)t * (size_t)nbc + i];
    }
    dB[i] = sb;
    dC[i] = sc;
  }
  free(pB);
  free(pC);
}

/*
 * Short causal depthwise convolution followed by SiLU, producing the scan input u from x (the
 * block step before the SSM: "Mamba" (elemedex), "How it works" / "State Spaces, Selectively"
 * (papermap) ch.02, which place a short convolution and a nonlinearity before the selective SSM;
 * the width is not on the pages and is a parameter here).  Cross-correlation with left zero
 * padding, the newest token multiplying the last tap:
 *     u[b,d,t] = silu(bias[d] + sum_{k=0}^{W-1} w[d,k] * x[b,d,t-(W-1)+k]),  x[.,.,t<0] = 0.
 * Layouts: x, u (batch, dim, L); w (dim, W); bias (dim) or NULL (zero).
 */
void ref_causal_conv1d_silu_f64(const double* x, const double* w, const double* bias, int64_t W,
                                int64_t batch, int64_t dim, int64_t L, double* u) {
  const int64_t nch = batch * dim;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int64_t d = ch % dim;
    const double* xr = x + ch * L;
    for (int64_t t = 0; t < L; ++t) {
      double acc = bias ? bias[d] : 0.0;
      for (int64_t k = 0; k < W; ++k) {
        const int64_t s = t - (W - 1) + k;
        if (s >= 0) acc += w[d * W + k] * xr[s];
      }
      u[ch * L + t] = silu(acc);
    }
  }
}
