/*
 * Host-memory check of the fp64 oracle (test infrastructure): built together with
 * oracle/mamba_oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer, it calls every
 * oracle entry point on small shapes with buffers allocated to their exact sizes, so an access
 * one element past any tensor, a read of an optional input passed as NULL, or undefined integer
 * arithmetic aborts the program.  Shapes include the degenerate ones (one token, one channel,
 * one state, every optional input absent).  Exit status 0 means every call ran clean and gave
 * finite results.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void ref_scan_fwd_f64(const double*, const double*, const double*, const double*, const double*,
                      const double*, const double*, const double*, int, int64_t, int64_t, int64_t,
                      int64_t, double*, double*);
void ref_state_update_f64(double*, const double*, const double*, const double*, const double*,
                          const double*, const double*, const double*, const double*, int, int64_t,
                          int64_t, int64_t, double*);
void ref_scan_bwd_f64(const double*, const double*, const double*, const double*, const double*,
                      const double*, const double*, const double*, int, const double*,
                      const double*, int64_t, int64_t, int64_t, int64_t, double*, double*, double*,
                      double*, double*, double*, double*, double*);
void ref_causal_conv1d_silu_f64(const double*, const double*, const double*, int64_t, int64_t,
                                int64_t, int64_t, double*);
void ref_affine_scan_f64(const double*, const double*, int64_t, double, double*);
void ref_set_threads(int);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

/* splitmix64, mapped to [-1, 1) */
static double uniform(void) {
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static double* filled(int64_t n, double scale, double offset) {
  double* p = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  for (int64_t i = 0; i < n; ++i) p[i] = offset + scale * uniform();
  return p;
}

static int all_finite(const double* p, int64_t n, const char* what) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) { fprintf(stderr, "%s: non-finite value at %lld\n", what, (long long)i); return 0; }
  return 1;
}

static int run_case(int64_t batch, int64_t dim, int64_t N, int64_t L, int opt_mask) {
  const int with_D = opt_mask & 1, with_z = opt_mask & 2, with_bias = opt_mask & 4,
            with_dlast = opt_mask & 8, softplus = (opt_mask & 16) ? 0 : 1;
  const int64_t nx = batch * dim * L, nbc = batch * N * L, na = dim * N, ns = batch * dim * N;
  double* u = filled(nx, 1.0, 0.0);
  double* delta = filled(nx, softplus ? 1.0 : 0.2, softplus ? 0.0 : 0.3);
  double* A = filled(na, 0.5, -1.0);
  double* B = filled(nbc, 1.0, 0.0);
  double* C = filled(nbc, 1.0, 0.0);
  double* D = with_D ? filled(dim, 1.0, 0.0) : NULL;
  double* z = with_z ? filled(nx, 1.0, 0.0) : NULL;
  double* bias = with_bias ? filled(dim, 0.1, 0.0) : NULL;
  double* out = filled(nx, 0.0, 0.0);
  double* last = filled(ns, 0.0, 0.0);
  int ok = 1;

  ref_scan_fwd_f64(u, delta, A, B, C, D, z, bias, softplus, batch, dim, N, L, out, last);
  ok &= all_finite(out, nx, "scan out") & all_finite(last, ns, "scan last_state");
  ref_scan_fwd_f64(u, delta, A, B, C, D, z, bias, softplus, batch, dim, N, L, out, NULL);

  /* one generation step from the final state, on the first token's inputs laid out per step */
  double* su = filled(batch * dim, 1.0, 0.0);
  double* sd = filled(batch * dim, 1.0, 0.0);
  double* sz = with_z ? filled(batch * dim, 1.0, 0.0) : NULL;
  double* sB = filled(batch * N, 1.0, 0.0);
  double* sC = filled(batch * N, 1.0, 0.0);
  double* sout = filled(batch * dim, 0.0, 0.0);
  if (softplus) {
    ref_state_update_f64(last, su, sd, A, sB, sC, D, sz, bias, softplus, batch, dim, N, sout);
    ok &= all_finite(sout, batch * dim, "step out");
  }

  double* dout = filled(nx, 1.0, 0.0);
  double* dlast = with_dlast ? filled(ns, 1.0, 0.0) : NULL;
  double* du = filled(nx, 0.0, 0.0);
  double* ddelta = filled(nx, 0.0, 0.0);
  double* dA = filled(na, 0.0, 0.0);
  double* dB = filled(nbc, 0.0, 0.0);
  double* dC = filled(nbc, 0.0, 0.0);
  double* dD = filled(dim, 0.0, 0.0);
  double* dz = with_z ? filled(nx, 0.0, 0.0) : NULL;
  double* dbias = filled(dim, 0.0, 0.0);
  ref_scan_bwd_f64(u, delta, A, B, C, D, z, bias, softplus, dout, dlast, batch, dim, N, L, du,
                   ddelta, dA, dB, dC, dD, dz, dbias);
  ok &= all_finite(du, nx, "du") & all_finite(ddelta, nx, "ddelta") & all_finite(dA, na, "dA") &
        all_finite(dB, nbc, "dB") & all_finite(dC, nbc, "dC") & all_finite(dD, dim, "dD") &
        all_finite(dbias, dim, "ddelta_bias");
  if (dz) ok &= all_finite(dz, nx, "dz");

  for (int64_t W = 1; W <= 4; ++W) {
    double* w = filled(dim * W, 0.5, 0.0);
    double* cb = with_bias ? filled(dim, 0.1, 0.0) : NULL;
    ref_causal_conv1d_silu_f64(u, w, cb, W, batch, dim, L, out);
    ok &= all_finite(out, nx, "conv out");
    free(w);
    free(cb);
  }

  double* a = filled(L, 0.5, 0.5);
  double* b = filled(L, 1.0, 0.0);
  double* h = filled(L, 0.0, 0.0);
  ref_affine_scan_f64(a, b, L, 0.25, h);
  ok &= all_finite(h, L, "affine scan");

  double* bufs[] = {u, delta, A, B, C, D, z, bias, out, last, su, sd, sz, sB, sC, sout, dout,
                    dlast, du, ddelta, dA, dB, dC, dD, dz, dbias, a, b, h};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) free(bufs[i]);
  if (!ok)
    fprintf(stderr, "failed: batch %lld dim %lld N %lld L %lld options %d\n", (long long)batch,
            (long long)dim, (long long)N, (long long)L, opt_mask);
  return ok;
}

int main(void) {
  static const int64_t shapes[][4] = {
      {1, 1, 1, 1}, {1, 1, 16, 1}, {1, 1, 1, 17}, {2, 3, 16, 1}, {2, 3, 16, 33},
      {3, 5, 4, 64}, {1, 7, 16, 100}, {2, 2, 2, 2}};
  int ok = 1;
  for (int threads = 1; threads <= 3; threads += 2) {
    ref_set_threads(threads);
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
      for (int opt = 0; opt < 32; ++opt)
        ok &= run_case(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], opt);
  }
  printf(ok ? "oracle sanitizer checks: clean\n" : "oracle sanitizer checks: FAILED\n");
  return ok ? 0 : 1;
}
