/* oracle_driver.c -- the C oracles under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure).
 *
 * Runs the forward, gradient, convolution and SSD oracles on small random
 * inputs over edge shapes (no tokens, one token, one channel, one state, the
 * optional inputs present and absent, one and several threads) and checks
 * that bad arguments are refused.  Every buffer is allocated at its exact
 * size, so a read or write past one is reported.  Exit status: the number of
 * failed checks (a sanitizer report aborts the run instead).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ssm_oracle_scan(const float *x, const float *delta, const float *delta_bias,
                    int delta_softplus, const float *A, const float *B, const float *C,
                    const float *D_skip, const float *z, const float *h0, double *out,
                    double *last_state, int64_t batch, int64_t L, int64_t dim, int64_t dstate,
                    int nthreads);
int ssm_oracle_scan_bwd(const float *x, const float *delta, const float *delta_bias,
                        int delta_softplus, const float *A, const float *B, const float *C,
                        const float *D_skip, const float *z, const float *h0, const float *dout,
                        const float *dlast, double *dx, double *ddelta, double *dA, double *dB,
                        double *dC, double *dD, double *dz, double *dbias, double *dh0,
                        int64_t batch, int64_t L, int64_t dim, int64_t dstate, int nthreads);
int conv_oracle_fwd(const float *x, const float *w, const float *bias, int silu,
                    const float *state0, double *out, double *state1, int64_t batch, int64_t L,
                    int64_t dim, int64_t W);
int ssd_oracle_fwd(const float *x, const float *dt, const float *dt_bias, int dt_softplus,
                   const float *A, const float *B, const float *C, const float *D,
                   const float *z, const float *h0, double *out, double *last, int64_t batch,
                   int64_t L, int64_t heads, int64_t headdim, int64_t dstate, int64_t groups);

static int g_bad = 0;
static unsigned g_seed = 12345u;

static float rnd(void) {
  g_seed = g_seed * 1664525u + 1013904223u;
  return (float)((g_seed >> 8) * (1.0 / 16777216.0)) - 0.5f;
}

/* n floats; an empty array is a valid pointer to zero bytes (any access to
 * it is reported) */
static float *fa(int64_t n, float lo, float span) {
  if (n <= 0) return (float *)malloc(0);
  float *p = (float *)malloc(sizeof(float) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) p[i] = lo + span * (rnd() + 0.5f);
  return p;
}
static double *da(int64_t n) {
  return n > 0 ? (double *)calloc((size_t)n, sizeof(double)) : (double *)malloc(0);
}

static void check(int cond, const char *what) {
  if (!cond) {
    printf("FAILED: %s\n", what);
    ++g_bad;
  }
}

static int all_finite(const double *p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static void scan_case(int64_t b, int64_t L, int64_t D, int64_t N, int opt, int threads) {
  const int64_t T = b * L * D, R = b * L * N;
  float *x = fa(T, -1, 2), *dl = fa(T, -3, 4), *z = opt ? fa(T, -2, 4) : NULL;
  float *A = fa(D * N, -2, 1.9f), *B = fa(R, -1, 2), *C = fa(R, -1, 2);
  float *bias = opt ? fa(D, -1, 1) : NULL, *Ds = opt ? fa(D, -1, 2) : NULL;
  float *h0 = opt ? fa(b * D * N, -1, 2) : NULL;
  double *out = da(T), *last = da(b * D * N);
  check(ssm_oracle_scan(x, dl, bias, 1, A, B, C, Ds, z, h0, out, last, b, L, D, N, threads) == 0,
        "scan runs");
  check(all_finite(out, T) && all_finite(last, b * D * N), "scan outputs finite");
  /* gradients of the same problem */
  float *dout = fa(T, -1, 2), *dlast = opt ? fa(b * D * N, -1, 2) : NULL;
  double *dx = da(T), *ddl = da(T), *dz = opt ? da(T) : NULL, *dA = da(D * N), *dB = da(R),
         *dC = da(R), *dD = da(D), *db = da(D), *dh0 = da(b * D * N);
  check(ssm_oracle_scan_bwd(x, dl, bias, 1, A, B, C, Ds, z, h0, dout, dlast, dx, ddl, dA,
                            dB, dC, dD, dz, db, dh0, b, L, D, N,
                            threads) == 0,
        "scan gradients run");
  check(all_finite(dx, T) && all_finite(dA, D * N) && all_finite(dh0, b * D * N),
        "gradients finite");
  free(x); free(dl); free(z); free(A); free(B); free(C); free(bias); free(Ds); free(h0);
  free(out); free(last); free(dout); free(dlast); free(dx); free(ddl); free(dz); free(dA);
  free(dB); free(dC); free(dD); free(db); free(dh0);
}

static void conv_case(int64_t b, int64_t L, int64_t D, int64_t W, int opt) {
  float *x = fa(b * L * D, -1, 2), *w = fa(D * W, -1, 2), *bias = opt ? fa(D, -1, 2) : NULL;
  float *s0 = opt ? fa(b * D * (W - 1), -1, 2) : NULL;
  double *out = da(b * L * D), *s1 = da(b * D * (W - 1));
  check(conv_oracle_fwd(x, w, bias, opt, s0, out, s1, b, L, D, W) == 0, "conv runs");
  check(all_finite(out, b * L * D), "conv outputs finite");
  free(x); free(w); free(bias); free(s0); free(out); free(s1);
}

static void ssd_case(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int opt) {
  float *x = fa(b * L * H * P, -1, 2), *dt = fa(b * L * H, -3, 4), *A = fa(H, -2, 1.9f);
  float *B = fa(b * L * G * N, -1, 2), *C = fa(b * L * G * N, -1, 2);
  float *bias = opt ? fa(H, -1, 1) : NULL, *D = opt ? fa(H, -1, 2) : NULL;
  float *z = opt ? fa(b * L * H * P, -2, 4) : NULL, *h0 = opt ? fa(b * H * P * N, -1, 2) : NULL;
  double *out = da(b * L * H * P), *last = da(b * H * P * N);
  check(ssd_oracle_fwd(x, dt, bias, 1, A, B, C, D, z, h0, out, last, b, L, H, P, N, G) == 0,
        "ssd runs");
  check(all_finite(out, b * L * H * P) && all_finite(last, b * H * P * N), "ssd outputs finite");
  free(x); free(dt); free(A); free(B); free(C); free(bias); free(D); free(z); free(h0);
  free(out); free(last);
}

int main(void) {
  const int64_t Ls[] = {0, 1, 2, 17};
  const int64_t Ds[] = {1, 3};
  const int64_t Ns[] = {1, 4, 16};
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 2; ++j)
      for (int k = 0; k < 3; ++k)
        for (int opt = 0; opt < 2; ++opt) {
          scan_case(1, Ls[i], Ds[j], Ns[k], opt, 1);
          scan_case(2, Ls[i], Ds[j], Ns[k], opt, 3);
        }
  for (int64_t W = 1; W <= 4; ++W)
    for (int opt = 0; opt < 2; ++opt) {
      conv_case(1, 0, 3, W, opt);
      conv_case(2, 5, 3, W, opt);
    }
  for (int opt = 0; opt < 2; ++opt) {
    ssd_case(1, 0, 2, 3, 4, 1, opt);
    ssd_case(2, 7, 4, 3, 5, 2, opt);
  }
  /* refused arguments */
  float f[16] = {0};
  double d[16] = {0};
  check(ssm_oracle_scan(NULL, f, NULL, 1, f, f, f, NULL, NULL, NULL, d, NULL, 1, 1, 1, 1, 1) < 0,
        "scan refuses a null input");
  check(ssm_oracle_scan(f, f, NULL, 1, f, f, f, NULL, NULL, NULL, d, NULL, 1, 1, 1, 0, 1) < 0,
        "scan refuses dstate 0");
  check(ssm_oracle_scan(f, f, NULL, 1, f, f, f, NULL, NULL, NULL, d, NULL, -1, 1, 1, 1, 1) < 0,
        "scan refuses batch < 0");
  check(ssm_oracle_scan_bwd(f, f, NULL, 1, f, f, f, NULL, f, NULL, f, NULL, d, d, d, d, d, d,
                            NULL, d, d, 1, 1, 1, 1, 1) < 0,
        "gradients refuse a gate without dz");
  check(conv_oracle_fwd(f, f, NULL, 0, NULL, d, NULL, 1, 1, 1, 0) < 0, "conv refuses width 0");
  check(ssd_oracle_fwd(f, f, NULL, 1, f, f, f, NULL, NULL, NULL, d, NULL, 1, 1, 3, 1, 1, 2) < 0,
        "ssd refuses groups that do not divide the heads");
  printf("oracle driver: %d failed check(s)\n", g_bad);
  return g_bad;
}
