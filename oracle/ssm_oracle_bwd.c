/*
 * ssm_oracle_bwd.c -- plain, slow, float64 CPU oracle for the gradients of
 * the selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests and the benchmark's cpu_baseline leg use
 * it.  It shares no code, header or constant with the HIP library.
 *
 * What it computes.  The forward is the sequential loop of ssm_oracle.c
 * ("Linear Attention vs Softmax Attention: Can RWKV or Mamba Replace
 * Transformers?", section "Implementation"; softplus step size from "State
 * Space Models in Large Language Models", section "Dynamic
 * Parameterization").  The pages give no gradient formulas: the gradients
 * are those of that loop, for the scalar
 *     loss = sum(dout * out) + sum(dlast * last_state),
 * with respect to every input: x, delta (before softplus), delta_bias, A, B,
 * C, D, z and the initial state.  They are obtained by running the loop's
 * steps backwards (reverse-mode chain rule), with the forward states of
 * the channel kept in a float64 history:
 *
 *   per token t, from the last to the first, with a = dloss/dh_t:
 *     dy      = dout * silu(z)   (or dout without a gate);
 *     dz      = dout * y * silu'(z),  silu'(v) = s (1 + v (1 - s)), s = sigmoid(v);
 *     dD     += dy x;   dx = D dy;
 *     a[n]   += C[n] dy;            dC[n] += dy h_t[n];
 *     ddt     = sum_n a[n] (A[n] e^{dt A[n]} h_{t-1}[n] + B[n] x);
 *     dA[n]  += a[n] dt e^{dt A[n]} h_{t-1}[n];
 *     dB[n]  += a[n] dt x;          dx += sum_n a[n] dt B[n];
 *     a[n]    = a[n] e^{dt A[n]}    (now dloss/dh_{t-1});
 *     ddelta  = ddt * sigmoid(delta + bias) (softplus' ; ddt itself without
 *               softplus);  dbias += ddelta;
 *   and dh0 = a after the first token (a = dlast before the last token).
 *
 * Threads own contiguous ranges of channels d (all sequences b): dA, dD,
 * dbias for a channel have one writer.  dB and dC sum over channels: each
 * thread sums its channels in order into a private buffer, and the buffers
 * are added in thread order (the grouping, hence the last bits, depends on
 * the thread count).
 *
 * Layouts as in ssm_oracle.c; dout like out (batch, L, dim); dlast and dh0
 * (batch, dim, dstate); dA (dim, dstate); dD, dbias (dim); dB, dC (batch,
 * L, dstate); every gradient is double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const float *x, *delta, *bias, *A, *B, *C, *D, *z, *h0, *dout, *dlast;
  double *dx, *ddelta, *dA, *dB, *dC, *dD, *dz, *dbias, *dh0;
  int softplus;
  int64_t batch, L, dim, N;
  int64_t d_begin, d_end;
  double *pB, *pC; /* private dB, dC */
} bjob_t;

static double softplus_exact(double u) { return (u > 0.0 ? u : 0.0) + log1p(exp(-fabs(u))); }
static double sigmoid(double u) { return 1.0 / (1.0 + exp(-u)); }

static void bwd_channel(const bjob_t *j, int64_t b, int64_t d, double *hist, double *a) {
  const int64_t N = j->N, dim = j->dim, L = j->L;
  const double bias = j->bias ? (double)j->bias[d] : 0.0;
  const double dskip = j->D ? (double)j->D[d] : 0.0;
  /* forward: hist[(t+1)*N + n] = h_t[n], hist[n] = h_{-1} = h0 */
  for (int64_t n = 0; n < N; ++n) hist[n] = j->h0 ? (double)j->h0[(b * dim + d) * N + n] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const int64_t i = (b * L + t) * dim + d, bc = (b * L + t) * N;
    const double u = (double)j->delta[i] + bias;
    const double dt = j->softplus ? softplus_exact(u) : u;
    const double xv = (double)j->x[i];
    for (int64_t n = 0; n < N; ++n)
      hist[(t + 1) * N + n] = exp(dt * (double)j->A[d * N + n]) * hist[t * N + n] +
                              dt * (double)j->B[bc + n] * xv;
  }
  /* backward */
  for (int64_t n = 0; n < N; ++n) a[n] = j->dlast ? (double)j->dlast[(b * dim + d) * N + n] : 0.0;
  for (int64_t t = L - 1; t >= 0; --t) {
    const int64_t i = (b * L + t) * dim + d, bc = (b * L + t) * N;
    const double u = (double)j->delta[i] + bias;
    const double dt = j->softplus ? softplus_exact(u) : u;
    const double xv = (double)j->x[i];
    const double *ht = hist + (t + 1) * N, *hp = hist + t * N;
    double y = dskip * xv;
    for (int64_t n = 0; n < N; ++n) y += (double)j->C[bc + n] * ht[n];
    const double g = (double)j->dout[i];
    double dy = g;
    if (j->z) {
      const double zv = (double)j->z[i];
      const double s = sigmoid(zv);
      dy = g * zv * s;
      j->dz[i] = g * y * s * (1.0 + zv * (1.0 - s));
    }
    j->dD[d] += dy * xv;
    double dxv = dskip * dy, ddt = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      a[n] += (double)j->C[bc + n] * dy;
      j->pC[bc + n] += dy * ht[n];
    }
    for (int64_t n = 0; n < N; ++n) {
      const double An = (double)j->A[d * N + n], Bn = (double)j->B[bc + n];
      const double dAn = exp(dt * An);
      ddt += a[n] * (An * dAn * hp[n] + Bn * xv);
      j->dA[d * N + n] += a[n] * dt * dAn * hp[n];
      j->pB[bc + n] += a[n] * dt * xv;
      dxv += a[n] * dt * Bn;
      a[n] *= dAn;
    }
    j->dx[i] = dxv;
    const double dd = j->softplus ? ddt * sigmoid(u) : ddt;
    j->ddelta[i] = dd;
    j->dbias[d] += dd;
  }
  for (int64_t n = 0; n < N; ++n) j->dh0[(b * dim + d) * N + n] = a[n];
}

static void *bworker(void *arg) {
  const bjob_t *j = (const bjob_t *)arg;
  double *hist = (double *)malloc(sizeof(double) * (size_t)((j->L + 1) * j->N));
  double *a = (double *)malloc(sizeof(double) * (size_t)j->N);
  if (!hist || !a) { free(hist); free(a); return (void *)1; }
  for (int64_t d = j->d_begin; d < j->d_end; ++d)
    for (int64_t b = 0; b < j->batch; ++b) bwd_channel(j, b, d, hist, a);
  free(hist); free(a);
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on thread/alloc failure.
 * dz may be NULL when z is NULL; every other gradient pointer is required. */
int ssm_oracle_scan_bwd(const float *x, const float *delta, const float *delta_bias,
                        int delta_softplus, const float *A, const float *B, const float *C,
                        const float *D_skip, const float *z, const float *h0, const float *dout,
                        const float *dlast, double *dx, double *ddelta, double *dA, double *dB,
                        double *dC, double *dD, double *dz, double *dbias, double *dh0,
                        int64_t batch, int64_t L, int64_t dim, int64_t dstate, int nthreads) {
  if (!A || !dA || !dD || !dbias || !dh0 || !dB || !dC || (z && !dz)) return -1;
  if (L > 0 && (!x || !delta || !B || !C || !dout || !dx || !ddelta)) return -1;
  if (batch < 1 || L < 0 || dim < 1 || dstate < 1) return -1;
  const int64_t N = dstate;
  memset(dA, 0, sizeof(double) * (size_t)(dim * N));
  memset(dD, 0, sizeof(double) * (size_t)dim);
  memset(dbias, 0, sizeof(double) * (size_t)dim);
  memset(dB, 0, sizeof(double) * (size_t)(batch * L * N));
  memset(dC, 0, sizeof(double) * (size_t)(batch * L * N));
  if (nthreads < 1) nthreads = 1;
  if (nthreads > dim) nthreads = (int)dim;
  bjob_t *jobs = (bjob_t *)calloc((size_t)nthreads, sizeof(bjob_t));
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) { free(jobs); free(th); return -2; }
  int rc = 0, started = 0;
  for (int k = 0; k < nthreads && rc == 0; ++k) {
    bjob_t *j = &jobs[k];
    j->x = x; j->delta = delta; j->bias = delta_bias; j->A = A; j->B = B; j->C = C;
    j->D = D_skip; j->z = z; j->h0 = h0; j->dout = dout; j->dlast = dlast;
    j->dx = dx; j->ddelta = ddelta; j->dA = dA; j->dB = dB; j->dC = dC; j->dD = dD; j->dz = dz;
    j->dbias = dbias; j->dh0 = dh0; j->softplus = delta_softplus;
    j->batch = batch; j->L = L; j->dim = dim; j->N = N;
    j->d_begin = dim * k / nthreads; j->d_end = dim * (k + 1) / nthreads;
    j->pB = (double *)calloc((size_t)(batch * L * N) + 1, sizeof(double));
    j->pC = (double *)calloc((size_t)(batch * L * N) + 1, sizeof(double));
    if (!j->pB || !j->pC) { rc = -2; break; }
  }
  if (rc == 0) {
    for (int k = 0; k < nthreads; ++k) {
      if (nthreads == 1) { if (bworker(&jobs[k])) rc = -2; continue; }
      if (pthread_create(&th[k], NULL, bworker, &jobs[k]) != 0) { rc = -2; break; }
      ++started;
    }
    for (int k = 0; k < started; ++k) {
      void *ret = NULL;
      pthread_join(th[k], &ret);
      if (ret) rc = -2;
    }
  }
  for (int k = 0; k < nthreads; ++k) {
    if (rc == 0 && jobs[k].pB)
      for (int64_t i = 0; i < batch * L * N; ++i) { dB[i] += jobs[k].pB[i]; dC[i] += jobs[k].pC[i]; }
    free(jobs[k].pB); free(jobs[k].pC);
  }
  free(jobs); free(th);
  return rc;
}
