/*
 * ssm_oracle.c -- plain, slow, float64 CPU oracle for the selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (the sequential selective recurrence, written out):
 *
 *   Discretisation and recurrence follow "Linear Attention vs Softmax
 *   Attention: Can RWKV or Mamba Replace Transformers?" (shyankdev.com),
 *   section "Implementation", the SelectiveSSMLayer forward loop:
 *     A_bar[n]  = exp(Delta_t * A[d,n])                 (zero-order-hold decay)
 *     B_bar x   = Delta_t * B_t[n] * x_t                (the simplified input term
 *                                                        the page's code uses)
 *     h_t[n]    = A_bar[n] * h_{t-1}[n] + Delta_t * B_t[n] * x_t
 *     y_t       = sum_n C_t[n] * h_t[n] + D[d] * x_t
 *   then the output is gated by SiLU(z): y_t * z_t * sigmoid(z_t).
 *   Delta_t = softplus(delta_t + bias[d]) follows "State Space Models in
 *   Large Language Models" (llms.blog), section "Dynamic Parameterization".
 *   The recurrent (one-token) view of the same system, section
 *   "Discretization" of that page, is this loop with L = 1.
 *
 * Readings where the pages leave a step open:
 *   - softplus is the exact log(1 + e^u), evaluated as max(u,0)+log1p(e^-|u|);
 *     with the flag off, Delta = delta + bias.
 *   - the D-skip is added before the gate (the page's code adds D*x inside the
 *     loop and gates afterwards).
 *   - missing optional inputs: bias -> 0, D -> no skip, z -> no gate,
 *     h0 -> zeros, last_state -> not written.
 *
 * Inputs are the exact values the device receives, as float32 (a bf16 value
 * widens to float32 without rounding); every step is done in double.
 * Channels (b,d) are independent; threads take contiguous ranges of them and
 * write disjoint outputs, so the result does not depend on the thread count.
 *
 * Layouts (row-major, contiguous):
 *   x, delta, z : (batch, L, dim)       B, C : (batch, L, dstate)
 *   A : (dim, dstate)   bias, D : (dim)  h0 : (batch, dim, dstate)
 *   out : (batch, L, dim) double         last_state : (batch, dim, dstate) double
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const float *x, *delta, *bias, *A, *B, *C, *D, *z, *h0;
  double *out, *last;
  int softplus;
  int64_t batch, L, dim, N;
  int64_t c_begin, c_end; /* channel range [begin, end) over batch*dim */
} job_t;

static double softplus_exact(double u) {
  /* log(1 + e^u) without overflow for large u and without cancellation */
  return (u > 0.0 ? u : 0.0) + log1p(exp(-fabs(u)));
}

static void run_channel(const job_t *j, int64_t ch, double *h) {
  const int64_t b = ch / j->dim, d = ch % j->dim;
  const int64_t N = j->N, dim = j->dim, L = j->L;
  for (int64_t n = 0; n < N; ++n)
    h[n] = j->h0 ? (double)j->h0[(b * dim + d) * N + n] : 0.0;
  const double bias = j->bias ? (double)j->bias[d] : 0.0;
  const double dskip = j->D ? (double)j->D[d] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const int64_t i = (b * L + t) * dim + d;     /* (b,t,d) */
    const int64_t bc = (b * L + t) * N;          /* (b,t,0) */
    const double u = (double)j->delta[i] + bias;
    const double dt = j->softplus ? softplus_exact(u) : u;
    const double xv = (double)j->x[i];
    double y = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double dA = exp(dt * (double)j->A[d * N + n]);
      h[n] = dA * h[n] + dt * (double)j->B[bc + n] * xv;
      y += (double)j->C[bc + n] * h[n];
    }
    y += dskip * xv;
    if (j->z) {
      const double zv = (double)j->z[i];
      y *= zv / (1.0 + exp(-zv));
    }
    j->out[i] = y;
  }
  if (j->last)
    for (int64_t n = 0; n < N; ++n) j->last[(b * dim + d) * N + n] = h[n];
}

static void *worker(void *arg) {
  const job_t *j = (const job_t *)arg;
  double *h = (double *)malloc(sizeof(double) * (size_t)(j->N > 0 ? j->N : 1));
  if (!h) return (void *)1;
  for (int64_t ch = j->c_begin; ch < j->c_end; ++ch) run_channel(j, ch, h);
  free(h);
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on thread/alloc failure. */
int ssm_oracle_scan(const float *x, const float *delta, const float *delta_bias,
                    int delta_softplus, const float *A, const float *B,
                    const float *C, const float *D_skip, const float *z,
                    const float *h0, double *out, double *last_state,
                    int64_t batch, int64_t L, int64_t dim, int64_t dstate,
                    int nthreads) {
  if (!x || !delta || !A || !B || !C || !out) return -1;
  if (batch < 0 || L < 0 || dim < 0 || dstate < 1) return -1;
  const int64_t nch = batch * dim;
  if (nch == 0) return 0;
  if (L == 0) {
    /* no tokens: the final state is the initial one */
    if (last_state)
      for (int64_t i = 0; i < nch * dstate; ++i) last_state[i] = h0 ? (double)h0[i] : 0.0;
    return 0;
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nch) nthreads = (int)nch;
  job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) { free(jobs); free(th); return -2; }
  int rc = 0, started = 0;
  for (int k = 0; k < nthreads; ++k) {
    job_t *j = &jobs[k];
    j->x = x; j->delta = delta; j->bias = delta_bias; j->A = A; j->B = B; j->C = C;
    j->D = D_skip; j->z = z; j->h0 = h0; j->out = out; j->last = last_state;
    j->softplus = delta_softplus; j->batch = batch; j->L = L; j->dim = dim; j->N = dstate;
    j->c_begin = nch * k / nthreads; j->c_end = nch * (k + 1) / nthreads;
    if (nthreads == 1) { if (worker(j)) rc = -2; continue; }
    if (pthread_create(&th[k], NULL, worker, j) != 0) { rc = -2; break; }
    ++started;
  }
  for (int k = 0; k < started; ++k) {
    void *ret = NULL;
    pthread_join(th[k], &ret);
    if (ret) rc = -2;
  }
  free(jobs); free(th);
  return rc;
}
