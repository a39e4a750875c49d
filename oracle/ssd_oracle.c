/*
 * ssd_oracle.c -- plain, slow, float64 CPU oracle for the state space dual
 * (SSD, Mamba-2) form of the selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes.  The pages describe Mamba-2's SSD only in words (their
 * equations were lost in extraction): a selective SSM whose sequence map is
 * a 1-semiseparable matrix, the same object as causal-masked linear
 * attention, computed blockwise by matrix products ("Linear Attention vs
 * Softmax Attention: Can RWKV or Mamba Replace Transformers?", section
 * "Mamba (Selective State Space Models)", which also gives the state as
 * (batch, head_dim, state_dim); "RWKV-v6 vs. Mamba-3 Selective State
 * Spaces" (lesty.tech), section "3.1. State Space Duality (SSD)"; "State
 * Space Models in Large Language Models" (llms.blog), section "Mamba-2 and
 * Structured State Space Duality (SSD)").  1-semiseparable means one scalar
 * decay per step, so the reading taken is: the selective recurrence of the
 * first page's Implementation section with the decay A reduced to one
 * scalar A[h] per head, for each sequence b and head h (group g = h /
 * (heads / groups) supplies B and C), with a state of headdim x dstate:
 *
 *   dt_t    = softplus(dt[b,t,h] + dt_bias[h])     (or dt + bias, flag off)
 *   h_t     = e^(dt_t A[h]) h_{t-1} + dt_t x[b,t,h,:] B[b,t,g,:]^T
 *   y_t[p]  = sum_n C[b,t,g,n] h_t[p,n] + D[h] x[b,t,h,p]
 *   out     = y * silu(z) when z is given
 *
 * and the state after the last token.  This loop is the recurrent side of
 * the duality; its matrix side (the masked quadratic form and the chunked
 * form) is what the tests pin it against.
 *
 * Inputs are the exact float32 values the device receives; the arithmetic
 * is double.  Layouts (row-major): x, z, out (batch, L, heads, headdim);
 * dt (batch, L, heads); B, C (batch, L, groups, dstate); A, D, dt_bias
 * (heads); h0, last (batch, heads, headdim, dstate).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

static double softplus_exact(double u) { return (u > 0.0 ? u : 0.0) + log1p(exp(-fabs(u))); }

int ssd_oracle_fwd(const float *x, const float *dt, const float *dt_bias, int dt_softplus,
                   const float *A, const float *B, const float *C, const float *D,
                   const float *z, const float *h0, double *out, double *last, int64_t batch,
                   int64_t L, int64_t heads, int64_t headdim, int64_t dstate, int64_t groups) {
  if (batch < 1 || L < 0 || heads < 1 || headdim < 1 || dstate < 1 || groups < 1 ||
      heads % groups != 0 || !A)
    return -1;
  if (L > 0 && (!x || !dt || !B || !C || !out)) return -1;
  const int64_t P = headdim, N = dstate, H = heads, G = groups;
  double *h = (double *)malloc(sizeof(double) * (size_t)(P * N));
  if (!h) return -2;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t hd = 0; hd < H; ++hd) {
      const int64_t g = hd / (H / G);
      for (int64_t i = 0; i < P * N; ++i) h[i] = h0 ? (double)h0[(b * H + hd) * P * N + i] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const double u = (double)dt[(b * L + t) * H + hd] + (dt_bias ? (double)dt_bias[hd] : 0.0);
        const double d = dt_softplus ? softplus_exact(u) : u;
        const double a = exp(d * (double)A[hd]);
        const float *xt = x + ((b * L + t) * H + hd) * P;
        const float *Bt = B + ((b * L + t) * G + g) * N;
        const float *Ct = C + ((b * L + t) * G + g) * N;
        for (int64_t p = 0; p < P; ++p) {
          double y = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            h[p * N + n] = a * h[p * N + n] + d * (double)xt[p] * (double)Bt[n];
            y += (double)Ct[n] * h[p * N + n];
          }
          if (D) y += (double)D[hd] * (double)xt[p];
          const int64_t o = ((b * L + t) * H + hd) * P + p;
          if (z) {
            const double zv = (double)z[o];
            y *= zv / (1.0 + exp(-zv));
          }
          out[o] = y;
        }
      }
      if (last)
        for (int64_t i = 0; i < P * N; ++i) last[(b * H + hd) * P * N + i] = h[i];
    }
  free(h);
  return 0;
}
