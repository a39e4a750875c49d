/*
 * conv_oracle.c -- plain, slow, float64 CPU oracle for the short causal
 * depthwise convolution that precedes the scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes.  "Linear Attention vs Softmax Attention: Can RWKV or
 * Mamba Replace Transformers?" (shyankdev.com), section "Implementation":
 * the block's main branch goes through a depthwise Conv1d (one filter of
 * kernel_size taps per channel, groups = channels, with bias) padded by
 * kernel_size - 1 on both sides and cut back to the first seq_len outputs,
 * which makes it causal, then through SiLU; the figure of the same page
 * ("Mamba-2 Blocks") names it a 1D causal convolution with k = 4.  With the
 * padding on the left, output t sees inputs t-(W-1) .. t, and the filter tap
 * k (0-based) multiplies input t-(W-1)+k:
 *
 *   out[b,t,d] = act( bias[d] + sum_{k=0}^{W-1} w[d,k] * xx[b, t-(W-1)+k, d] )
 *
 * with act = SiLU (v / (1 + e^-v)) or the identity, and xx the input
 * extended to the left by a conv state: xx[b, s, d] = x[b, s, d] for s >= 0
 * and state0[b, d, (W-1)+s] for -(W-1) <= s < 0 (zeros without a state,
 * which is the page's zero padding).  The state after the call holds the
 * last W-1 inputs, oldest first: state1[b, d, j] = xx[b, L-(W-1)+j, d].
 * One decoding step is this with L = 1.
 *
 * Inputs are the exact values the device receives, as float32; the
 * arithmetic is double.  Layouts (row-major): x (batch, L, dim); w (dim, W);
 * bias (dim); state0 / state1 (batch, dim, W-1); out (batch, L, dim) double.
 */
#include <math.h>
#include <stdint.h>

static double xx_at(const float *x, const float *state0, int64_t b, int64_t s, int64_t d,
                    int64_t L, int64_t dim, int64_t W) {
  if (s >= 0) return (double)x[(b * L + s) * dim + d];
  return state0 ? (double)state0[(b * dim + d) * (W - 1) + (W - 1) + s] : 0.0;
}

int conv_oracle_fwd(const float *x, const float *w, const float *bias, int silu,
                    const float *state0, double *out, double *state1, int64_t batch, int64_t L,
                    int64_t dim, int64_t W) {
  if (batch < 1 || L < 0 || dim < 1 || W < 1) return -1;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t d = 0; d < dim; ++d) {
      for (int64_t t = 0; t < L; ++t) {
        double acc = bias ? (double)bias[d] : 0.0;
        for (int64_t k = 0; k < W; ++k)
          acc += (double)w[d * W + k] * xx_at(x, state0, b, t - (W - 1) + k, d, L, dim, W);
        out[(b * L + t) * dim + d] = silu ? acc / (1.0 + exp(-acc)) : acc;
      }
      if (state1)
        for (int64_t j = 0; j < W - 1; ++j)
          state1[(b * dim + d) * (W - 1) + j] = xx_at(x, state0, b, L - (W - 1) + j, d, L, dim, W);
    }
  return 0;
}
