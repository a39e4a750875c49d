/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective-scan library.
 *
 * Two operations, both defined by the sequential loop of the SelectiveSSMLayer
 * in "Linear Attention vs Softmax Attention: Can RWKV or Mamba Replace
 * Transformers?" (shyankdev.com), section "Implementation", with the step size
 * Delta = softplus(parameter + projection) of "State Space Models in Large
 * Language Models" (llms.blog), section "Dynamic Parameterization":
 *
 *   for each sequence b and channel d, with state h[0..N) (float32):
 *     Delta_t = softplus(delta[b,t,d] + delta_bias[d])   (or delta+bias if the flag is 0)
 *     h[n]    = exp(Delta_t * A[d,n]) * h[n] + Delta_t * B[b,t,n] * x[b,t,d]
 *     y       = sum_n C[b,t,n] * h[n] + D_skip[d] * x[b,t,d]
 *     out[b,t,d] = z ? y * z*sigmoid(z) : y
 *
 * ssm_scan_fwd runs it over a whole sequence (the fused "hardware-aware scan"
 * of llms.blog, section "The Hardware-Aware Parallel Associative Scan": inputs
 * read once, only outputs written, no (b,L,D,N) intermediate in memory);
 * ssm_state_update is the one-token recurrent step used in decoding (same
 * page, section "Discretization", recurrent view), updating the state in place.
 *
 * Conventions common to every entry point:
 *   - Pointers named as tensors are DEVICE pointers (hipMalloc'd or torch
 *     device memory) on the current HIP device; all tensors are contiguous and
 *     row-major in the layouts given below.
 *   - "act" tensors (x, delta, z, B, C, out) have the element type `dtype`
 *     (SSM_DTYPE_F32 or SSM_DTYPE_BF16); A, D_skip, delta_bias and every state
 *     tensor are always float32.  Arithmetic and the state are float32; bf16
 *     outputs are rounded to nearest even.
 *   - The caller owns every buffer.  The library allocates no device memory,
 *     keeps no per-call state and never synchronises: work is enqueued on
 *     `stream` (NULL = the default stream) and the call returns at once.
 *     Results are valid once the caller orders later work after the stream.
 *   - Argument errors are detected on the host before anything is enqueued:
 *     the call returns a negative ssm_status_t, leaves every output untouched
 *     and records a message for ssm_last_error().  A failed launch returns
 *     SSM_ERR_HIP.  Faults during execution surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - Alignment: act tensors must be aligned to their element size; A, D_skip,
 *     delta_bias to 4 bytes; B and C to 4 bytes; state tensors to 16 bytes.
 *   - Outputs may not overlap inputs (nor the workspace), except that in
 *     ssm_scan_fwd last_state may be the same buffer as initial_state
 *     (resume in place).
 *   - Not thread-hostile: concurrent calls on different streams are fine.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_SCAN_ABI_VERSION 7

typedef enum { SSM_DTYPE_F32 = 0, SSM_DTYPE_BF16 = 1 } ssm_dtype_t;

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = -1,        /* a required pointer is NULL                        */
  SSM_ERR_SHAPE = -2,       /* a size is negative / zero where it may not be, or too large */
  SSM_ERR_UNSUPPORTED = -3, /* dstate outside [1, 64], unknown dtype, flag not 0/1 */
  SSM_ERR_ALIGN = -4,       /* a pointer violates the alignment rules above        */
  SSM_ERR_ALIAS = -5,       /* an output overlaps an input                         */
  SSM_ERR_WORKSPACE = -6,   /* workspace smaller than ssm_scan_fwd_workspace_bytes */
  SSM_ERR_HIP = -7          /* the HIP runtime refused a launch or query           */
} ssm_status_t;

/*
 * Forward selective scan over whole sequences.
 *   x, delta, z, out : (batch, seqlen, dim) act     -- delta is the raw step
 *                      parameter, before softplus; z may be NULL (no gate)
 *   delta_bias       : (dim) float32 or NULL (= 0)
 *   delta_softplus   : 1 = Delta = softplus(delta + bias), 0 = Delta = delta + bias
 *   A                : (dim, dstate) float32 (negative for a decaying state)
 *   B, C             : (batch, seqlen, dstate) act, shared by all channels
 *   D_skip           : (dim) float32 or NULL (no skip term)
 *   initial_state    : (batch, dim, dstate) float32 or NULL (= zeros)
 *   last_state       : (batch, dim, dstate) float32 or NULL; receives h after
 *                      the last token
 *   batch, dim >= 1; seqlen >= 0 (seqlen == 0 only copies the initial state
 *   into last_state); 1 <= dstate <= 64.
 *   workspace        : device scratch of at least
 *                      ssm_scan_fwd_workspace_bytes(...) bytes, 256-byte
 *                      aligned; may be NULL when that size is 0.  Its contents
 *                      need no initialisation and are garbage afterwards.
 * The result does not depend on how the work is partitioned beyond float32
 * rounding order, and is bitwise reproducible run to run on one device.
 */
int ssm_scan_fwd(const void* x, const void* delta, const float* delta_bias, int delta_softplus,
                 const float* A, const void* B, const void* C, const float* D_skip,
                 const void* z, void* out, float* last_state, const float* initial_state,
                 int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace size the call above needs for these sizes on the current device
 * (0 when none is needed).  Never fails; returns 0 for invalid sizes. */
size_t ssm_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                    int dtype);

/*
 * ssm_scan_fwd with the time split chosen by the caller.  The sequence is
 * cut into chunks of chunk_len tokens (rounded up to a multiple of 8) that
 * run in parallel and are chained through the associative composition of
 * the per-token affine maps h -> a h + b (the local transforms that the
 * chenyuan1125.github.io page on Mamba's selective state spaces, section
 * "Selectivity Removes the Convolution Shortcut; Scan Restores
 * Parallelism", combines into intervals); chunk_len >= seqlen runs every
 * sequence as one chunk (no workspace).  chunk_len == 0 is the library's
 * own choice, i.e. ssm_scan_fwd.  At most 65535 chunks per sequence
 * (SSM_ERR_SHAPE beyond; chunk_len < 0 is SSM_ERR_SHAPE too).  Arguments
 * and results as ssm_scan_fwd: any split gives the same values up to
 * float32 rounding order.  For tuning the split on other devices and
 * shapes, and for checking that results do not depend on it.
 */
int ssm_scan_fwd_chunked(const void* x, const void* delta, const float* delta_bias,
                         int delta_softplus, const float* A, const void* B, const void* C,
                         const float* D_skip, const void* z, void* out, float* last_state,
                         const float* initial_state, int64_t batch, int64_t seqlen, int64_t dim,
                         int64_t dstate, int dtype, int64_t chunk_len, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Workspace size ssm_scan_fwd_chunked needs (0 when none is needed, or for
 * invalid sizes). */
size_t ssm_scan_fwd_chunked_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim,
                                            int64_t dstate, int dtype, int64_t chunk_len);

/*
 * ssm_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments and results as ssm_scan_fwd, without the workspace: the chunk
 * summaries go to a scratch array that the library holds on each device it
 * runs on (64 MiB, reserved with the library's code on that device until
 * the process ends; its device address is looked up once per device, on
 * the first call made with that device current).  This call allocates
 * nothing.  Sizes whose ssm_scan_fwd_workspace_bytes exceeds 64 MiB are
 * refused with SSM_ERR_WORKSPACE (use ssm_scan_fwd with a workspace).
 * Every call on one device shares that device's scratch, which keeps the
 * last call's contents (nothing in it needs to start at zero): calls that
 * overlap in time on one device -- on different streams, or from different
 * host threads without ordering -- race and give wrong results.  Calls
 * ordered on one stream are fine.
 */
int ssm_scan_fwd_noalloc(const void* x, const void* delta, const float* delta_bias,
                         int delta_softplus, const float* A, const void* B, const void* C,
                         const float* D_skip, const void* z, void* out, float* last_state,
                         const float* initial_state, int64_t batch, int64_t seqlen, int64_t dim,
                         int64_t dstate, int dtype, hipStream_t stream);

/*
 * Forward selective scan over packed variable-length sequences.
 * Padding a batch of unequal sequences on the right feeds the padding tokens
 * through the recurrence and changes the state they leave behind; the
 * remedy that "Linear Attention vs Softmax Attention: Can RWKV or Mamba
 * Replace Transformers?" (shyankdev.com) gives in "Common Mistakes" (mistake
 * 1 and "1. Naive Sequence Padding in Batched Training") and in "Best
 * Practices" (item 4) is to concatenate the sequences without padding and
 * pass their offsets.  Each sequence starts from its own state, as in the
 * same page's "State Reset and Isolation" (section "Production Deployment
 * Considerations", item 2).
 *   x, delta, z, out : (total_len, dim) act, the sequences one after another
 *   B, C             : (total_len, dstate) act
 *   cu_seqlens       : (nseq + 1) int32 DEVICE array of token offsets:
 *                      sequence s is tokens [cu_seqlens[s], cu_seqlens[s+1]);
 *                      must satisfy 0 = cu[0] <= cu[1] <= ... <= cu[nseq] =
 *                      total_len (empty sequences are allowed).  The contents
 *                      are not checked (that would need a synchronisation):
 *                      offsets that break this rule give unspecified values
 *                      but every memory access stays inside the buffers.
 *   initial_state    : (nseq, dim, dstate) float32 or NULL (= zeros)
 *   last_state       : (nseq, dim, dstate) float32 or NULL; receives each
 *                      sequence's state after its last token (its initial
 *                      state if it is empty).  May not overlap initial_state.
 *   A, D_skip, delta_bias, delta_softplus, dtype : as in ssm_scan_fwd.
 *   1 <= nseq < 2^24; total_len >= 0.
 *   workspace        : at least ssm_scan_fwd_varlen_workspace_bytes(...)
 *                      bytes, 256-byte aligned, as in ssm_scan_fwd.
 * Each sequence's out and last_state equal those of ssm_scan_fwd run on that
 * sequence alone (batch = 1) with its initial state, up to float32 rounding
 * order.
 */
int ssm_scan_fwd_varlen(const void* x, const void* delta, const float* delta_bias,
                        int delta_softplus, const float* A, const void* B, const void* C,
                        const float* D_skip, const void* z, void* out, float* last_state,
                        const float* initial_state, const int32_t* cu_seqlens, int64_t nseq,
                        int64_t total_len, int64_t dim, int64_t dstate, int dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace size ssm_scan_fwd_varlen needs (0 when none is needed, or for
 * invalid sizes). */
size_t ssm_scan_fwd_varlen_workspace_bytes(int64_t nseq, int64_t total_len, int64_t dim,
                                           int64_t dstate, int dtype);

/*
 * Gradients of ssm_scan_fwd (the backward pass used in training).  The
 * pages give the forward only; the gradients are those of its loop, for the
 * scalar loss = sum(dout * out) + sum(dlast_state * last_state), with
 * respect to every input.  Like the forward, it keeps no per-token states
 * in memory but recomputes them stripe by stripe, the memory trick that the
 * chenyuan1125.github.io page on Mamba's selective state spaces (section
 * "Selectivity Removes the Convolution Shortcut; Scan Restores
 * Parallelism") attributes to the original kernel's backward pass.
 *   inputs: as ssm_scan_fwd (x, delta, delta_bias, delta_softplus, A, B, C,
 *           D_skip, z, initial_state; same layouts and dtypes), plus
 *     dout         : (batch, seqlen, dim) act, the gradient of out
 *     dlast_state  : (batch, dim, dstate) float32 or NULL (= 0)
 *   outputs (all overwritten, none accumulated into):
 *     dx, ddelta   : (batch, seqlen, dim) act; ddelta is the gradient of
 *                    the raw delta (before bias and softplus)
 *     dz           : (batch, seqlen, dim) act; required when z is given
 *     dA           : (dim, dstate) float32
 *     dB, dC       : (batch, seqlen, dstate) float32
 *     dD           : (dim) float32 or NULL (must be NULL without D_skip)
 *     ddelta_bias  : (dim) float32 or NULL
 *     dinitial_state : (batch, dim, dstate) float32 or NULL
 *   dstate must be 4, 8 or 16 (SSM_ERR_UNSUPPORTED otherwise); alignment as
 *   ssm_scan_fwd, with B and C aligned to 4 elements and dB, dC to 16 bytes.
 *   seqlen is at most 65535 * 32 = 2097120 (one launch holds the stripes of
 *   32 tokens), and batch * seqlen * dstate and batch * dim * dstate stay
 *   below 2^31 - 256 (SSM_ERR_SHAPE beyond).
 *   workspace: at least ssm_scan_bwd_workspace_bytes(...) bytes, 256-byte
 *   aligned (0 when seqlen is 0).
 * Arithmetic is float32; the sums over channels, tokens and sequences are
 * formed from per-workgroup partials added in a fixed order, so results are
 * bitwise reproducible run to run on one device.  Outputs may not overlap
 * inputs, each other or the workspace.
 */
int ssm_scan_bwd(const void* x, const void* delta, const float* delta_bias, int delta_softplus,
                 const float* A, const void* B, const void* C, const float* D_skip,
                 const void* z, const float* initial_state, const void* dout,
                 const float* dlast_state, void* dx, void* ddelta, void* dz, float* dA, float* dB,
                 float* dC, float* dD, float* ddelta_bias, float* dinitial_state, int64_t batch,
                 int64_t seqlen, int64_t dim, int64_t dstate, int dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* Workspace size ssm_scan_bwd needs (0 for invalid sizes or seqlen 0). */
size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                    int dtype);

/*
 * The state space dual (SSD, Mamba-2) form of the selective scan, on the
 * matrix cores.  The pages describe it in words: with one scalar decay per
 * head the selective SSM is a 1-semiseparable matrix (the same object as
 * causal-masked linear attention), computed blockwise: matrix products
 * inside chunks of 64-128 tokens, boundary states passed between chunks
 * ("Linear Attention vs Softmax Attention: Can RWKV or Mamba Replace
 * Transformers?" (shyankdev.com), section "Mamba (Selective State Space
 * Models)"; "RWKV-v6 vs. Mamba-3 Selective State Spaces" (lesty.tech),
 * sections "3.1. State Space Duality (SSD)" and "4. Hardware Acceleration";
 * "State Space Models in Large Language Models" (llms.blog), section
 * "Mamba-2 and Structured State Space Duality (SSD)").  Per sequence b and
 * head h (group g = h / (nheads / ngroups) supplies B and C), with a
 * float32 state of headdim x dstate:
 *   dt_t = softplus(dt[b,t,h] + dt_bias[h])   (or dt + dt_bias if the flag is 0)
 *   h_t  = e^(dt_t A[h]) h_{t-1} + dt_t x[b,t,h,:] B[b,t,g,:]^T
 *   y[b,t,h,p] = sum_n C[b,t,g,n] h_t[p,n] + D[h] x[b,t,h,p];  out = y silu(z)
 *   x, z, out     : (batch, seqlen, nheads, headdim) bf16; z may be NULL
 *   dt            : (batch, seqlen, nheads) bf16, the raw step before bias/softplus
 *   A, D, dt_bias : (nheads) float32; D and dt_bias may be NULL
 *   B, C          : (batch, seqlen, ngroups, dstate) bf16
 *   initial_state, last_state : (batch, nheads, headdim, dstate) float32 or NULL
 *                   (last_state may be the initial_state buffer: resume in place)
 *   dtype must be SSM_DTYPE_BF16, headdim 64, dstate 64 or 128, ngroups
 *   dividing nheads; x, B, C 16-byte aligned, z and out 8-byte aligned.
 *   workspace: at least ssm_ssd_fwd_workspace_bytes(...) bytes, 256-byte
 *   aligned (may be NULL when that size is 0: when (batch, head) pairs
 *   already fill the device the sequence is not cut into segments).
 * Chunks of 64 tokens; the products are bf16 matrix-core operations with
 * float32 accumulation and a float32 state (their bf16 operands: the
 * masked C B^T, the decay-weighted x, a bf16 copy of the state for the
 * readout), so results match the float64 definition to bf16 accuracy.
 */
int ssm_ssd_fwd(const void* x, const void* dt, const float* dt_bias, int dt_softplus,
                const float* A, const void* B, const void* C, const float* D, const void* z,
                void* out, float* last_state, const float* initial_state, int64_t batch,
                int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace size ssm_ssd_fwd needs (0 when none, or for invalid sizes). */
size_t ssm_ssd_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int64_t ngroups);

/*
 * One decoding step for `batch` sequences: the recurrence above with one token.
 *   state       : (batch, dim, dstate) float32, read and overwritten in place
 *   x, delta, z, out : (batch, dim) act; z may be NULL
 *   B, C        : (batch, dstate) act
 *   delta_bias, D_skip : (dim) float32 or NULL;  A : (dim, dstate) float32
 * Equivalent to ssm_scan_fwd with seqlen = 1 and initial_state = last_state =
 * state.  One launch: batch * dim * (dstate / 4 when dstate % 4 == 0, else 1)
 * must stay below 2^31 - 256 (SSM_ERR_SHAPE otherwise).
 * Alignment (SSM_ERR_ALIGN otherwise): state 16 bytes; every other array to
 * its element size; and when dstate % 4 == 0 (each lane then updates four
 * states with vector accesses) A 16 bytes and B, C to four elements (16
 * bytes for float32, 8 for bf16).  Tensors from a PyTorch allocation meet
 * all of these; views offset into one may not.
 */
int ssm_state_update(float* state, const void* x, const void* delta, const float* delta_bias,
                     int delta_softplus, const float* A, const void* B, const void* C,
                     const float* D_skip, const void* z, void* out,
                     int64_t batch, int64_t dim, int64_t dstate, int dtype, hipStream_t stream);

/*
 * Causal depthwise convolution + SiLU, the step that produces the scan's x.
 * "Linear Attention vs Softmax Attention: Can RWKV or Mamba Replace
 * Transformers?" (shyankdev.com), section "Implementation": the main branch
 * passes through a depthwise Conv1d (kernel_size taps per channel, bias,
 * padding kernel_size - 1, output cut to seq_len: causal) and then SiLU; the
 * figure on the same page gives k = 4.  With W = width:
 *   out[b,t,d] = silu( bias[d] + sum_{k<W} weight[d,k] * xx[b, t-(W-1)+k, d] )
 * where xx is x with the conv state in front: xx[b,s,d] = x[b,s,d] for s >= 0
 * and initial_conv_state[b, d, (W-1)+s] for -(W-1) <= s < 0 (zeros if NULL,
 * the page's zero padding).  Tap W-1 multiplies the current token.
 *   x, out             : (batch, seqlen, dim) act
 *   weight             : (dim, width) float32;  bias : (dim) float32 or NULL
 *   initial_conv_state : (batch, dim, width-1) act or NULL; the inputs
 *                        before the first token, oldest first
 *   final_conv_state   : (batch, dim, width-1) act or NULL; receives the last
 *                        width-1 inputs (exact copies), oldest first
 *   silu               : 1 = apply SiLU, 0 = the convolution alone
 *   2 <= width <= 4; batch, dim >= 1; seqlen >= 0; one launch holds
 *   batch * ceil(seqlen / 16) * ceil(dim / 64) < 2^25 (SSM_ERR_SHAPE beyond).
 * Arithmetic is float32 (fused multiply-adds in tap order); bf16 outputs are
 * rounded to nearest even.  Outputs may not overlap inputs.
 */
int ssm_causal_conv1d_fwd(const void* x, const float* weight, const float* bias,
                          const void* initial_conv_state, void* out, void* final_conv_state,
                          int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int silu,
                          int dtype, hipStream_t stream);

/*
 * One decoding step of the convolution above for `batch` sequences:
 *   conv_state : (batch, dim, width-1) act, read and shifted in place (the
 *                oldest input drops out, x becomes the newest)
 *   x, out     : (batch, dim) act;  weight, bias, silu, width, dtype as above.
 *   batch * dim < 2^31 - 256 (one lane per channel in one launch).
 * Equivalent to ssm_causal_conv1d_fwd with seqlen = 1 and initial_conv_state
 * = final_conv_state = conv_state.
 */
int ssm_causal_conv1d_update(void* conv_state, const void* x, const float* weight,
                             const float* bias, void* out, int64_t batch, int64_t dim,
                             int64_t width, int silu, int dtype, hipStream_t stream);

/* Message for the most recent non-OK status returned on the calling thread
 * ("" if none).  The pointer stays valid until the next call on that thread. */
const char* ssm_last_error(void);

/* SSM_SCAN_ABI_VERSION of the loaded library. */
int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SSM_SCAN_H */
