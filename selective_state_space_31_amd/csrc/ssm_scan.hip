// ssm_scan.hip -- selective scan forward and one-token state update for
// MI355X (gfx950, CDNA4), behind the C ABI declared in include/ssm_scan.h.
//
// The arithmetic per token and channel (see the header for the citation):
//   Delta = softplus(delta + bias);  h[n] = exp(Delta*A[n]) h[n] + Delta*B[n]*x;
//   y = C.h + D*x;  out = y * silu(z).
//
// Layout decisions (all tensors channel-last, as the pages' module keeps
// them):
//   * one lane owns one channel's N-wide float32 state in VGPRs for the whole
//     time range it scans; the state never goes to memory;
//   * the 64 lanes of a wave own 64 consecutive channels, so every per-token
//     load of x / delta / z and every store of out is one contiguous 128-byte
//     (bf16) or 256-byte (fp32) row segment;
//   * B_t and C_t are shared by all channels of a sequence, so they are
//     wave-uniform: scalar loads into SGPRs, converted by the scalar ALU,
//     consumed directly as SGPR operands of the vector FMAs;
//   * exp(Delta*A) is computed as exp2(Delta * A*log2(e)) with the product
//     A*log2(e) formed once per lane.  When a channel's A has the S4D-real
//     shape A[n] = (n+1)*A[0] (detected from the data, never assumed), the N
//     decays are the powers r, r^2, ... of r = exp(Delta*A[0]), one
//     transcendental and N-1 multiplies instead of N transcendentals.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "ssm_scan.h"

#include "host_util.hpp"
#include "kernels.hpp"

namespace ssm {

// Forward launchers are instantiated in the fwd_*.hip units (compiled in
// parallel); see _build.py.
#define SSM_FWD_INSTANCES(X)                                                       \
  X(float, 4, true) X(float, 8, true) X(float, 16, true) X(float, 32, true)        \
  X(float, 4, false) X(float, 16, false) X(float, 64, false)                       \
  X(bf16_t, 4, true) X(bf16_t, 8, true) X(bf16_t, 16, true) X(bf16_t, 32, true)    \
  X(bf16_t, 4, false) X(bf16_t, 16, false) X(bf16_t, 64, false)
#define SSM_EXTERN_FWD(TA, NT, EX)                                                     \
  extern template int launch_fwd_flags<TA, NT, EX, false>(const FwdArgs<TA>&, int64_t, bool,  \
                                                          bool, hipStream_t);                 \
  extern template int launch_fwd_flags<TA, NT, EX, true>(const FwdArgs<TA>&, int64_t, bool,   \
                                                         bool, hipStream_t);
SSM_FWD_INSTANCES(SSM_EXTERN_FWD)

// Carry pass (the backward's recomputation of the states entering its
// stripes, and of the adjoints entering them from the end).  For each
// (sequence b, state n, channel d) the chunk summaries are folded in order,
// h <- e^(A[d,n] S_c) h + H_c; slot 0 of ws_H receives the initial state and
// slot c+1 is overwritten with the state entering chunk c+1.
//
// The fold is split over the G waves of a workgroup (block = 64 channels of
// one (b, n), G waves), so that its serial depth is about (K-1)/G and not
// K-1 even when there are few (b, n, d) lanes:
//   1. wave g composes the summaries of its range of chunks into one,
//      (S, H) = "decay the incoming state by e^(A S), then add H" -- the
//      affine maps compose as (a1,b1) then (a2,b2) = (a2 a1, a2 b1 + b2), and
//      the decays multiply by adding S;
//   2. through LDS, wave g folds the composites of waves 0..g-1 onto the
//      initial state: the state entering its range;
//   3. wave g walks its range again from there, storing the entering states.
// Decays use exp_acc (the fold runs over the whole sequence in float32).
constexpr int kCarryMaxWaves = 16;
constexpr int kCarryRegs = 16;  // summaries a wave keeps in registers between steps 1 and 3
constexpr int kCarryUnroll = 8;

__device__ __forceinline__ float carry_decay(float an, float S) {
  float unused;
  return exp_acc(an * S, unused);
}

// Block (channel tile [and chain], state n, sequence b): x-blocks from
// `tiles` on run the second chain (the backward carries the forward states
// and the adjoints in one launch); the chains share A and the split.
__global__ void __launch_bounds__(64 * kCarryMaxWaves) fwd_carry_kernel(
    const float* __restrict__ A, CarryChain c0, CarryChain c1, int tiles, int dim, int N, int K,
    int per) {
  __shared__ float lds_S[kCarryMaxWaves][64], lds_H[kCarryMaxWaves][64];
  const bool second = static_cast<int>(blockIdx.x) >= tiles;
  const CarryChain& cc = second ? c1 : c0;
  const int lane = threadIdx.x & 63;
  const int g = threadIdx.x >> 6;
  const int n = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int d = (static_cast<int>(blockIdx.x) - (second ? tiles : 0)) * 64 + lane;
  const bool valid = d < dim;
  const int dl = valid ? d : dim - 1;
  const float an = A[static_cast<size_t>(dl) * N + n];
  const size_t sstride = static_cast<size_t>(dim), hstride = static_cast<size_t>(N) * dim;
  const float* sp = cc.ws_S + static_cast<size_t>(b) * (K - 1) * sstride + dl;  // chunk 0
  float* hslot0 = cc.ws_H + (static_cast<size_t>(b) * K * N + n) * dim + dl;     // slot 0
  float* hp = hslot0 + hstride;  // slot c+1 <- chunk c (read, then overwritten)
  const int c0i = g * per;
  const int c1i = (c0i + per < K - 1) ? c0i + per : K - 1;
  const float hinit = cc.h0 ? cc.h0[(b * dim + dl) * N + n] : 0.0f;
  if (g == 0 && valid) hslot0[0] = hinit;
  // step 2: the composites of waves 0..g-1 (in LDS) applied to h
  auto prefix = [&](float h) {
    for (int w = 0; w < g; ++w) h = __builtin_fmaf(carry_decay(an, lds_S[w][lane]), h, lds_H[w][lane]);
    return h;
  };

  if (per <= kCarryRegs) {
    // the wave's summaries stay in registers from step 1 to step 3
    float Sv[kCarryRegs], Hv[kCarryRegs];
#pragma unroll
    for (int j = 0; j < kCarryRegs; ++j) {
      const int c = (c0i + j < c1i) ? c0i + j : c1i - 1;
      Sv[j] = sp[c * sstride];
      Hv[j] = hp[c * hstride];
    }
    float cS = 0.0f, cH = 0.0f;
#pragma unroll
    for (int j = 0; j < kCarryRegs; ++j) {
      if (c0i + j < c1i) {
        const float e = carry_decay(an, Sv[j]);  // chunk j's decay, kept for step 3
        cH = __builtin_fmaf(e, cH, Hv[j]);
        cS += Sv[j];
        Sv[j] = e;
      }
    }
    lds_S[g][lane] = cS;
    lds_H[g][lane] = cH;
    __syncthreads();
    float h = prefix(hinit);
#pragma unroll
    for (int j = 0; j < kCarryRegs; ++j) {
      if (c0i + j < c1i) {
        h = __builtin_fmaf(Sv[j], h, Hv[j]);
        if (valid) hp[(c0i + j) * hstride] = h;
      }
    }
    return;
  }

  // long ranges: read the summaries twice, kCarryUnroll at a time
  float cS = 0.0f, cH = 0.0f;
  for (int c = c0i; c < c1i; c += kCarryUnroll) {
    float Sv[kCarryUnroll], Hv[kCarryUnroll];
#pragma unroll
    for (int j = 0; j < kCarryUnroll; ++j) {
      const int ci = (c + j < c1i) ? c + j : c1i - 1;
      Sv[j] = sp[ci * sstride];
      Hv[j] = hp[ci * hstride];
    }
#pragma unroll
    for (int j = 0; j < kCarryUnroll; ++j) {
      if (c + j < c1i) {
        cH = __builtin_fmaf(carry_decay(an, Sv[j]), cH, Hv[j]);
        cS += Sv[j];
      }
    }
  }
  lds_S[g][lane] = cS;
  lds_H[g][lane] = cH;
  __syncthreads();
  float h = prefix(hinit);
  for (int c = c0i; c < c1i; c += kCarryUnroll) {
    float Sv[kCarryUnroll], Hv[kCarryUnroll];
#pragma unroll
    for (int j = 0; j < kCarryUnroll; ++j) {
      const int ci = (c + j < c1i) ? c + j : c1i - 1;
      Sv[j] = sp[ci * sstride];
      Hv[j] = hp[ci * hstride];
    }
#pragma unroll
    for (int j = 0; j < kCarryUnroll; ++j) {
      if (c + j < c1i) {
        h = __builtin_fmaf(carry_decay(an, Sv[j]), h, Hv[j]);
        if (valid) hp[(c + j) * hstride] = h;
      }
    }
  }
}

// Packed sequences with no tokens: last_state = initial state (or zeros).
// Used when the call has no tokens at all (else the output pass stores them).
// Block (s, part): the blocks of a sequence that has tokens leave at once.
__global__ void __launch_bounds__(256) fwd_varlen_empty_kernel(const int* __restrict__ cu,
                                                               const float* __restrict__ h0,
                                                               float* __restrict__ last_state,
                                                               int dim, int N) {
  const int s = blockIdx.x;
  if (cu[s + 1] > cu[s]) return;
  const size_t per = static_cast<size_t>(dim) * N;
  const size_t base = static_cast<size_t>(s) * per;
  for (size_t i = static_cast<size_t>(blockIdx.y) * 256 + threadIdx.x; i < per;
       i += static_cast<size_t>(gridDim.y) * 256)
    last_state[base + i] = h0 ? h0[base + i] : 0.0f;
}

// ----------------------------------------------------------------------------
// decode: one token per sequence, state streamed once (read, update, write)
// ----------------------------------------------------------------------------
template <typename TA>
struct DecArgs {
  float* __restrict__ state;
  const TA* __restrict__ x;
  const TA* __restrict__ delta;
  const float* __restrict__ bias;
  const float* __restrict__ A;
  const TA* __restrict__ B;
  const TA* __restrict__ C;
  const float* __restrict__ Dsk;
  const TA* __restrict__ z;
  TA* __restrict__ out;
  int64_t batch;
  int dim;
  int N;
  int softplus;
};

// Four consecutive values of a B or C row (the row start is aligned to 4
// elements, so float32 rows give one 16-byte load, bf16 rows one 8-byte load).
__device__ __forceinline__ void load_quad(const float* p, float (&v)[4]) {
  const float4 w = *reinterpret_cast<const float4*>(p);
  v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
}
__device__ __forceinline__ void load_quad(const bf16_t* p, float (&v)[4]) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(w.x << 16);
  v[1] = __uint_as_float(w.x & 0xffff0000u);
  v[2] = __uint_as_float(w.y << 16);
  v[3] = __uint_as_float(w.y & 0xffff0000u);
}

// The state is touched once per step, so its 16-byte accesses carry the
// nontemporal hint: streamed through the caches instead of kept in them
// (measured on the 256 x 5120 x 16 step: 44.5 -> 36 us).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t load_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
}
__device__ __forceinline__ void store_stream(float* p, f32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}

// dstate = 4G (G = 1, 2, 4, 8, 16): G lanes per (sequence, channel), each
// owning 4 consecutive states, so a wave's state accesses are one contiguous
// 1 KiB stretch per instruction.  The lanes of a channel each compute the
// channel's softplus (cheaper than sharing it: the step is bound by HBM) and
// sum their partial readouts with G-lane shuffles.  When every channel of the
// wave has A of the S4D-real shape, A[n] = (n+1) A[0], the lane's decays are
// e^(Delta A[4q]) and three further factors r = e^(Delta A[0]) applied against
// r's two-float value; otherwise every decay is its own accurate exponential.
template <typename TA, int G>
__global__ void __launch_bounds__(256) decode_quad_kernel(DecArgs<TA> a) {
  constexpr int N = 4 * G;
  // lane counts stay below 2^31 (checked on the host): 32-bit index arithmetic
  const uint32_t nch = static_cast<uint32_t>(a.batch * a.dim);
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  const bool valid = gid < nch * G;
  const uint32_t c = valid ? gid / G : nch - 1;
  const int q = static_cast<int>(gid % G);
  float* sp = a.state + static_cast<size_t>(c) * N + 4 * q;
  const f32x4_t hv = load_stream(sp);
  const float xv = to_f32(a.x[c]);
  const float raw0 = to_f32(a.delta[c]);
  const float zv = a.z ? to_f32(a.z[c]) : 0.0f;
  const uint32_t b = c / static_cast<uint32_t>(a.dim);
  const int d = static_cast<int>(c - b * static_cast<uint32_t>(a.dim));
  const float4 Av = *reinterpret_cast<const float4*>(a.A + static_cast<size_t>(d) * N + 4 * q);
  const float A0 = a.A[static_cast<size_t>(d) * N];
  float Bv[4], Cv[4];
  load_quad(a.B + static_cast<size_t>(b) * N + 4 * q, Bv);
  load_quad(a.C + static_cast<size_t>(b) * N + 4 * q, Cv);
  const float raw = raw0 + (a.bias ? a.bias[d] : 0.0f);
  const float dt = a.softplus ? softplus_f32(raw) : raw;
  const float dx = dt * xv;
  float h[4] = {hv[0], hv[1], hv[2], hv[3]};
  const float Aa[4] = {Av.x, Av.y, Av.z, Av.w};
  bool pow_ok = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) pow_ok = pow_ok && (Aa[i] == static_cast<float>(4 * q + i + 1) * A0);
  float y = 0.0f;
  if (__all(pow_ok)) {
    float rl, pl;
    const float rh = exp_acc(dt * A0, rl);
    float p = exp_acc(dt * Aa[0], pl);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = __builtin_fmaf(p, h[i], dx * Bv[i]);
      y = __builtin_fmaf(Cv[i], h[i], y);
      if (i < 3) p = __builtin_fmaf(p, rh, p * rl);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float unused;
      h[i] = __builtin_fmaf(exp_acc(dt * Aa[i], unused), h[i], dx * Bv[i]);
      y = __builtin_fmaf(Cv[i], h[i], y);
    }
  }
  // sum the partial readouts of the G lanes of this channel
#pragma unroll
  for (int s = 1; s < G; s <<= 1) y += __shfl_xor(y, s, G);
  if (valid) {
    store_stream(sp, f32x4_t{h[0], h[1], h[2], h[3]});
    if (q == 0) {
      y += (a.Dsk ? a.Dsk[d] : 0.0f) * xv;
      if (a.z) y *= silu_f32(zv);
      store_act(a.out + c, y);
    }
  }
}

// Any dstate <= 64: one lane per channel, state row walked element by element.
template <typename TA>
__global__ void __launch_bounds__(256) decode_scalar_kernel(DecArgs<TA> a) {
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (ch >= a.batch * a.dim) return;
  const int64_t b = ch / a.dim;
  const int d = static_cast<int>(ch % a.dim);
  const int N = a.N;
  const float xv = to_f32(a.x[ch]);
  const float raw = to_f32(a.delta[ch]) + (a.bias ? a.bias[d] : 0.0f);
  const float dt = a.softplus ? softplus_f32(raw) : raw;
  const float dx = dt * xv;
  float y = 0.0f;
  float* sp = a.state + ch * N;
  for (int n = 0; n < N; ++n) {
    float unused;
    const float dA = exp_acc(dt * a.A[static_cast<size_t>(d) * N + n], unused);
    const float hn = __builtin_fmaf(dA, sp[n], dx * to_f32(a.B[b * N + n]));
    sp[n] = hn;
    y = __builtin_fmaf(to_f32(a.C[b * N + n]), hn, y);
  }
  y += (a.Dsk ? a.Dsk[d] : 0.0f) * xv;
  if (a.z) y *= silu_f32(to_f32(a.z[ch]));
  store_act(a.out + ch, y);
}

// ----------------------------------------------------------------------------
// host side: validation, dispatch, errors
// ----------------------------------------------------------------------------
thread_local char g_err[512] = "";

void clear_error() { g_err[0] = '\0'; }

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, size_t k) { return (reinterpret_cast<uintptr_t>(p) % k) == 0; }

bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

int launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return SSM_OK;
}

// Waves per carry workgroup: enough in total for a few waves per SIMD, at
// least kCarryUnroll chunk summaries per wave, and at most kCarryRegs where
// kCarryMaxWaves waves allow it.
void launch_carry(const float* A, const CarryChain& c0, const CarryChain& c1, int64_t batch,
                  int dim, int N, int K, hipStream_t s) {
  const int tiles = (dim + 63) / 64;
  const int chains = c1.ws_H ? 2 : 1;
  const int64_t blocks = static_cast<int64_t>(tiles) * chains * N * batch;
  const int64_t target = 4LL * 4 * device_cus();
  int G = static_cast<int>((target + blocks - 1) / blocks);
  const int gmax = (K - 1 + kCarryUnroll - 1) / kCarryUnroll;
  G = G < gmax ? G : gmax;
  // keep each wave's range within its registers where 16 waves allow it
  const int gregs = (K - 1 + kCarryRegs - 1) / kCarryRegs;
  G = G > gregs ? G : gregs;
  G = G < kCarryMaxWaves ? (G > 1 ? G : 1) : kCarryMaxWaves;
  const int per = (K - 1 + G - 1) / G;
  G = (K - 1 + per - 1) / per;
  hipLaunchKernelGGL(fwd_carry_kernel,
                     dim3(static_cast<unsigned>(tiles * chains), static_cast<unsigned>(N),
                          static_cast<unsigned>(batch)),
                     dim3(64 * G), 0, s, A, c0, c1, tiles, dim, N, K, per);
}

void launch_varlen_empty(const int* cu, int nseq, const float* h0, float* last_state, int dim,
                         int N, hipStream_t s) {
  const int64_t per = static_cast<int64_t>(dim) * N;
  const int64_t parts = (per + 255) / 256;
  hipLaunchKernelGGL(fwd_varlen_empty_kernel,
                     dim3(static_cast<unsigned>(nseq), static_cast<unsigned>(parts < 16 ? parts : 16)),
                     dim3(256), 0, s, cu, h0, last_state, dim, N);
}

// Chunking plan.  The sequence is cut into K chunks of Lc tokens (a multiple
// of 2 kGroup), run as Kg = ceil(K / G) groups of G chunks, a workgroup of G
// waves per (channel tile, group, sequence).  Every wave of a launch runs the
// same number of tokens and the kernels are bound by their vector-ALU issue,
// so a launch takes about as long as its busiest compute unit needs for its
// share: ceil(workgroups / CUs) x G waves x (Lc + overhead) token-steps.  The
// overhead counts the group compositions (a scan round or a prologue fold
// each, ~0.3 token-steps) and the aggregate loads a prologue wave waits for
// one after another (~0.3 token-steps each: other groups run meanwhile).
// Splits that leave wave slots empty are charged for the idle share.  Measured on the 130M-, 2.8B-shaped
// and long-context layers (chunk lengths 24-768, groups of 1-8), this picks
// splits within ~1% of the fastest: 32-token chunks for the first,
// 256-token chunks for the others.
constexpr int kMinChunk = 32;
static_assert(kMinChunk % (2 * kGroup) == 0, "chunks are whole pairs of token groups");

struct Plan {
  int K;
  int Lc;
  int G;
};

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = 256;  // MI355X
  }
  return cus;
}

// Register width of the state the forward kernels run for dstate N.
int fwd_width(int64_t N) {
  if (N == 4 || N == 8 || N == 16 || N == 32) return static_cast<int>(N);
  return N < 4 ? 4 : (N < 16 ? 16 : 64);
}

// Waves per SIMD the forward kernels of this width hold (as group_min_waves;
// the wide states from their VGPRs).
int fwd_waves_per_simd(int64_t N) {
  const int nt = fwd_width(N);
  if (nt <= 16) return nt == N ? 6 : 2;
  return nt == 32 ? 4 : 1;
}

// Largest group for this width (as group_max).
int fwd_group_max(int64_t N) {
  const int nt = fwd_width(N);
  return (nt == N && nt <= 32) ? 8 : 4;
}

// Estimated time (token-steps of the busiest compute unit) of a plan.
double plan_cost(int64_t rows, int64_t K, int64_t Lc, int G, int cus, int64_t slots) {
  const int64_t Kg = (K + G - 1) / G;
  const int64_t wgs = rows * Kg;
  int lg = 0;
  while ((1 << lg) < G) ++lg;
  const int64_t folds = Kg - 1 < G ? Kg - 1 : G;
  const double over = K > 1 ? 0.3 * static_cast<double>(folds + lg + 1) +
                                  0.3 * static_cast<double>((Kg - 1 + G - 1) / G)
                            : 0.0;
  const int64_t waves = rows * K;
  const double idle = waves >= slots ? 1.0 : 1.0 + static_cast<double>(slots - waves) / slots;
  return static_cast<double>((wgs + cus - 1) / cus) * G * (static_cast<double>(Lc) + over) * idle;
}

int64_t round_chunk(int64_t Lc) { return (Lc + 2 * kGroup - 1) / (2 * kGroup) * (2 * kGroup); }

// The group size for a given split: 4 or 8 waves once there are 4 chunks
// (smaller groups measured 6-80% slower: their prologues fold many group
// aggregates one after another), the cheaper of the two with ties within 1%
// going to 4; fewer chunks take one group of them all.
Plan plan_groups(int64_t rows, int64_t K, int64_t Lc, int cus, int64_t slots, int gmax,
                 double* cost_out) {
  Plan best{static_cast<int>(K), static_cast<int>(Lc), 1};
  if (K < 4 || gmax < 4) {
    int G = 1;
    while (G * 2 <= K && G * 2 <= gmax) G *= 2;
    best.G = G;
    if (cost_out) *cost_out = plan_cost(rows, K, Lc, G, cus, slots);
    return best;
  }
  best.G = 4;
  double bc = plan_cost(rows, K, Lc, 4, cus, slots);
  if (gmax >= 8 && K >= 8) {
    const double c = plan_cost(rows, K, Lc, 8, cus, slots);
    if (c < bc * 0.99) {
      bc = c;
      best.G = 8;
    }
  }
  if (cost_out) *cost_out = bc;
  return best;
}

Plan plan_fwd(int64_t batch, int64_t L, int64_t dim, int64_t N, bool varlen) {
  (void)varlen;
  Plan p{1, static_cast<int>(L > 0 ? L : 1), 1};
  const int64_t rows = batch * ((dim + 63) / 64);
  const int cus = device_cus();
  const int64_t slots = static_cast<int64_t>(4 * fwd_waves_per_simd(N)) * cus;
  if (L <= 0 || rows >= slots || L < 2 * kMinChunk) return p;
  const int gmax = fwd_group_max(N);
  double bc = plan_cost(rows, 1, L, 1, cus, slots);
  // splits from the one that just fills every wave slot up to four times it
  const int64_t kmax = L / kMinChunk;
  int64_t k0 = (slots + rows - 1) / rows;
  k0 = k0 < kmax ? k0 : kmax;
  int64_t last_lc = -1;
  for (int64_t K = k0 < 2 ? 2 : k0; K <= 4 * k0 && K <= kmax; ++K) {
    const int64_t Lc = round_chunk((L + K - 1) / K);
    if (Lc == last_lc) continue;
    last_lc = Lc;
    const int64_t Kc = (L + Lc - 1) / Lc;
    double c;
    const Plan q = plan_groups(rows, Kc, Lc, cus, slots, gmax, &c);
    if (c < bc * 0.999) {
      bc = c;
      p = q;
    }
  }
  return p;
}

// Plan with the chunk length chosen by the caller: chunk_len rounded up to
// whole pairs of token groups; one chunk (no workspace) when it covers the
// sequence.  K above kMaxChunks is refused by the caller.
constexpr int64_t kMaxChunks = 65535;  // chunks per sequence: one grid dimension
Plan plan_fwd_chunked(int64_t batch, int64_t L, int64_t dim, int64_t N, bool varlen,
                      int64_t chunk_len) {
  (void)varlen;
  Plan p{1, static_cast<int>(L > 0 ? L : 1), 1};
  if (L <= 0 || chunk_len >= L) return p;  // (before rounding: chunk_len may be near INT64_MAX)
  const int64_t Lc = round_chunk(chunk_len);
  if (Lc >= L) return p;
  const int64_t K = (L + Lc - 1) / Lc;
  if (K > kMaxChunks) {
    p.K = static_cast<int>(kMaxChunks + 1);
    return p;
  }
  const int cus = device_cus();
  return plan_groups(batch * ((dim + 63) / 64), K, Lc, cus,
                     static_cast<int64_t>(4 * fwd_waves_per_simd(N)) * cus, fwd_group_max(N),
                     nullptr);
}

// Workspace of the grouped forward, each part 256-byte aligned:
//   E: every chunk's exclusive prefix within its group, S (batch, K, dim),
//      H (batch, K, N, dim), F (batch, K) int;
//   A: every group's aggregate, S (batch, Kg, dim), H (batch, Kg, N, dim),
//      F (batch, Kg) int.
struct WsLayout {
  size_t es, eh, ef, as, ah, af, total;
};

WsLayout workspace_layout(int64_t batch, int64_t dim, int64_t N, const Plan& p) {
  WsLayout w{0, 0, 0, 0, 0, 0, 0};
  if (p.K <= 1) return w;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t K = static_cast<size_t>(p.K), Kg = static_cast<size_t>((p.K + p.G - 1) / p.G);
  const size_t B = static_cast<size_t>(batch), D = static_cast<size_t>(dim), n = static_cast<size_t>(N);
  w.eh = up(B * K * D * 4);
  w.ef = up(w.eh + B * K * n * D * 4);
  w.as = up(w.ef + B * K * 4);
  w.ah = up(w.as + B * Kg * D * 4);
  w.af = up(w.ah + B * Kg * n * D * 4);
  w.total = up(w.af + B * Kg * 4);
  return w;
}

// Dynamic LDS above the default per-launch allowance needs the kernel's
// attribute raised once.
int allow_dynamic_lds(const void* kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return 0;
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(bytes));
  return e == hipSuccess ? 0 : -1;
}

template <typename TA, bool VL>
int dispatch_fwd_vl(const FwdArgs<TA>& a, int64_t batch, bool sp, hipStream_t s) {
  const bool gate = a.z != nullptr;
  switch (a.N) {
    case 16: return launch_fwd_flags<TA, 16, true, VL>(a, batch, sp, gate, s);
    case 8: return launch_fwd_flags<TA, 8, true, VL>(a, batch, sp, gate, s);
    case 4: return launch_fwd_flags<TA, 4, true, VL>(a, batch, sp, gate, s);
    case 32: return launch_fwd_flags<TA, 32, true, VL>(a, batch, sp, gate, s);
    default: break;
  }
  // other state sizes (and 64, whose fully unrolled exact form compiles very
  // slowly) run padded with zero states up to the next supported width
  if (a.N < 4) return launch_fwd_flags<TA, 4, false, VL>(a, batch, sp, gate, s);
  if (a.N < 16) return launch_fwd_flags<TA, 16, false, VL>(a, batch, sp, gate, s);
  return launch_fwd_flags<TA, 64, false, VL>(a, batch, sp, gate, s);
}

template <typename TA>
int dispatch_fwd(const FwdArgs<TA>& a, int64_t batch, bool sp, hipStream_t s) {
  return a.cu ? dispatch_fwd_vl<TA, true>(a, batch, sp, s)
              : dispatch_fwd_vl<TA, false>(a, batch, sp, s);
}

template <typename TA>
int dispatch_decode(const DecArgs<TA>& a, hipStream_t s) {
  const int64_t nch = a.batch * a.dim;
  auto quad = [&](auto kern, int G) {
    const int64_t threads = nch * G;
    const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, a);
    return launch_status("ssm_state_update");
  };
  switch (a.N) {
    case 4: return quad(decode_quad_kernel<TA, 1>, 1);
    case 8: return quad(decode_quad_kernel<TA, 2>, 2);
    case 16: return quad(decode_quad_kernel<TA, 4>, 4);
    case 32: return quad(decode_quad_kernel<TA, 8>, 8);
    case 64: return quad(decode_quad_kernel<TA, 16>, 16);
    default: {
      const unsigned blocks = static_cast<unsigned>((nch + 255) / 256);
      hipLaunchKernelGGL((decode_scalar_kernel<TA>), dim3(blocks), dim3(256), 0, s, a);
      return launch_status("ssm_state_update");
    }
  }
}

constexpr int64_t kMaxDim = (int64_t{1} << 24);   // rows of a token group stay < 4 GiB
constexpr int64_t kMaxLen = (int64_t{1} << 31) - 64;
constexpr int64_t kMaxSeqs = (int64_t{1} << 24) - 1;  // packed sequences per call (x 256 lanes < 2^32)
constexpr int64_t kMaxDecodeLanes = (int64_t{1} << 31) - 256;  // lanes of one decode launch

// Checks and launch shared by both forward entry points.  Dense layout:
// `batch` sequences of `seqlen` tokens, cu == NULL.  Packed layout: one row
// of seqlen = total tokens cut by cu into nseq sequences (batch is 1).
// States are (nstate, dim, dstate) with nstate = batch or nseq.
int fwd_impl(const char* fn, const void* x, const void* delta, const float* delta_bias,
             int delta_softplus, const float* A, const void* B, const void* C,
             const float* D_skip, const void* z, void* out, float* last_state,
             const float* initial_state, const int* cu, int64_t nseq, int64_t batch,
             int64_t seqlen, int64_t dim, int64_t dstate, int dtype, int64_t chunk_len,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const bool varlen = cu != nullptr;
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (delta_softplus != 0 && delta_softplus != 1)
    return fail(SSM_ERR_UNSUPPORTED, "%s: delta_softplus must be 0 or 1, got %d", fn,
                delta_softplus);
  if (batch < 1 || dim < 1 || seqlen < 0)
    return fail(SSM_ERR_SHAPE, "%s: need batch >= 1, dim >= 1, seqlen >= 0 (got %lld, %lld, %lld)",
                fn, (long long)batch, (long long)dim, (long long)seqlen);
  if (varlen && (nseq < 1 || nseq > kMaxSeqs))
    return fail(SSM_ERR_SHAPE, "%s: nseq must be in [1, %lld], got %lld", fn,
                (long long)kMaxSeqs, (long long)nseq);
  if (dstate < 1 || dstate > 64)
    return fail(SSM_ERR_UNSUPPORTED, "%s: dstate must be in [1, 64], got %lld", fn,
                (long long)dstate);
  if (dim > kMaxDim || batch > 65535 || seqlen > kMaxLen)
    return fail(SSM_ERR_SHAPE, "%s: dim %lld, batch %lld or seqlen %lld too large", fn,
                (long long)dim, (long long)batch, (long long)seqlen);
  // a chunk summary's dim x dstate floats are addressed with 32-bit offsets
  if (dim * dstate >= (int64_t{1} << 29))
    return fail(SSM_ERR_SHAPE, "%s: dim x dstate = %lld is 2^29 or more", fn,
                (long long)(dim * dstate));
  if (seqlen > 0 && (!x || !delta || !B || !C || !out))
    return fail(SSM_ERR_NULL, "%s: x, delta, B, C and out are required", fn);
  if (!A) return fail(SSM_ERR_NULL, "%s: A is required", fn);
  const size_t es = dtype == SSM_DTYPE_F32 ? 4 : 2;
  const struct { const void* p; size_t k; const char* n; } al[] = {
      {x, es, "x"}, {delta, es, "delta"}, {z, es, "z"}, {out, es, "out"}, {B, 4, "B"}, {C, 4, "C"},
      {A, 4, "A"}, {D_skip, 4, "D_skip"}, {delta_bias, 4, "delta_bias"},
      {last_state, 16, "last_state"}, {initial_state, 16, "initial_state"}, {cu, 4, "cu_seqlens"}};
  for (const auto& e : al)
    if (e.p && !aligned(e.p, e.k))
      return fail(SSM_ERR_ALIGN, "%s: %s is not %zu-byte aligned", fn, e.n, e.k);
  const int64_t nstate = varlen ? nseq : batch;
  const size_t tok = static_cast<size_t>(batch) * seqlen * dim * es;
  const size_t bc = static_cast<size_t>(batch) * seqlen * dstate * es;
  const size_t st = static_cast<size_t>(nstate) * dim * dstate * 4;
  const Span ins[] = {{x, tok, "x"}, {delta, tok, "delta"}, {z, z ? tok : 0, "z"}, {B, bc, "B"},
                      {C, bc, "C"}, {A, static_cast<size_t>(dim) * dstate * 4, "A"},
                      {D_skip, D_skip ? static_cast<size_t>(dim) * 4 : 0, "D_skip"},
                      {delta_bias, delta_bias ? static_cast<size_t>(dim) * 4 : 0, "delta_bias"},
                      {initial_state, initial_state ? st : 0, "initial_state"},
                      {cu, varlen ? static_cast<size_t>(nseq + 1) * 4 : 0, "cu_seqlens"}};
  const Span outs[] = {{out, tok, "out"}, {last_state, last_state ? st : 0, "last_state"}};
  for (const auto& o : outs)
    for (const auto& i : ins) {
      // dense layout: resume in place (last_state == initial_state) is allowed
      if (!varlen && o.p == last_state && i.p == initial_state && o.p == i.p) continue;
      if (overlap(o, i))
        return fail(SSM_ERR_ALIAS, "%s: output %s overlaps input %s", fn, o.name, i.name);
    }
  if (overlap(outs[0], outs[1])) return fail(SSM_ERR_ALIAS, "%s: out overlaps last_state", fn);
  if (chunk_len < 0)
    return fail(SSM_ERR_SHAPE, "%s: chunk_len must be >= 0, got %lld", fn, (long long)chunk_len);
  const Plan plan = chunk_len > 0 ? plan_fwd_chunked(batch, seqlen, dim, dstate, varlen, chunk_len)
                                  : plan_fwd(batch, seqlen, dim, dstate, varlen);
  if (plan.K > kMaxChunks)
    return fail(SSM_ERR_SHAPE, "%s: chunk_len %lld cuts seqlen %lld into more than %lld chunks", fn,
                (long long)chunk_len, (long long)seqlen, (long long)kMaxChunks);
  const WsLayout wl = workspace_layout(batch, dim, dstate, plan);
  if (workspace_bytes < wl.total || (wl.total > 0 && !workspace))
    return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, wl.total,
                workspace_bytes);
  if (wl.total > 0 && !aligned(workspace, 256))
    return fail(SSM_ERR_ALIGN, "%s: workspace is not 256-byte aligned", fn);
  if (overlap(Span{workspace, wl.total, "workspace"}, outs[0]) ||
      overlap(Span{workspace, wl.total, "workspace"}, outs[1]))
    return fail(SSM_ERR_ALIAS, "%s: workspace overlaps an output", fn);
  for (const auto& i : ins)
    if (overlap(Span{workspace, wl.total, "workspace"}, i))
      return fail(SSM_ERR_ALIAS, "%s: workspace overlaps input %s", fn, i.name);
  if (seqlen == 0 && !last_state) return SSM_OK;
  char* wsb = static_cast<char*>(workspace);
  auto wf = [&](size_t off) { return wl.total ? reinterpret_cast<float*>(wsb + off) : nullptr; };
  auto wi = [&](size_t off) { return wl.total ? reinterpret_cast<int*>(wsb + off) : nullptr; };
  const int nq = static_cast<int>(varlen ? nseq : 0);

  if (dtype == SSM_DTYPE_F32) {
    FwdArgs<float> a{static_cast<const float*>(x), static_cast<const float*>(delta), delta_bias, A,
                     static_cast<const float*>(B), static_cast<const float*>(C), D_skip,
                     static_cast<const float*>(z), static_cast<float*>(out), last_state,
                     initial_state, wf(wl.es), wf(wl.eh), wi(wl.ef), cu, nq,
                     static_cast<int>(seqlen), plan.Lc, plan.K, static_cast<int>(dim),
                     static_cast<int>(dstate), plan.G, wf(wl.as), wf(wl.ah), wi(wl.af)};
    return dispatch_fwd(a, batch, delta_softplus != 0, stream);
  }
  FwdArgs<bf16_t> a{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(delta), delta_bias, A,
                    static_cast<const bf16_t*>(B), static_cast<const bf16_t*>(C), D_skip,
                    static_cast<const bf16_t*>(z), static_cast<bf16_t*>(out), last_state,
                    initial_state, wf(wl.es), wf(wl.eh), wi(wl.ef), cu, nq,
                    static_cast<int>(seqlen), plan.Lc, plan.K, static_cast<int>(dim),
                    static_cast<int>(dstate), plan.G, wf(wl.as), wf(wl.ah), wi(wl.af)};
  return dispatch_fwd(a, batch, delta_softplus != 0, stream);
}

// ----------------------------------------------------------------------------
// library-held scratch for ssm_scan_fwd_noalloc
//
// The forward's chunk summaries live in a file-scope device array instead of
// a caller-provided workspace, for callers that cannot allocate.  Each
// device that runs the call holds its own copy (allocated with the code
// object, kept until the process ends).  In host code `scratch` names a
// host-side stand-in, never the device memory: the device address is taken
// once per device with hipGetSymbolAddress and only that address is passed
// to kernels.
// ----------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t{64} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device), or nullptr with the status in *rc.
void* scratch_on_current_device(int* rc) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = fail(SSM_ERR_HIP, "ssm_scan_fwd_noalloc: no usable current device (%s)",
               e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *rc = fail(SSM_ERR_HIP, "ssm_scan_fwd_noalloc: hipGetSymbolAddress(scratch) failed: %s",
                 hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *rc = SSM_OK;
  return g_scratch_ptr[dev];
}

}  // namespace ssm

using namespace ssm;

extern "C" {

const char* ssm_last_error(void) { return g_err; }

int ssm_abi_version(void) { return SSM_SCAN_ABI_VERSION; }

size_t ssm_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                    int dtype) {
  (void)dtype;
  if (batch < 1 || dim < 1 || seqlen < 0 || dstate < 1 || dstate > 64 || dim > kMaxDim ||
      batch > 65535 || seqlen > kMaxLen)
    return 0;
  return workspace_layout(batch, dim, dstate, plan_fwd(batch, seqlen, dim, dstate, false)).total;
}

size_t ssm_scan_fwd_varlen_workspace_bytes(int64_t nseq, int64_t total_len, int64_t dim,
                                           int64_t dstate, int dtype) {
  (void)dtype;
  if (nseq < 1 || nseq > kMaxSeqs || dim < 1 || total_len < 0 || dstate < 1 || dstate > 64 ||
      dim > kMaxDim || total_len > kMaxLen)
    return 0;
  return workspace_layout(1, dim, dstate, plan_fwd(1, total_len, dim, dstate, true)).total;
}

int ssm_scan_fwd(const void* x, const void* delta, const float* delta_bias, int delta_softplus,
                 const float* A, const void* B, const void* C, const float* D_skip, const void* z,
                 void* out, float* last_state, const float* initial_state, int64_t batch,
                 int64_t seqlen, int64_t dim, int64_t dstate, int dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  return fwd_impl("ssm_scan_fwd", x, delta, delta_bias, delta_softplus, A, B, C, D_skip, z, out,
                  last_state, initial_state, nullptr, 0, batch, seqlen, dim, dstate, dtype, 0,
                  workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_noalloc(const void* x, const void* delta, const float* delta_bias,
                         int delta_softplus, const float* A, const void* B, const void* C,
                         const float* D_skip, const void* z, void* out, float* last_state,
                         const float* initial_state, int64_t batch, int64_t seqlen, int64_t dim,
                         int64_t dstate, int dtype, hipStream_t stream) {
  g_err[0] = '\0';
  const size_t need = ssm_scan_fwd_workspace_bytes(batch, seqlen, dim, dstate, dtype);
  if (need > kScratchBytes)
    return fail(SSM_ERR_WORKSPACE,
                "ssm_scan_fwd_noalloc: these sizes need %zu bytes of scratch, the library holds %zu "
                "(use ssm_scan_fwd with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int rc = SSM_OK;
    ws = scratch_on_current_device(&rc);
    if (!ws) return rc;
  }
  return fwd_impl("ssm_scan_fwd_noalloc", x, delta, delta_bias, delta_softplus, A, B, C, D_skip,
                  z, out, last_state, initial_state, nullptr, 0, batch, seqlen, dim, dstate, dtype,
                  0, ws, ws ? kScratchBytes : 0, stream);
}

size_t ssm_scan_fwd_chunked_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim,
                                            int64_t dstate, int dtype, int64_t chunk_len) {
  if (chunk_len < 0) return 0;
  if (chunk_len == 0) return ssm_scan_fwd_workspace_bytes(batch, seqlen, dim, dstate, dtype);
  if (batch < 1 || dim < 1 || seqlen < 0 || dstate < 1 || dstate > 64 || dim > kMaxDim ||
      batch > 65535 || seqlen > kMaxLen)
    return 0;
  const Plan p = plan_fwd_chunked(batch, seqlen, dim, dstate, false, chunk_len);
  if (p.K > kMaxChunks) return 0;
  return workspace_layout(batch, dim, dstate, p).total;
}

int ssm_scan_fwd_chunked(const void* x, const void* delta, const float* delta_bias,
                         int delta_softplus, const float* A, const void* B, const void* C,
                         const float* D_skip, const void* z, void* out, float* last_state,
                         const float* initial_state, int64_t batch, int64_t seqlen, int64_t dim,
                         int64_t dstate, int dtype, int64_t chunk_len, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  return fwd_impl("ssm_scan_fwd_chunked", x, delta, delta_bias, delta_softplus, A, B, C, D_skip,
                  z, out, last_state, initial_state, nullptr, 0, batch, seqlen, dim, dstate, dtype,
                  chunk_len, workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_varlen(const void* x, const void* delta, const float* delta_bias,
                        int delta_softplus, const float* A, const void* B, const void* C,
                        const float* D_skip, const void* z, void* out, float* last_state,
                        const float* initial_state, const int32_t* cu_seqlens, int64_t nseq,
                        int64_t total_len, int64_t dim, int64_t dstate, int dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  if (!cu_seqlens) return fail(SSM_ERR_NULL, "ssm_scan_fwd_varlen: cu_seqlens is required");
  return fwd_impl("ssm_scan_fwd_varlen", x, delta, delta_bias, delta_softplus, A, B, C, D_skip, z,
                  out, last_state, initial_state, cu_seqlens, nseq, 1, total_len, dim, dstate,
                  dtype, 0, workspace, workspace_bytes, stream);
}

int ssm_state_update(float* state, const void* x, const void* delta, const float* delta_bias,
                     int delta_softplus, const float* A, const void* B, const void* C,
                     const float* D_skip, const void* z, void* out, int64_t batch, int64_t dim,
                     int64_t dstate, int dtype, hipStream_t stream) {
  g_err[0] = '\0';
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "ssm_state_update: unknown dtype %d", dtype);
  if (delta_softplus != 0 && delta_softplus != 1)
    return fail(SSM_ERR_UNSUPPORTED, "ssm_state_update: delta_softplus must be 0 or 1, got %d",
                delta_softplus);
  if (batch < 1 || dim < 1)
    return fail(SSM_ERR_SHAPE, "ssm_state_update: need batch >= 1 and dim >= 1 (got %lld, %lld)",
                (long long)batch, (long long)dim);
  if (dstate < 1 || dstate > 64)
    return fail(SSM_ERR_UNSUPPORTED, "ssm_state_update: dstate must be in [1, 64], got %lld",
                (long long)dstate);
  // one lane per channel (per 4 states when dstate % 4 == 0): the lane count
  // must fit one launch (grid size in work-items below 2^31)
  const int64_t lanes_per_ch = dstate % 4 == 0 ? dstate / 4 : 1;
  if (batch > kMaxDecodeLanes || dim > kMaxDecodeLanes ||
      batch * dim > kMaxDecodeLanes / lanes_per_ch)
    return fail(SSM_ERR_SHAPE,
                "ssm_state_update: batch %lld x dim %lld x %lld lanes per channel exceeds %lld lanes",
                (long long)batch, (long long)dim, (long long)lanes_per_ch,
                (long long)kMaxDecodeLanes);
  if (!state || !x || !delta || !A || !B || !C || !out)
    return fail(SSM_ERR_NULL, "ssm_state_update: state, x, delta, A, B, C and out are required");
  const size_t es = dtype == SSM_DTYPE_F32 ? 4 : 2;
  const struct { const void* p; size_t k; const char* n; } al[] = {
      {x, es, "x"}, {delta, es, "delta"}, {z, es, "z"}, {out, es, "out"}, {B, es, "B"},
      {C, es, "C"}, {A, 4, "A"}, {D_skip, 4, "D_skip"}, {delta_bias, 4, "delta_bias"},
      {state, 16, "state"}};
  for (const auto& e : al)
    if (e.p && !aligned(e.p, e.k))
      return fail(SSM_ERR_ALIGN, "ssm_state_update: %s is not %zu-byte aligned", e.n, e.k);
  if (dstate % 4 == 0 && (!aligned(A, 16) || !aligned(B, 4 * es) || !aligned(C, 4 * es)))
    return fail(SSM_ERR_ALIGN,
                "ssm_state_update: with dstate %% 4 == 0, A must be 16-byte aligned and B, C aligned "
                "to 4 elements");
  const size_t tok = static_cast<size_t>(batch) * dim * es;
  const size_t bc = static_cast<size_t>(batch) * dstate * es;
  const size_t st = static_cast<size_t>(batch) * dim * dstate * 4;
  const Span ins[] = {{x, tok, "x"}, {delta, tok, "delta"}, {z, z ? tok : 0, "z"}, {B, bc, "B"},
                      {C, bc, "C"}, {A, static_cast<size_t>(dim) * dstate * 4, "A"},
                      {D_skip, D_skip ? static_cast<size_t>(dim) * 4 : 0, "D_skip"},
                      {delta_bias, delta_bias ? static_cast<size_t>(dim) * 4 : 0, "delta_bias"}};
  const Span outs[] = {{out, tok, "out"}, {state, st, "state"}};
  for (const auto& o : outs)
    for (const auto& i : ins)
      if (overlap(o, i))
        return fail(SSM_ERR_ALIAS, "ssm_state_update: %s overlaps input %s", o.name, i.name);
  if (overlap(outs[0], outs[1])) return fail(SSM_ERR_ALIAS, "ssm_state_update: out overlaps state");

  if (dtype == SSM_DTYPE_F32) {
    DecArgs<float> a{state, static_cast<const float*>(x), static_cast<const float*>(delta),
                     delta_bias, A, static_cast<const float*>(B), static_cast<const float*>(C),
                     D_skip, static_cast<const float*>(z), static_cast<float*>(out), batch,
                     static_cast<int>(dim), static_cast<int>(dstate), delta_softplus};
    return dispatch_decode(a, stream);
  }
  DecArgs<bf16_t> a{state, static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(delta),
                    delta_bias, A, static_cast<const bf16_t*>(B), static_cast<const bf16_t*>(C),
                    D_skip, static_cast<const bf16_t*>(z), static_cast<bf16_t*>(out), batch,
                    static_cast<int>(dim), static_cast<int>(dstate), delta_softplus};
  return dispatch_decode(a, stream);
}

}  // extern "C"
