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

#include "ssm_scan.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ----------------------------------------------------------------------------
// element access
// ----------------------------------------------------------------------------
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v.bits) << 16);
}
__device__ __forceinline__ void store_act(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_act(bf16_t* p, float v) {
  // round to nearest even (gfx950 converts natively)
  __bf16 b = static_cast<__bf16>(v);
  p->bits = __builtin_bit_cast(uint16_t, b);
}

// Buffer-resource access to the per-token activation rows.  The descriptor
// base is wave-uniform (a token row start, kept in SGPRs), the lane's column
// is a constant VGPR byte offset, and the token within a group is a scalar
// offset: no per-access vector address arithmetic.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) 32-bit access, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

template <typename TA>
struct Io;
template <>
struct Io<float> {
  using raw_t = uint32_t;
  static constexpr int es = 4;
  __device__ static raw_t load(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  }
  __device__ static float f32(raw_t v) { return __uint_as_float(v); }
  __device__ static void store(float v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
  }
};
template <>
struct Io<bf16_t> {
  using raw_t = uint16_t;
  static constexpr int es = 2;
  __device__ static raw_t load(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  }
  __device__ static float f32(raw_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
  __device__ static void store(float v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __bf16 b = static_cast<__bf16>(v);  // round to nearest even
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, b), r, voff, soff, 0);
  }
};

// B_t / C_t rows are read through the constant address space: the address is
// wave-uniform, so these become scalar loads into SGPRs.
typedef const __attribute__((address_space(4))) float cfloat_t;
typedef const __attribute__((address_space(4))) uint32_t cu32_t;
typedef const __attribute__((address_space(4))) uint16_t cu16_t;

// Row of NT values of B_t or C_t, widened to f32; with EXACT (dstate == NT)
// whole dwords are read, otherwise elements up to N with zeros after.
template <int NT, bool EXACT>
__device__ __forceinline__ void load_row(const float* p, int N, float (&v)[NT]) {
  cfloat_t* q = (cfloat_t*)p;
#pragma unroll
  for (int n = 0; n < NT; ++n) v[n] = (EXACT || n < N) ? q[n] : 0.0f;
}
template <int NT, bool EXACT>
__device__ __forceinline__ void load_row(const bf16_t* p, int N, float (&v)[NT]) {
  if constexpr (EXACT && (NT % 2 == 0)) {
    cu32_t* w = (cu32_t*)p;
#pragma unroll
    for (int i = 0; i < NT / 2; ++i) {
      const uint32_t u = w[i];
      v[2 * i] = __uint_as_float(u << 16);
      v[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
    }
  } else {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
    for (int n = 0; n < NT; ++n)
      v[n] = (EXACT || n < N) ? __uint_as_float(static_cast<uint32_t>(q[n]) << 16) : 0.0f;
  }
}

// ----------------------------------------------------------------------------
// scalar functions of the step
// ----------------------------------------------------------------------------
// softplus(u) = log(1 + e^u) in float32, accurate to a few ulp relative:
//   u > 15      : u (the dropped log1p(e^-u) < 3.1e-7 is below u's half-ulp)
//   e^u < 1/16  : log1p(e) by its series to e^5 (relative error < e^5/6)
//   otherwise   : log2(1 + e) * ln 2 (1 + e >= 1.0625 keeps cancellation small)
__device__ __forceinline__ float softplus_f32(float u) {
  const float e = __builtin_amdgcn_exp2f(u * kLog2e);
  const float lg = __builtin_amdgcn_logf(1.0f + e) * kLn2;
  const float p =
      e * __builtin_fmaf(e, __builtin_fmaf(e, __builtin_fmaf(e, __builtin_fmaf(e, 0.2f, -0.25f),
                                                               0.33333334f),
                                             -0.5f),
                         1.0f);
  const float r = e < 0.0625f ? p : lg;
  return u > 15.0f ? u : r;
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z); e^-z = inf gives 0 * z = -0.
__device__ __forceinline__ float silu_f32(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// e^x for float32 x, returned as hi + lo with hi = e^x rounded to nearest
// (error ~0.5 ulp, no bias) and lo the part of e^x that hi drops.
// The hardware exp2 is within an ulp but rounds low on average (about
// -0.05 ulp); a decay factor applied a thousand times over a long memory
// turns that bias into a relative drift of ~3e-6 in the state, so the paths
// whose float32 results must track a float64 reference over long horizons
// use this instead.  Method: x = k ln2 + f with |f| <= ln2/2 (Cody-Waite, ln2
// split in two), e^f = 1 + f q(f) with q the Taylor series of (e^f - 1)/f to
// f^6 (truncation < 6e-9 relative), result scaled by 2^k.
constexpr float kLn2Hi = 0.693145751953125f;        // 11 leading bits of ln 2
constexpr float kLn2Lo = 1.428606765330187e-06f;    // ln 2 - kLn2Hi
__device__ __forceinline__ float exp_acc(float x, float& lo) {
  x = __builtin_fmaxf(x, -104.0f);  // e^-104 is below the smallest float32
  const float k = __builtin_rintf(x * kLog2e);
  float f = __builtin_fmaf(-k, kLn2Hi, x);
  f = __builtin_fmaf(-k, kLn2Lo, f);
  float q = __builtin_fmaf(f, 1.0f / 5040.0f, 1.0f / 720.0f);
  q = __builtin_fmaf(f, q, 1.0f / 120.0f);
  q = __builtin_fmaf(f, q, 1.0f / 24.0f);
  q = __builtin_fmaf(f, q, 1.0f / 6.0f);
  q = __builtin_fmaf(f, q, 0.5f);
  q = __builtin_fmaf(f, q, 1.0f);
  const float hi = __builtin_fmaf(f, q, 1.0f);
  const float l = __builtin_fmaf(f, q, 1.0f - hi);  // 1 - hi is exact (hi in [0.7, 1.5])
  const int ki = static_cast<int>(k);
  lo = __builtin_ldexpf(l, ki);
  return __builtin_ldexpf(hi, ki);
}

// h = a*h + b with the result in h's own register.  Written out so the
// compiler does not pick the accumulate form (whose accumulator is b) and
// then copy h back every step.
__device__ __forceinline__ void fma_inplace(float& h, float a, float b) {
  h = __builtin_fmaf(a, h, b);
}

// ----------------------------------------------------------------------------
// forward: one lane per channel, sequential over the whole sequence
// ----------------------------------------------------------------------------
template <typename TA>
struct FwdArgs {
  const TA* x;
  const TA* delta;
  const float* bias;
  const float* A;
  const TA* B;
  const TA* C;
  const float* Dsk;
  const TA* z;
  TA* out;
  float* last_state;
  const float* h0;
  int64_t L;
  int dim;
  int N;
};

constexpr int kGroup = 4;  // tokens per group; the next group's loads are in flight

// One token: discretise, update the N states, read out, gate.  Returns the
// output value (before rounding to the activation type).
//   POW : the channel's A is (n+1)*A[0], decays are powers of r = e^(Delta*A[0]).
//   ACC : float32 activations; r is formed to ~0.5 ulp as a two-float hi + lo
//         and every power is taken against both parts, so r's own rounding is
//         not amplified (n+1)-fold in r^(n+1).  With bf16 activations the
//         output rounding (2^-9) dwarfs these errors and the single-float
//         chain on the hardware exp is used.
template <int NT, bool SP, bool GATE, bool POW, bool ACC>
__device__ __forceinline__ float token_step(float (&h)[NT], const float (&A2)[NT], float A0,
                                            const float (&Bv)[NT], const float (&Cv)[NT],
                                            float xv, float draw, float zv, float bias, float dsk) {
  const float raw = draw + bias;
  const float dt = SP ? softplus_f32(raw) : raw;
  const float dx = dt * xv;
  float y = dsk * xv;
  if constexpr (POW && ACC) {
    float rl;
    const float rh = exp_acc(dt * A0, rl);
    float p = rh;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      fma_inplace(h[n], p, dx * Bv[n]);
      y = __builtin_fmaf(Cv[n], h[n], y);
      if (n + 1 < NT) p = __builtin_fmaf(p, rh, p * rl);
    }
  } else if constexpr (POW) {
    const float r = __builtin_amdgcn_exp2f(dt * A2[0]);
    float p = r;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      fma_inplace(h[n], p, dx * Bv[n]);
      y = __builtin_fmaf(Cv[n], h[n], y);
      p *= r;
    }
  } else {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float dA = __builtin_amdgcn_exp2f(dt * A2[n]);
      fma_inplace(h[n], dA, dx * Bv[n]);
      y = __builtin_fmaf(Cv[n], h[n], y);
    }
  }
  if constexpr (GATE) y *= silu_f32(zv);
  return y;
}

template <typename TA, int NT, bool EXACT, bool SP, bool GATE, bool POW>
__device__ __forceinline__ void fwd_seq_body(const FwdArgs<TA>& a, int b, int d0, uint32_t voff_ld,
                                             uint32_t voff_st, bool valid, const float (&A2)[NT],
                                             float A0, float bias, float dsk, float (&h)[NT]) {
  using IO = Io<TA>;
  using raw_t = typename IO::raw_t;
  const int dim = a.dim, N = a.N;
  const int L = static_cast<int>(a.L);  // < 2^31, checked on the host
  const size_t rowblk = static_cast<size_t>(b) * static_cast<size_t>(L);
  const uint32_t rowbytes = static_cast<uint32_t>(dim) * IO::es;
  // bytes a group's descriptor may touch: kGroup rows (offsets are clamped
  // to the last row and to the last valid column before use)
  const uint32_t span = kGroup * rowbytes;
  const TA* B = a.B + rowblk * N;
  const TA* C = a.C + rowblk * N;

  // x/delta/z of kGroup tokens starting at t0 (token indices clamped to the
  // sequence, so reads past the end repeat the last row and are unused)
  auto fetch = [&](int t0, raw_t(&xs)[kGroup], raw_t(&ds)[kGroup], raw_t(&zs)[kGroup]) {
    const int tb = t0 < L ? t0 : L - 1;
    const size_t base = (rowblk + tb) * dim + d0;
    const rsrc_t rx = make_rsrc(a.x + base, span), rd = make_rsrc(a.delta + base, span);
    const rsrc_t rz = make_rsrc(GATE ? a.z + base : a.x + base, span);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int t = (tb + u < L) ? tb + u : L - 1;
      const uint32_t so = static_cast<uint32_t>(t - tb) * rowbytes;
      xs[u] = IO::load(rx, voff_ld, so);
      ds[u] = IO::load(rd, voff_ld, so);
      if constexpr (GATE) zs[u] = IO::load(rz, voff_ld, so);
    }
  };
  // kGroup tokens starting at t0, all inside the sequence
  auto compute = [&](int t0, const raw_t(&xs)[kGroup], const raw_t(&ds)[kGroup],
                     const raw_t(&zs)[kGroup]) {
    const size_t obase = (rowblk + t0) * dim + d0;
    const rsrc_t ro = make_rsrc(a.out + obase, span);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      float Bv[NT], Cv[NT];
      load_row<NT, EXACT>(B + static_cast<size_t>(t0 + u) * N, N, Bv);
      load_row<NT, EXACT>(C + static_cast<size_t>(t0 + u) * N, N, Cv);
      const float y = token_step<NT, SP, GATE, POW, IO::es == 4>(
          h, A2, A0, Bv, Cv, IO::f32(xs[u]), IO::f32(ds[u]), GATE ? IO::f32(zs[u]) : 0.0f, bias,
          dsk);
      if (valid) IO::store(y, ro, voff_st, static_cast<uint32_t>(u) * rowbytes);
    }
  };

  // Main part: pairs of full groups, ping-ponging two register buffers so the
  // loads of the next group are in flight while the current one computes,
  // and no per-token branch splits the unrolled recurrence.
  const int npair = L / (2 * kGroup);
  raw_t xa[kGroup], da[kGroup], za[kGroup], xb2[kGroup], db2[kGroup], zb2[kGroup];
  fetch(0, xa, da, za);
  for (int i = 0; i < npair; ++i) {
    const int t0 = i * 2 * kGroup;
    fetch(t0 + kGroup, xb2, db2, zb2);
    compute(t0, xa, da, za);
    fetch(t0 + 2 * kGroup, xa, da, za);
    compute(t0 + kGroup, xb2, db2, zb2);
  }
  // Tail: the last L mod 2*kGroup tokens one at a time.
  for (int t = npair * 2 * kGroup; t < L; ++t) {
    const size_t base = (rowblk + t) * dim + d0;
    const rsrc_t rx = make_rsrc(a.x + base, rowbytes), rd = make_rsrc(a.delta + base, rowbytes);
    const rsrc_t ro = make_rsrc(a.out + base, rowbytes);
    float Bv[NT], Cv[NT];
    load_row<NT, EXACT>(B + static_cast<size_t>(t) * N, N, Bv);
    load_row<NT, EXACT>(C + static_cast<size_t>(t) * N, N, Cv);
    float zv = 0.0f;
    if constexpr (GATE) zv = IO::f32(IO::load(make_rsrc(a.z + base, rowbytes), voff_ld, 0));
    const float y = token_step<NT, SP, GATE, POW, IO::es == 4>(
        h, A2, A0, Bv, Cv, IO::f32(IO::load(rx, voff_ld, 0)), IO::f32(IO::load(rd, voff_ld, 0)), zv,
        bias, dsk);
    if (valid) IO::store(y, ro, voff_st, 0);
  }
}

template <typename TA, int NT, bool EXACT, bool SP, bool GATE>
__global__ void __launch_bounds__(64) fwd_seq_kernel(FwdArgs<TA> a) {
  const int lane = threadIdx.x;
  const int d0 = blockIdx.x * 64;
  const int b = blockIdx.y;
  const int d = d0 + lane;
  const bool valid = d < a.dim;
  const int dl = valid ? d : a.dim - 1;  // masked lanes compute on a valid channel
  const int N = a.N;

  float A2[NT], h[NT];
  bool pow_ok = true;
  const float a0 = a.A[static_cast<size_t>(dl) * N];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float an = (EXACT || n < N) ? a.A[static_cast<size_t>(dl) * N + n] : 0.0f;
    A2[n] = an * kLog2e;
    if (EXACT || n < N) pow_ok = pow_ok && (an == static_cast<float>(n + 1) * a0);
    h[n] = 0.0f;
  }
  if (a.h0) {
    const float* hp = a.h0 + (static_cast<size_t>(b) * a.dim + dl) * N;
#pragma unroll
    for (int n = 0; n < NT; ++n)
      if (EXACT || n < N) h[n] = hp[n];
  }
  const float bias = a.bias ? a.bias[dl] : 0.0f;
  const float dsk = a.Dsk ? a.Dsk[dl] : 0.0f;
  const uint32_t es = Io<TA>::es;
  const uint32_t voff_ld = static_cast<uint32_t>(dl - d0) * es;
  const uint32_t voff_st = static_cast<uint32_t>(lane) * es;

  if (a.L > 0) {  // an empty sequence only carries the initial state through
    if (__all(pow_ok))
      fwd_seq_body<TA, NT, EXACT, SP, GATE, true>(a, b, d0, voff_ld, voff_st, valid, A2, a0, bias,
                                                  dsk, h);
    else
      fwd_seq_body<TA, NT, EXACT, SP, GATE, false>(a, b, d0, voff_ld, voff_st, valid, A2, a0, bias,
                                                   dsk, h);
  }

  if (a.last_state && valid) {
    float* lp = a.last_state + (static_cast<size_t>(b) * a.dim + d) * N;
#pragma unroll
    for (int n = 0; n < NT; ++n)
      if (EXACT || n < N) lp[n] = h[n];
  }
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

// G lanes per channel, 4 consecutive states per lane (N = 4G): each wave
// reads and writes one contiguous 1 KiB stretch of the state per instruction.
template <typename TA, int G>
__global__ void __launch_bounds__(256) decode_vec_kernel(DecArgs<TA> a) {
  constexpr int N = 4 * G;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nch = a.batch * a.dim;
  const int64_t ch = gid / G;
  const int q = static_cast<int>(gid % G);
  const bool valid = ch < nch;
  const int64_t c = valid ? ch : nch - 1;
  const int64_t b = c / a.dim;
  const int d = static_cast<int>(c % a.dim);

  float4* sp = reinterpret_cast<float4*>(a.state + c * N) + q;
  const float4 hv = *sp;
  const float4 Av = reinterpret_cast<const float4*>(a.A + static_cast<size_t>(d) * N)[q];
  float Bv[4], Cv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Bv[i] = to_f32(a.B[b * N + 4 * q + i]);
    Cv[i] = to_f32(a.C[b * N + 4 * q + i]);
  }
  const float xv = to_f32(a.x[c]);
  const float raw = to_f32(a.delta[c]) + (a.bias ? a.bias[d] : 0.0f);
  const float dt = a.softplus ? softplus_f32(raw) : raw;
  const float dx = dt * xv;
  float h[4] = {hv.x, hv.y, hv.z, hv.w};
  const float Aa[4] = {Av.x, Av.y, Av.z, Av.w};
  float y = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float unused;
    const float dA = exp_acc(dt * Aa[i], unused);  // HBM-bound: the accurate exp is free here
    h[i] = __builtin_fmaf(dA, h[i], dx * Bv[i]);
    y = __builtin_fmaf(Cv[i], h[i], y);
  }
  // sum the partial readouts of the G lanes of this channel
#pragma unroll
  for (int s = 1; s < G; s <<= 1) y += __shfl_xor(y, s, G);
  if (valid) {
    *sp = make_float4(h[0], h[1], h[2], h[3]);
    if (q == 0) {
      y += (a.Dsk ? a.Dsk[d] : 0.0f) * xv;
      if (a.z) y *= silu_f32(to_f32(a.z[c]));
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

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, size_t k) { return (reinterpret_cast<uintptr_t>(p) % k) == 0; }

struct Span {
  const void* p;
  size_t bytes;
  const char* name;
};

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

template <typename TA, int NT, bool EXACT, bool SP, bool GATE>
int launch_fwd(const FwdArgs<TA>& a, int64_t batch, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.dim + 63) / 64), static_cast<unsigned>(batch));
  hipLaunchKernelGGL((fwd_seq_kernel<TA, NT, EXACT, SP, GATE>), grid, dim3(64), 0, s, a);
  return launch_status("ssm_scan_fwd");
}

template <typename TA, int NT, bool EXACT>
int launch_fwd_flags(const FwdArgs<TA>& a, int64_t batch, bool sp, bool gate, hipStream_t s) {
  if (sp)
    return gate ? launch_fwd<TA, NT, EXACT, true, true>(a, batch, s)
                : launch_fwd<TA, NT, EXACT, true, false>(a, batch, s);
  return gate ? launch_fwd<TA, NT, EXACT, false, true>(a, batch, s)
              : launch_fwd<TA, NT, EXACT, false, false>(a, batch, s);
}

template <typename TA>
int dispatch_fwd(const FwdArgs<TA>& a, int64_t batch, bool sp, hipStream_t s) {
  const bool gate = a.z != nullptr;
  switch (a.N) {
    case 16: return launch_fwd_flags<TA, 16, true>(a, batch, sp, gate, s);
    case 8: return launch_fwd_flags<TA, 8, true>(a, batch, sp, gate, s);
    case 4: return launch_fwd_flags<TA, 4, true>(a, batch, sp, gate, s);
    case 32: return launch_fwd_flags<TA, 32, true>(a, batch, sp, gate, s);
    case 64: return launch_fwd_flags<TA, 64, true>(a, batch, sp, gate, s);
    default: break;
  }
  // other state sizes run padded with zero states up to the next supported width
  if (a.N < 4) return launch_fwd_flags<TA, 4, false>(a, batch, sp, gate, s);
  if (a.N < 16) return launch_fwd_flags<TA, 16, false>(a, batch, sp, gate, s);
  return launch_fwd_flags<TA, 64, false>(a, batch, sp, gate, s);
}

template <typename TA>
int dispatch_decode(const DecArgs<TA>& a, hipStream_t s) {
  const int64_t nch = a.batch * a.dim;
  auto vec = [&](auto kern, int G) {
    const int64_t threads = nch * G;
    const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, a);
    return launch_status("ssm_state_update");
  };
  switch (a.N) {
    case 4: return vec(decode_vec_kernel<TA, 1>, 1);
    case 8: return vec(decode_vec_kernel<TA, 2>, 2);
    case 16: return vec(decode_vec_kernel<TA, 4>, 4);
    case 32: return vec(decode_vec_kernel<TA, 8>, 8);
    case 64: return vec(decode_vec_kernel<TA, 16>, 16);
    default: {
      const unsigned blocks = static_cast<unsigned>((nch + 255) / 256);
      hipLaunchKernelGGL((decode_scalar_kernel<TA>), dim3(blocks), dim3(256), 0, s, a);
      return launch_status("ssm_state_update");
    }
  }
}

constexpr int64_t kMaxDim = (int64_t{1} << 24);   // rows of a token group stay < 4 GiB
constexpr int64_t kMaxLen = (int64_t{1} << 31) - 64;

}  // namespace

extern "C" {

const char* ssm_last_error(void) { return g_err; }

int ssm_abi_version(void) { return SSM_SCAN_ABI_VERSION; }

size_t ssm_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                    int dtype) {
  (void)batch; (void)seqlen; (void)dim; (void)dstate; (void)dtype;
  return 0;
}

int ssm_scan_fwd(const void* x, const void* delta, const float* delta_bias, int delta_softplus,
                 const float* A, const void* B, const void* C, const float* D_skip, const void* z,
                 void* out, float* last_state, const float* initial_state, int64_t batch,
                 int64_t seqlen, int64_t dim, int64_t dstate, int dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "ssm_scan_fwd: unknown dtype %d", dtype);
  if (delta_softplus != 0 && delta_softplus != 1)
    return fail(SSM_ERR_UNSUPPORTED, "ssm_scan_fwd: delta_softplus must be 0 or 1, got %d",
                delta_softplus);
  if (batch < 1 || dim < 1 || seqlen < 0)
    return fail(SSM_ERR_SHAPE, "ssm_scan_fwd: need batch >= 1, dim >= 1, seqlen >= 0 (got %lld, %lld, %lld)",
                (long long)batch, (long long)dim, (long long)seqlen);
  if (dstate < 1 || dstate > 64)
    return fail(SSM_ERR_UNSUPPORTED, "ssm_scan_fwd: dstate must be in [1, 64], got %lld",
                (long long)dstate);
  if (dim > kMaxDim || batch > 65535 || seqlen > kMaxLen)
    return fail(SSM_ERR_SHAPE, "ssm_scan_fwd: dim %lld, batch %lld or seqlen %lld too large",
                (long long)dim, (long long)batch, (long long)seqlen);
  if (seqlen > 0 && (!x || !delta || !B || !C || !out))
    return fail(SSM_ERR_NULL, "ssm_scan_fwd: x, delta, B, C and out are required");
  if (!A) return fail(SSM_ERR_NULL, "ssm_scan_fwd: A is required");
  const size_t es = dtype == SSM_DTYPE_F32 ? 4 : 2;
  const struct { const void* p; size_t k; const char* n; } al[] = {
      {x, es, "x"}, {delta, es, "delta"}, {z, es, "z"}, {out, es, "out"}, {B, 4, "B"}, {C, 4, "C"},
      {A, 4, "A"}, {D_skip, 4, "D_skip"}, {delta_bias, 4, "delta_bias"},
      {last_state, 16, "last_state"}, {initial_state, 16, "initial_state"}};
  for (const auto& e : al)
    if (e.p && !aligned(e.p, e.k))
      return fail(SSM_ERR_ALIGN, "ssm_scan_fwd: %s is not %zu-byte aligned", e.n, e.k);
  const size_t tok = static_cast<size_t>(batch) * seqlen * dim * es;
  const size_t bc = static_cast<size_t>(batch) * seqlen * dstate * es;
  const size_t st = static_cast<size_t>(batch) * dim * dstate * 4;
  const Span ins[] = {{x, tok, "x"}, {delta, tok, "delta"}, {z, z ? tok : 0, "z"}, {B, bc, "B"},
                      {C, bc, "C"}, {A, static_cast<size_t>(dim) * dstate * 4, "A"},
                      {D_skip, D_skip ? static_cast<size_t>(dim) * 4 : 0, "D_skip"},
                      {delta_bias, delta_bias ? static_cast<size_t>(dim) * 4 : 0, "delta_bias"},
                      {initial_state, initial_state ? st : 0, "initial_state"}};
  const Span outs[] = {{out, tok, "out"}, {last_state, last_state ? st : 0, "last_state"}};
  for (const auto& o : outs)
    for (const auto& i : ins) {
      if (o.p == last_state && i.p == initial_state && o.p == i.p) continue;  // resume in place
      if (overlap(o, i))
        return fail(SSM_ERR_ALIAS, "ssm_scan_fwd: output %s overlaps input %s", o.name, i.name);
    }
  if (overlap(outs[0], outs[1]))
    return fail(SSM_ERR_ALIAS, "ssm_scan_fwd: out overlaps last_state");
  const size_t need = ssm_scan_fwd_workspace_bytes(batch, seqlen, dim, dstate, dtype);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(SSM_ERR_WORKSPACE, "ssm_scan_fwd: workspace of %zu bytes needed, %zu given", need,
                workspace_bytes);
  if (seqlen == 0 && !last_state) return SSM_OK;

  if (dtype == SSM_DTYPE_F32) {
    FwdArgs<float> a{static_cast<const float*>(x), static_cast<const float*>(delta), delta_bias, A,
                     static_cast<const float*>(B), static_cast<const float*>(C), D_skip,
                     static_cast<const float*>(z), static_cast<float*>(out), last_state,
                     initial_state, seqlen, static_cast<int>(dim), static_cast<int>(dstate)};
    return dispatch_fwd(a, batch, delta_softplus != 0, stream);
  }
  FwdArgs<bf16_t> a{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(delta), delta_bias, A,
                    static_cast<const bf16_t*>(B), static_cast<const bf16_t*>(C), D_skip,
                    static_cast<const bf16_t*>(z), static_cast<bf16_t*>(out), last_state,
                    initial_state, seqlen, static_cast<int>(dim), static_cast<int>(dstate)};
  return dispatch_fwd(a, batch, delta_softplus != 0, stream);
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
  if (batch * dim * 16 > (int64_t{1} << 40))
    return fail(SSM_ERR_SHAPE, "ssm_state_update: batch*dim too large");
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
  if (dstate % 4 == 0 && !aligned(A, 16))
    return fail(SSM_ERR_ALIGN, "ssm_state_update: A must be 16-byte aligned when dstate %% 4 == 0");
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
