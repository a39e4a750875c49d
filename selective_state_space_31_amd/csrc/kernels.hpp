// kernels.hpp -- device code of the forward scan (templates), shared by the
// translation units that instantiate it for each activation type and state
// width.  Host entry points and the remaining kernels are in ssm_scan.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace ssm {

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
// Cache-policy operand of the buffer stores of per-token outputs: the
// nontemporal bit (written once, never read back by the kernel that writes
// them; ~1.5% on the forward).
constexpr int kStoreStream = 2;

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
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, kStoreStream);
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
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, b), r, voff, soff, kStoreStream);
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
// forward
//
// Time is cut into K chunks of Lc tokens so that every workload offers the
// chip enough independent lanes (a lane = one channel over one chunk).  The
// affine maps h -> a*h + b of consecutive tokens compose associatively
// (a1,b1) then (a2,b2) = (a2*a1, a2*b1 + b2), so a chunk is summarised by
// its total decay exp(A[n] * sum Delta) and the state it reaches from zero;
// three launches then finish the scan:
//   agg   : per chunk 0..K-2, sum Delta and the local end state from h = 0;
//   carry : per (sequence, channel, state), fold the chunk summaries in
//           order, leaving the exact state entering every chunk;
//   scan  : per chunk, the recurrence from its entering state, with the
//           readout, skip, gate and store fused in.
// With K = 1 only the scan runs.
//
// Packed variable-length sequences (cu != NULL) run as one long sequence of
// L = total tokens; the offsets cu[0..nseq] cut it into sequences, and at
// each sequence start the state is set to that sequence's initial state
// (or zero) instead of being carried.  A chunk that holds a start then has
// the summary "forget the incoming state, end at H", which the carry pass
// applies through the per-chunk flag F.
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
  float* ws_S;  // (batch, K-1, dim): sum of Delta over chunk c
  float* ws_H;  // (batch, K, N, dim): slot c+1 first holds chunk c's end state from
                // zero (or from its last sequence start); after the carry pass slot c
                // holds the state entering chunk c
  int* ws_F;    // (K-1), packed sequences only: 1 if chunk c holds a sequence start
  const int* cu;  // packed sequences: nseq+1 token offsets; NULL for (batch, L) layout
  int nseq;
  int L;
  int Lc;
  int K;
  int dim;
  int N;
};

constexpr int kGroup = 4;  // tokens per group; the next group's loads are in flight
constexpr uint32_t kOutOfRange = 0x80000000u;  // > any descriptor's byte range (those are < 2^31)

// Per-lane channel constants.  The exponents A[d,n]*log2(e) of the general
// path live in LDS, not in registers: that path is bound by its N
// transcendentals per token, so reading them back costs little, while
// holding N more values per lane would cut the resident waves of the whole
// kernel (the power path needs only A[d,0]).  Table layout: float4 q of
// lane l at [q][l], so each per-token read is one contiguous 1 KiB row.
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int NT>
__device__ __forceinline__ f32x4* a2_table() {
  __shared__ f32x4 tab[NT / 4 * 64];
  return tab;
}

template <int NT>
struct Chan {
  float A2_0;    // A[d,0] * log2(e)
  float A0;      // A[d,0]
  float bias, dsk;
  int d0;        // first channel of the wave
  uint32_t voff_ld, voff_st;
  bool valid;
  bool pow;      // every lane of the wave has A[d,n] == (n+1) A[d,0]
};

template <typename TA, int NT, bool EXACT>
__device__ __forceinline__ Chan<NT> load_chan(const FwdArgs<TA>& a, int d0) {
  Chan<NT> c;
  const int lane = threadIdx.x;
  const int d = d0 + lane;
  const int N = a.N;
  c.d0 = d0;
  c.valid = d < a.dim;
  const int dl = c.valid ? d : a.dim - 1;  // masked lanes compute on a valid channel
  static_assert(NT % 4 == 0, "state widths are padded to multiples of 4");
  bool pow_ok = true;
  c.A0 = a.A[static_cast<size_t>(dl) * N];
  c.A2_0 = c.A0 * kLog2e;
  f32x4* tab = a2_table<NT>();
#pragma unroll
  for (int q = 0; q < NT / 4; ++q) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = 4 * q + j;
      const float an = (EXACT || n < N) ? a.A[static_cast<size_t>(dl) * N + n] : 0.0f;
      v[j] = an * kLog2e;
      if (EXACT || n < N) pow_ok = pow_ok && (an == static_cast<float>(n + 1) * c.A0);
    }
    tab[q * 64 + lane] = f32x4{v[0], v[1], v[2], v[3]};
  }
  c.pow = __all(pow_ok);
  c.bias = a.bias ? a.bias[dl] : 0.0f;
  c.dsk = a.Dsk ? a.Dsk[dl] : 0.0f;
  c.voff_ld = static_cast<uint32_t>(dl - d0) * Io<TA>::es;
  // Lanes past the last channel store to an offset beyond every descriptor's
  // range: raw buffer stores out of range are dropped by the hardware, so the
  // store needs no branch (which would split the unrolled token group).
  c.voff_st = c.valid ? static_cast<uint32_t>(lane) * Io<TA>::es : kOutOfRange;
  return c;
}

// One token: discretise, update the N states, read out, gate.  Returns the
// output value (before rounding to the activation type).
//   POW : the channel's A is (n+1)*A[0], decays are powers of r = e^(Delta*A[0]).
//   ACC : float32 activations; r is formed to ~0.5 ulp as a two-float hi + lo
//         and every power is taken against both parts, so r's own rounding is
//         not amplified (n+1)-fold in r^(n+1).  With bf16 activations the
//         output rounding (2^-9) dwarfs these errors and the single-float
//         chain on the hardware exp is used.
//   AGG : summary pass: no readout, the step size is summed into S instead.
// The step is split in three so that the B_t/C_t rows can be supplied either
// whole (already in SGPRs) or in blocks of 16 states (wide states).
struct StepScalars {
  float dt, dx, y, rh, rl, p;
};

template <int NT, bool SP, bool POW, bool ACC, bool AGG>
__device__ __forceinline__ StepScalars step_begin(const Chan<NT>& ch, float xv, float draw,
                                                  float& S) {
  StepScalars s;
  const float raw = draw + ch.bias;
  s.dt = SP ? softplus_f32(raw) : raw;
  s.dx = s.dt * xv;
  s.y = ch.dsk * xv;
  if constexpr (AGG) S += s.dt;
  s.rh = s.rl = s.p = 0.0f;
  if constexpr (POW && ACC) {
    s.rh = exp_acc(s.dt * ch.A0, s.rl);
    s.p = s.rh;
  } else if constexpr (POW) {
    s.rh = __builtin_amdgcn_exp2f(s.dt * ch.A2_0);
    s.p = s.rh;
  }
  return s;
}

// States n0 .. n0+NB-1 given their B_t and C_t values.
template <int NT, int NB, bool POW, bool ACC, bool AGG>
__device__ __forceinline__ void step_block(float (&h)[NT], const Chan<NT>& ch, StepScalars& s,
                                           int n0, const float (&Bv)[NB], const float (&Cv)[NB]) {
  static_assert(NB % 4 == 0, "");
  if constexpr (POW) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + j;
      const float dA = s.p;
      if constexpr (ACC) {
        if (n + 1 < NT) s.p = __builtin_fmaf(s.p, s.rh, s.p * s.rl);
      } else {
        s.p *= s.rh;
      }
      fma_inplace(h[n], dA, s.dx * Bv[j]);
      if constexpr (!AGG) s.y = __builtin_fmaf(Cv[j], h[n], s.y);
    }
  } else {
    // Four states at a time, exponents read from the LDS table (volatile:
    // read per token, never hoisted out of the token loop); the scheduling
    // barrier keeps the compiler from lifting all N exponentials ahead of
    // their uses, which would hold N more values per lane.
    const volatile f32x4* tab = a2_table<NT>();
#pragma unroll
    for (int q = 0; q < NB / 4; ++q) {
      const f32x4 v = tab[(n0 / 4 + q) * 64 + threadIdx.x];
      const float a2[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + 4 * q + j;
        const float dA = __builtin_amdgcn_exp2f(s.dt * a2[j]);
        fma_inplace(h[n], dA, s.dx * Bv[4 * q + j]);
        if constexpr (!AGG) s.y = __builtin_fmaf(Cv[4 * q + j], h[n], s.y);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <bool GATE, bool AGG>
__device__ __forceinline__ float step_end(const StepScalars& s, float zv) {
  float y = s.y;
  if constexpr (GATE && !AGG) y *= silu_f32(zv);
  return y;
}

// Wide or padded states: rows read in blocks of up to 16 inside the step.
template <typename TA, int NT, bool EXACT, bool SP, bool GATE, bool POW, bool ACC, bool AGG>
__device__ __forceinline__ float token_step(float (&h)[NT], const Chan<NT>& ch, const TA* Brow,
                                            const TA* Crow, int N, float xv, float draw, float zv,
                                            float& S) {
  constexpr int NB = NT < 16 ? NT : 16;
  StepScalars s = step_begin<NT, SP, POW, ACC, AGG>(ch, xv, draw, S);
#pragma unroll
  for (int n0 = 0; n0 < NT; n0 += NB) {
    float Bv[NB], Cv[NB];
    load_row<NB, EXACT>(Brow + n0, N - n0, Bv);
    if constexpr (!AGG) load_row<NB, EXACT>(Crow + n0, N - n0, Cv);
    step_block<NT, NB, POW, ACC, AGG>(h, ch, s, n0, Bv, Cv);
  }
  return step_end<GATE, AGG>(s, zv);
}

// Raw words of one token's B and C rows (whole rows of NT <= 16 states),
// loaded by scalar loads one token ahead of their use.
template <typename TA, int NT>
struct RowsRaw {
  static constexpr int W = static_cast<int>(sizeof(TA)) * NT / 4;  // dwords per row
  uint32_t b[W], c[W];
};

template <typename TA, int NT, bool AGG>
__device__ __forceinline__ void rows_load(RowsRaw<TA, NT>& r, const TA* Brow, const TA* Crow) {
  cu32_t* qb = (cu32_t*)Brow;
  cu32_t* qc = (cu32_t*)Crow;
#pragma unroll
  for (int i = 0; i < RowsRaw<TA, NT>::W; ++i) {
    r.b[i] = qb[i];
    if constexpr (!AGG) r.c[i] = qc[i];
  }
}

template <int NT>
__device__ __forceinline__ void rows_unpack(const uint32_t* w, float (&v)[NT], float) {
#pragma unroll
  for (int n = 0; n < NT; ++n) v[n] = __uint_as_float(w[n]);
}
template <int NT>
__device__ __forceinline__ void rows_unpack(const uint32_t* w, float (&v)[NT], bf16_t) {
#pragma unroll
  for (int i = 0; i < NT / 2; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Tokens [t_begin, t_begin + len) of sequence b for the wave's 64 channels.
// AGG: summary pass (S, h); otherwise the output pass.
template <typename TA, int NT, bool EXACT, bool SP, bool GATE, bool POW, bool AGG>
__device__ __forceinline__ void run_tokens(const FwdArgs<TA>& a, const Chan<NT>& ch, int b,
                                           int t_begin, int len, float (&h)[NT], float& S) {
  using IO = Io<TA>;
  using raw_t = typename IO::raw_t;
  constexpr bool Z = GATE && !AGG;
  const int dim = a.dim, N = a.N;
  const size_t rowblk = static_cast<size_t>(b) * static_cast<size_t>(a.L) + t_begin;
  const uint32_t rowbytes = static_cast<uint32_t>(dim) * IO::es;
  const uint32_t span = kGroup * rowbytes;
  const TA* B = a.B + rowblk * N;
  const TA* C = a.C + rowblk * N;
  const int d0 = ch.d0;
  const uint32_t voff_ld = ch.voff_ld, voff_st = ch.voff_st;

  // x/delta/z of kGroup tokens starting at t0 (token indices clamped to the
  // range, so reads past its end repeat the last row and are unused)
  auto fetch = [&](int t0, raw_t(&xs)[kGroup], raw_t(&ds)[kGroup], raw_t(&zs)[kGroup]) {
    const int tb = t0 < len ? t0 : len - 1;
    const size_t base = (rowblk + tb) * dim + d0;
    const rsrc_t rx = make_rsrc(a.x + base, span), rd = make_rsrc(a.delta + base, span);
    const rsrc_t rz = make_rsrc(Z ? a.z + base : a.x + base, span);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int t = (tb + u < len) ? tb + u : len - 1;
      const uint32_t so = static_cast<uint32_t>(t - tb) * rowbytes;
      xs[u] = IO::load(rx, voff_ld, so);
      ds[u] = IO::load(rd, voff_ld, so);
      if constexpr (Z) zs[u] = IO::load(rz, voff_ld, so);
    }
  };
  // Rows of B_t/C_t run one token ahead in SGPRs (whole-row state widths):
  // the wait for token t's rows is followed by the loads for token t+1, and
  // scheduling barriers keep the compiler from hoisting a whole group's loads
  // (which would overflow the scalar registers into vector lanes).
  constexpr bool PF = EXACT && NT <= 16 && (sizeof(TA) * NT) % 4 == 0;
  RowsRaw<TA, NT> nxt;
  if constexpr (PF) rows_load<TA, NT, AGG>(nxt, B, C);
  auto one = [&](int t, float xv, float draw, float zv) -> float {
    if constexpr (PF) {
      float Bv[NT], Cv[NT];
      rows_unpack<NT>(nxt.b, Bv, TA{});
      if constexpr (!AGG) rows_unpack<NT>(nxt.c, Cv, TA{});
      __builtin_amdgcn_sched_barrier(0);
      const size_t rn = static_cast<size_t>(t + 1 < len ? t + 1 : len - 1) * N;
      rows_load<TA, NT, AGG>(nxt, B + rn, C + rn);
      __builtin_amdgcn_sched_barrier(0);
      StepScalars st = step_begin<NT, SP, POW, IO::es == 4, AGG>(ch, xv, draw, S);
      step_block<NT, NT, POW, IO::es == 4, AGG>(h, ch, st, 0, Bv, Cv);
      return step_end<GATE, AGG>(st, zv);
    } else {
      const size_t row = static_cast<size_t>(t) * N;
      return token_step<TA, NT, EXACT, SP, GATE, POW, IO::es == 4, AGG>(h, ch, B + row, C + row, N,
                                                                       xv, draw, zv, S);
    }
  };
  // kGroup tokens starting at t0, all inside the range
  auto compute = [&](int t0, const raw_t(&xs)[kGroup], const raw_t(&ds)[kGroup],
                     const raw_t(&zs)[kGroup]) {
    const size_t obase = (rowblk + t0) * dim + d0;
    const rsrc_t ro = make_rsrc(a.out + (AGG ? 0 : obase), span);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const float y = one(t0 + u, IO::f32(xs[u]), IO::f32(ds[u]), Z ? IO::f32(zs[u]) : 0.0f);
      if constexpr (!AGG) IO::store(y, ro, voff_st, static_cast<uint32_t>(u) * rowbytes);
    }
  };

  // Main part: pairs of full groups, ping-ponging two register buffers so the
  // loads of the next group are in flight while the current one computes,
  // and no per-token branch splits the unrolled recurrence.  Wide states
  // (N > 16) and the general path (bound by its N exponentials per token,
  // where the buffers would only add register pressure) take the compact
  // token-at-a-time loop below for all tokens.
  int t_tail = 0;
  if constexpr (NT <= 16 && POW) {
    const int npair = len / (2 * kGroup);
    raw_t xa[kGroup], da[kGroup], za[kGroup], xb2[kGroup], db2[kGroup], zb2[kGroup];
    fetch(0, xa, da, za);
    for (int i = 0; i < npair; ++i) {
      const int t0 = i * 2 * kGroup;
      fetch(t0 + kGroup, xb2, db2, zb2);
      compute(t0, xa, da, za);
      fetch(t0 + 2 * kGroup, xa, da, za);
      compute(t0 + kGroup, xb2, db2, zb2);
    }
    t_tail = npair * 2 * kGroup;
  }
  // Tail: the remaining tokens one at a time.
  for (int t = t_tail; t < len; ++t) {
    const size_t base = (rowblk + t) * dim + d0;
    const rsrc_t rx = make_rsrc(a.x + base, rowbytes), rd = make_rsrc(a.delta + base, rowbytes);
    float zv = 0.0f;
    if constexpr (Z) zv = IO::f32(IO::load(make_rsrc(a.z + base, rowbytes), voff_ld, 0));
    const float y = one(t, IO::f32(IO::load(rx, voff_ld, 0)), IO::f32(IO::load(rd, voff_ld, 0)), zv);
    if constexpr (!AGG) IO::store(y, make_rsrc(a.out + base, rowbytes), voff_st, 0);
  }
}

// Summary of a full chunk by reverse accumulation (power-structured A,
// single-float chain): the state the chunk reaches from zero is
//   H[n] = sum_t (prod_{s>t} r_s)^(n+1) * dx_t * B_t[n],
// so walking the tokens from last to first with Q = prod_{s>t} r_s, the weight
// w_n = dx_t * Q^(n+1) follows the chain w_n = w_(n-1) * Q and each state costs
// one multiply plus one FMA whose addend operand B_t[n] is a scalar register
// (the forward recurrence needs a third operation, dx * B, per state).
template <typename TA, int NT, bool SP>
__device__ __forceinline__ void agg_reverse(const FwdArgs<TA>& a, const Chan<NT>& ch, int b,
                                            int t_begin, int len, float (&H)[NT], float& S) {
  using IO = Io<TA>;
  using raw_t = typename IO::raw_t;
  const int dim = a.dim, N = a.N;
  const size_t rowblk = static_cast<size_t>(b) * static_cast<size_t>(a.L) + t_begin;
  const uint32_t rowbytes = static_cast<uint32_t>(dim) * IO::es;
  const uint32_t span = kGroup * rowbytes;
  const TA* B = a.B + rowblk * N;
  const uint32_t voff_ld = ch.voff_ld;
  float Q = 1.0f;
  // x/delta of the kGroup tokens starting at t0 (t0 >= 0, all inside the chunk)
  auto fetch = [&](int t0, raw_t(&xs)[kGroup], raw_t(&ds)[kGroup]) {
    const size_t base = (rowblk + t0) * dim + ch.d0;
    const rsrc_t rx = make_rsrc(a.x + base, span), rd = make_rsrc(a.delta + base, span);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      xs[u] = IO::load(rx, voff_ld, static_cast<uint32_t>(u) * rowbytes);
      ds[u] = IO::load(rd, voff_ld, static_cast<uint32_t>(u) * rowbytes);
    }
  };
  RowsRaw<TA, NT> nxt;
  rows_load<TA, NT, true>(nxt, B + static_cast<size_t>(len - 1) * N, B);
  auto one = [&](int t, float xv, float draw) {
    float Bv[NT];
    rows_unpack<NT>(nxt.b, Bv, TA{});
    __builtin_amdgcn_sched_barrier(0);
    const size_t rn = static_cast<size_t>(t > 0 ? t - 1 : 0) * N;
    rows_load<TA, NT, true>(nxt, B + rn, B);
    __builtin_amdgcn_sched_barrier(0);
    const float raw = draw + ch.bias;
    const float dt = SP ? softplus_f32(raw) : raw;
    S += dt;
    const float r = __builtin_amdgcn_exp2f(dt * ch.A2_0);
    float w = dt * xv * Q;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      H[n] = __builtin_fmaf(w, Bv[n], H[n]);
      w *= Q;
    }
    Q *= r;
  };
  // len is a multiple of 2*kGroup: walk pairs of groups from the end,
  // ping-ponging two register buffers
  raw_t xa[kGroup], da[kGroup], xb2[kGroup], db2[kGroup];
  const int npair = len / (2 * kGroup);
  fetch(len - kGroup, xa, da);
  for (int i = npair - 1; i >= 0; --i) {
    const int t0 = i * 2 * kGroup;  // this pair covers [t0, t0 + 2 kGroup)
    fetch(t0, xb2, db2);
#pragma unroll
    for (int u = kGroup - 1; u >= 0; --u) one(t0 + kGroup + u, IO::f32(xa[u]), IO::f32(da[u]));
    fetch(t0 >= 2 * kGroup ? t0 - kGroup : t0, xa, da);
#pragma unroll
    for (int u = kGroup - 1; u >= 0; --u) one(t0 + u, IO::f32(xb2[u]), IO::f32(db2[u]));
  }
}

// Packed sequences: the sequence that token t belongs to, the largest s in
// [0, nseq) with cu[s] <= t (sequence s is tokens [cu[s], cu[s+1])), found by
// a 64-way search: the wave's lanes probe 64 offsets at once, so nseq <= 64
// takes one round of loads and each further factor of 64 one more.  Every
// probe stays inside cu[0, nseq), so offsets that are not sorted still give
// an index in range.  t is wave-uniform and all 64 lanes must be active.
__device__ __forceinline__ int seq_owner(const int* cu, int nseq, int t) {
  const int lane = static_cast<int>(threadIdx.x & 63);
  int lo = 0, cnt = nseq;
  for (;;) {
    const int stride = (cnt + 63) >> 6;
    const int i = lane * stride;
    const bool p = i < cnt && cu[lo + i] <= t;
    const unsigned long long m = __ballot(p);
    const int k = m ? 63 - __builtin_clzll(m) : 0;
    lo = __builtin_amdgcn_readfirstlane(lo + k * stride);
    if (stride == 1) return lo;
    cnt = (cnt - k * stride < stride) ? cnt - k * stride : stride;
  }
}

// Lane's initial state of sequence s (zeros without one).
template <int NT, bool EXACT>
__device__ __forceinline__ void load_h0(const float* h0, int s, int dim, int dl, int N,
                                        float (&h)[NT]) {
  const float* hp = h0 ? h0 + (static_cast<size_t>(s) * dim + dl) * N : nullptr;
#pragma unroll
  for (int n = 0; n < NT; ++n) h[n] = (hp && (EXACT || n < N)) ? hp[n] : 0.0f;
}

// Summary pass: block (channel tile, chunk c < K-1, sequence b).  With
// packed sequences, a chunk in which a sequence starts is summarised from
// its last start: the state there is that sequence's initial state, and
// the chunk's end state no longer depends on the state entering it.
template <typename TA, int NT, bool EXACT, bool SP, bool VL>
__global__ void __launch_bounds__(64) fwd_agg_kernel(FwdArgs<TA> a) {
  const int d0 = blockIdx.x * 64;
  const int c = blockIdx.y;
  const int b = blockIdx.z;
  const Chan<NT> ch = load_chan<TA, NT, EXACT>(a, d0);
  const int dl = ch.valid ? d0 + static_cast<int>(threadIdx.x) : a.dim - 1;
  float h[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) h[n] = 0.0f;
  float S = 0.0f;
  const int t_begin = c * a.Lc;  // chunks before the last are full (Lc is a multiple of 2*kGroup)
  bool reset = false;
  if constexpr (VL) {
    const int t_end = t_begin + a.Lc;
    const int s = seq_owner(a.cu, a.nseq, t_end - 1);
    const int st = a.cu[s];
    if (st >= t_begin && st < t_end) {
      reset = true;
      load_h0<NT, EXACT>(a.h0, s, a.dim, dl, a.N, h);
      if (ch.pow)
        run_tokens<TA, NT, EXACT, SP, false, true, true>(a, ch, b, st, t_end - st, h, S);
      else
        run_tokens<TA, NT, EXACT, SP, false, false, true>(a, ch, b, st, t_end - st, h, S);
    }
  }
  if (!reset) {
    constexpr bool REV = EXACT && NT <= 16 && sizeof(TA) == 2 && (sizeof(TA) * NT) % 4 == 0;
    if (ch.pow) {
      if constexpr (REV)
        agg_reverse<TA, NT, SP>(a, ch, b, t_begin, a.Lc, h, S);
      else
        run_tokens<TA, NT, EXACT, SP, false, true, true>(a, ch, b, t_begin, a.Lc, h, S);
    } else
      run_tokens<TA, NT, EXACT, SP, false, false, true>(a, ch, b, t_begin, a.Lc, h, S);
  }
  if (ch.valid) {
    const int d = d0 + threadIdx.x;
    a.ws_S[(static_cast<size_t>(b) * (a.K - 1) + c) * a.dim + d] = S;
    const size_t slot = static_cast<size_t>(b) * a.K + c + 1;
#pragma unroll
    for (int n = 0; n < NT; ++n)
      if (EXACT || n < a.N) a.ws_H[(slot * a.N + n) * a.dim + d] = h[n];
  }
  if (VL && blockIdx.x == 0 && threadIdx.x == 0) a.ws_F[c] = reset ? 1 : 0;
}

// Output pass: block (channel tile, chunk c, sequence b).  With packed
// sequences the chunk is walked segment by segment (the parts of it that
// belong to one sequence): the state is reset at each sequence start and
// stored to last_state at each sequence end.
template <typename TA, int NT, bool EXACT, bool SP, bool GATE, bool VL>
__global__ void __launch_bounds__(64) fwd_scan_kernel(FwdArgs<TA> a) {
  const int d0 = blockIdx.x * 64;
  const int c = blockIdx.y;
  const int b = blockIdx.z;
  const Chan<NT> ch = load_chan<TA, NT, EXACT>(a, d0);
  const int N = a.N;
  const int d = d0 + threadIdx.x;
  const int dl = ch.valid ? d : a.dim - 1;
  float h[NT];
  if (a.K > 1) {
    // state entering the chunk, left by the carry pass (also for c = 0, so
    // that this pass never reads initial_state, which may be last_state)
    const size_t slot = static_cast<size_t>(b) * a.K + c;
#pragma unroll
    for (int n = 0; n < NT; ++n)
      h[n] = (EXACT || n < N) ? a.ws_H[(slot * N + n) * a.dim + dl] : 0.0f;
  } else {
    load_h0<NT, EXACT>(VL ? nullptr : a.h0, b, a.dim, dl, N, h);
  }
  const int t_begin = c * a.Lc;
  const int len = (a.L - t_begin < a.Lc) ? a.L - t_begin : a.Lc;
  float S = 0.0f;
  if constexpr (!VL) {
    if (len > 0) {  // an empty sequence only carries the initial state through
      if (ch.pow)
        run_tokens<TA, NT, EXACT, SP, GATE, true, false>(a, ch, b, t_begin, len, h, S);
      else
        run_tokens<TA, NT, EXACT, SP, GATE, false, false>(a, ch, b, t_begin, len, h, S);
    }
    if (a.last_state && ch.valid && c == a.K - 1) {
      float* lp = a.last_state + (static_cast<size_t>(b) * a.dim + d) * N;
#pragma unroll
      for (int n = 0; n < NT; ++n)
        if (EXACT || n < N) lp[n] = h[n];
    }
  } else {
    // last_state of sequence s (lanes of valid channels)
    auto store_last = [&](int s, const float (&v)[NT]) {
      if (a.last_state && ch.valid) {
        float* lp = a.last_state + (static_cast<size_t>(s) * a.dim + d) * N;
#pragma unroll
        for (int n = 0; n < NT; ++n)
          if (EXACT || n < N) lp[n] = v[n];
      }
    };
    // empty sequences s, s+1, ... placed at token offset `at`: their last
    // state is their initial state
    auto store_empty_from = [&](int s, int at) {
      if (!a.last_state) return;
      for (; s < a.nseq && a.cu[s] == at && a.cu[s + 1] == at; ++s) {
        float e0[NT];
        load_h0<NT, EXACT>(a.h0, s, a.dim, dl, N, e0);
        store_last(s, e0);
      }
    };
    const int t_end = t_begin + (len > 0 ? len : 0);
    int t = t_begin;
    if (c == 0) store_empty_from(0, 0);  // empty sequences before the first token
    while (t < t_end) {
      const int s = seq_owner(a.cu, a.nseq, t);
      const int st = a.cu[s], en = a.cu[s + 1];
      int e = en < t_end ? en : t_end;
      if (e <= t) e = t + 1;  // (offsets not sorted: still move on)
      if (st == t) load_h0<NT, EXACT>(a.h0, s, a.dim, dl, N, h);
      if (ch.pow)
        run_tokens<TA, NT, EXACT, SP, GATE, true, false>(a, ch, 0, t, e - t, h, S);
      else
        run_tokens<TA, NT, EXACT, SP, GATE, false, false>(a, ch, 0, t, e - t, h, S);
      if (e == en) {
        store_last(s, h);
        store_empty_from(s + 1, en);  // empty sequences right after this one
      }
      t = e;
    }
  }
}

// ----------------------------------------------------------------------------
// launchers (host side of the templates above)
// ----------------------------------------------------------------------------
int launch_status(const char* what);
void launch_carry(const float* A, const float* h0, const float* ws_S, float* ws_H,
                  const int* ws_F, int64_t batch, int dim, int N, int K, hipStream_t s);
void launch_varlen_empty(const int* cu, int nseq, const float* h0, float* last_state, int dim,
                         int N, hipStream_t s);

template <typename TA, int NT, bool EXACT, bool SP, bool GATE, bool VL>
int launch_fwd(const FwdArgs<TA>& a, int64_t batch, hipStream_t s) {
  const unsigned tiles = static_cast<unsigned>((a.dim + 63) / 64);
  if (a.K > 1) {
    hipLaunchKernelGGL((fwd_agg_kernel<TA, NT, EXACT, SP, VL>),
                       dim3(tiles, static_cast<unsigned>(a.K - 1), static_cast<unsigned>(batch)),
                       dim3(64), 0, s, a);
    launch_carry(a.A, VL ? nullptr : a.h0, a.ws_S, a.ws_H, VL ? a.ws_F : nullptr, batch, a.dim,
                 a.N, a.K, s);
  }
  if (!VL || a.L > 0)
    hipLaunchKernelGGL((fwd_scan_kernel<TA, NT, EXACT, SP, GATE, VL>),
                       dim3(tiles, static_cast<unsigned>(a.K), static_cast<unsigned>(batch)),
                       dim3(64), 0, s, a);
  // no tokens at all: every packed sequence's last_state is its initial state
  // (otherwise the output pass stores those of the empty ones)
  if (VL && a.L == 0 && a.last_state)
    launch_varlen_empty(a.cu, a.nseq, a.h0, a.last_state, a.dim, a.N, s);
  return launch_status(VL ? "ssm_scan_fwd_varlen" : "ssm_scan_fwd");
}

// The state entering every chunk (summary and carry passes only; ws_H slot
// c holds it for c >= 1 afterwards), for the backward's recomputation.
template <typename TA, int NT, bool EXACT>
int launch_fwd_states(const FwdArgs<TA>& a, int64_t batch, bool sp, hipStream_t s) {
  if (a.K <= 1) return launch_status("ssm_scan_bwd");
  const dim3 grid(static_cast<unsigned>((a.dim + 63) / 64), static_cast<unsigned>(a.K - 1),
                  static_cast<unsigned>(batch));
  if (sp)
    hipLaunchKernelGGL((fwd_agg_kernel<TA, NT, EXACT, true, false>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_agg_kernel<TA, NT, EXACT, false, false>), grid, dim3(64), 0, s, a);
  launch_carry(a.A, a.h0, a.ws_S, a.ws_H, nullptr, batch, a.dim, a.N, a.K, s);
  return launch_status("ssm_scan_bwd");
}

template <typename TA, int NT, bool EXACT, bool VL>
int launch_fwd_flags(const FwdArgs<TA>& a, int64_t batch, bool sp, bool gate, hipStream_t s) {
  if (sp)
    return gate ? launch_fwd<TA, NT, EXACT, true, true, VL>(a, batch, s)
                : launch_fwd<TA, NT, EXACT, true, false, VL>(a, batch, s);
  return gate ? launch_fwd<TA, NT, EXACT, false, true, VL>(a, batch, s)
              : launch_fwd<TA, NT, EXACT, false, false, VL>(a, batch, s);
}

}  // namespace ssm
