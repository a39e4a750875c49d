// conv1d.hip -- the short causal depthwise convolution (+ SiLU) that feeds
// the scan, and its one-token decoding update, for MI355X (gfx950), behind
// the C ABI in include/ssm_scan.h (see there for the citation).
//
//   out[b,t,d] = silu( bias[d] + sum_{k<W} w[d,k] * xx[b, t-(W-1)+k, d] )
//
// where xx is x extended to the left by the conv state (the W-1 inputs
// before the first token; zeros without one).  The operation moves each
// activation once in and once out and does W multiply-adds per value: it is
// bound by HBM bandwidth, so the kernels are laid out for wide coalesced
// accesses rather than arithmetic:
//   * a lane owns V consecutive channels (2 bf16 or 4 float32: 4- or 16-byte
//     accesses; for bf16 the narrower vector measured faster than 8, as it
//     gives more waves for the same bytes) and a stretch of kConvTokens
//     tokens; a wave covers 64*V channels of one token per access;
//   * the lane loads the W-1 inputs before its stretch itself (from x or the
//     conv state), so stretches are independent and the launch has enough
//     waves for the whole chip at any sequence length;
//   * all loads of a stretch are issued before the first use (fully unrolled)
//     so that many accesses per wave are in flight.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_scan.h"

#include "host_util.hpp"
#include "kernels.hpp"

namespace ssm {

constexpr int kConvTokens = 16;  // tokens per lane in the forward
constexpr int kConvVecBf16 = 2;  // bf16 channels per lane and access

template <typename TA>
struct ConvArgs {
  const TA* x;
  const float* w;
  const float* bias;
  const TA* state0;  // (batch, dim, W-1) or NULL
  TA* out;
  TA* state1;        // (batch, dim, W-1) or NULL
  int64_t batch;
  int64_t L;
  int dim;
  int tiles;   // channel tiles of 64*V
  int64_t chunks;  // token stretches per sequence
};

// V activations moved as one 16-byte access (V > 1) or one element: the raw
// bits are kept (fewer registers for a window of them) and widened at use.
// Output rows are written once and not read again here, so the vector stores
// carry the nontemporal hint (130M-shaped forward: 17.8 -> 14.1 us).  The
// input loads do not: neighbouring stretches re-read 3 rows through L2.
typedef float f32x4_e __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_e __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_e __attribute__((ext_vector_type(2)));
template <typename TA, int V>
struct VecIo;
template <>
struct VecIo<float, 4> {
  using raw_t = float4;
  __device__ static raw_t load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static float get(const raw_t& r, int v) {
    return v == 0 ? r.x : v == 1 ? r.y : v == 2 ? r.z : r.w;
  }
  __device__ static raw_t from(const float (&v)[4]) { return make_float4(v[0], v[1], v[2], v[3]); }
  __device__ static void store(float* p, const float (&v)[4]) {
    __builtin_nontemporal_store(f32x4_e{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4_e*>(p));
  }
};
// bf16: V = 2, 4 or 8 values in one 4-, 8- or 16-byte access.
template <int V>
struct VecBf16 {
  static constexpr int NW = V / 2;  // 32-bit words
  struct raw_t {
    uint32_t w[NW];
  };
  __device__ static raw_t load(const bf16_t* p) {
    raw_t r;
    if constexpr (NW == 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(p);
      r.w[0] = q.x; r.w[1] = q.y; r.w[2] = q.z; r.w[3] = q.w;
    } else if constexpr (NW == 2) {
      const uint2 q = *reinterpret_cast<const uint2*>(p);
      r.w[0] = q.x; r.w[1] = q.y;
    } else {
      r.w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
    return r;
  }
  __device__ static float get(const raw_t& r, int v) {
    const uint32_t w = r.w[v >> 1];
    return __uint_as_float((v & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ static uint32_t bits(float f) {
    __bf16 b = static_cast<__bf16>(f);  // round to nearest even (exact for bf16 values)
    return __builtin_bit_cast(uint16_t, b);
  }
  __device__ static raw_t from(const float (&v)[V]) {
    raw_t r;
#pragma unroll
    for (int i = 0; i < NW; ++i) r.w[i] = bits(v[2 * i]) | (bits(v[2 * i + 1]) << 16);
    return r;
  }
  __device__ static void store(bf16_t* p, const float (&v)[V]) {
    const raw_t r = from(v);
    if constexpr (NW == 4) {
      __builtin_nontemporal_store(u32x4_e{r.w[0], r.w[1], r.w[2], r.w[3]},
                                  reinterpret_cast<u32x4_e*>(p));
    } else if constexpr (NW == 2) {
      __builtin_nontemporal_store(u32x2_e{r.w[0], r.w[1]}, reinterpret_cast<u32x2_e*>(p));
    } else {
      __builtin_nontemporal_store(r.w[0], reinterpret_cast<uint32_t*>(p));
    }
  }
};
template <>
struct VecIo<bf16_t, 8> : VecBf16<8> {};
template <>
struct VecIo<bf16_t, 4> : VecBf16<4> {};
template <>
struct VecIo<bf16_t, 2> : VecBf16<2> {};

template <typename TA>
struct VecIo1 {
  using raw_t = float;
  __device__ static raw_t load(const TA* p) { return to_f32(*p); }
  __device__ static float get(const raw_t& r, int) { return r; }
  __device__ static raw_t from(const float (&v)[1]) { return v[0]; }
  __device__ static void store(TA* p, const float (&v)[1]) { store_act(p, v[0]); }
};
template <>
struct VecIo<float, 1> : VecIo1<float> {};
template <>
struct VecIo<bf16_t, 1> : VecIo1<bf16_t> {};

// Input at token s (s may be negative: the conv state) of channel c.
template <typename TA, int W>
__device__ __forceinline__ float conv_input(const ConvArgs<TA>& a, int64_t b, int64_t s, int c) {
  if (s >= 0) return to_f32(a.x[(b * a.L + s) * a.dim + c]);
  return a.state0 ? to_f32(a.state0[(b * a.dim + c) * (W - 1) + (W - 1) + s]) : 0.0f;
}

// Block = one wave: a unit (channel tile, token stretch, sequence), tiles
// fastest.  Workgroups are dealt to the 8 XCDs in turn (block i to XCD i mod
// 8), each with its own L2; the units are handed out so that every XCD
// works through one contiguous range of them, so the W-1 rows a stretch
// shares with the one before it are found in that XCD's L2.
constexpr int kXcds = 8;
template <typename TA, int W, int V, bool SILU>
__global__ void __launch_bounds__(64) conv_fwd_kernel(ConvArgs<TA> a) {
  constexpr int T = kConvTokens;
  const int64_t per_xcd = gridDim.x / kXcds;  // the grid is a multiple of kXcds
  const int64_t blk = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (blk >= static_cast<int64_t>(a.tiles) * a.chunks * a.batch) return;
  const int tile = static_cast<int>(blk % a.tiles);
  const int64_t rest = blk / a.tiles;
  const int64_t t0 = (rest % a.chunks) * T;
  const int64_t b = rest / a.chunks;
  const int c0 = (tile * 64 + static_cast<int>(threadIdx.x)) * V;
  if (c0 >= a.dim) return;  // (no barriers below)
  const int64_t L = a.L;

  // inputs t0-(W-1) .. t0+T-1 (raw), all loads issued up front.  Interior
  // stretches (every row inside the sequence; the common case, uniform per
  // wave) load without a branch per row, so the loads are in flight together.
  using IO = VecIo<TA, V>;
  typename IO::raw_t win[T + W - 1];
  const TA* xrow = a.x + (b * L + t0 - (W - 1)) * a.dim + c0;
  if (t0 >= W - 1 && t0 + T <= L) {
#pragma unroll
    for (int r = 0; r < T + W - 1; ++r) win[r] = IO::load(xrow + static_cast<int64_t>(r) * a.dim);
  } else {
#pragma unroll
    for (int r = 0; r < T + W - 1; ++r) {
      const int64_t t = t0 - (W - 1) + r;
      if (t >= 0 && t < L) {
        win[r] = IO::load(a.x + (b * L + t) * a.dim + c0);
      } else {
        float v0[V];
#pragma unroll
        for (int v = 0; v < V; ++v) v0[v] = (t < 0) ? conv_input<TA, W>(a, b, t, c0 + v) : 0.0f;
        win[r] = IO::from(v0);
      }
    }
  }
  float wt[V][W], bs[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int k = 0; k < W; ++k) wt[v][k] = a.w[static_cast<size_t>(c0 + v) * W + k];
    bs[v] = a.bias ? a.bias[c0 + v] : 0.0f;
  }
  const int jend = (L - t0 < T) ? static_cast<int>(L - t0) : T;  // outputs in this stretch
#pragma unroll
  for (int j = 0; j < T; ++j) {
    const int64_t t = t0 + j;
    if (j < jend) {
      float o[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float acc = bs[v];
#pragma unroll
        for (int k = 0; k < W; ++k) acc = __builtin_fmaf(wt[v][k], IO::get(win[j + k], v), acc);
        o[v] = SILU ? silu_f32(acc) : acc;
      }
      IO::store(a.out + (b * L + t) * a.dim + c0, o);
    }
  }
  // the stretch holding the last token (or the first stretch of an empty
  // sequence) leaves the last W-1 inputs as the new conv state; they are
  // read again (cache-resident) rather than indexed out of registers
  const bool last = (L > 0) ? (t0 <= L - 1 && L - 1 < t0 + T) : (t0 == 0);
  if (a.state1 && last) {
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int j = 0; j < W - 1; ++j)
        store_act(a.state1 + (b * a.dim + c0 + v) * (W - 1) + j,
                  conv_input<TA, W>(a, b, L - (W - 1) + j, c0 + v));
  }
}

template <typename TA>
struct ConvUpdArgs {
  TA* state;  // (batch, dim, W-1), in place
  const TA* x;
  const float* w;
  const float* bias;
  TA* out;
  int64_t batch;
  int dim;
};

// Element access with the nontemporal hint: the decode update streams the
// conv state, the input and the output once (256 x 5120, W = 4: 12.0 -> 11.1 us).
template <typename T>
__device__ __forceinline__ T ntld(const T* p) {
  return __builtin_nontemporal_load(p);
}
template <>
__device__ __forceinline__ bf16_t ntld(const bf16_t* p) {
  bf16_t r;
  r.bits = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
  return r;
}
template <typename T>
__device__ __forceinline__ void ntst(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}
template <>
__device__ __forceinline__ void ntst(bf16_t* p, bf16_t v) {
  __builtin_nontemporal_store(v.bits, reinterpret_cast<uint16_t*>(p));
}
// an activation value rounded to the element type (bf16: nearest even)
__device__ __forceinline__ void ntact(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void ntact(bf16_t* p, float v) {
  __bf16 b = static_cast<__bf16>(v);
  __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, b), reinterpret_cast<uint16_t*>(p));
}

// One lane per (sequence, channel): out from the state and the new input,
// then the state shifts by one (the oldest input drops out).
template <typename TA, int W, bool SILU>
__global__ void __launch_bounds__(256) conv_update_kernel(ConvUpdArgs<TA> a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= a.batch * a.dim) return;
  const int d = static_cast<int>(i % a.dim);
  TA* st = a.state + i * (W - 1);
  TA prev[W - 1];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) prev[j] = ntld(st + j);
  const TA xin = ntld(a.x + i);
  const float* wd = a.w + static_cast<size_t>(d) * W;
  float acc = a.bias ? a.bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < W - 1; ++k) acc = __builtin_fmaf(wd[k], to_f32(prev[k]), acc);
  acc = __builtin_fmaf(wd[W - 1], to_f32(xin), acc);
  ntact(a.out + i, SILU ? silu_f32(acc) : acc);
#pragma unroll
  for (int j = 0; j + 1 < W - 1; ++j) ntst(st + j, prev[j + 1]);
  ntst(st + (W - 2), xin);
}

template <typename TA, int V>
int launch_conv_fwd(const ConvArgs<TA>& a0, int W, bool silu, hipStream_t s) {
  ConvArgs<TA> a = a0;
  a.tiles = (a.dim + 64 * V - 1) / (64 * V);
  a.chunks = a.L > 0 ? (a.L + kConvTokens - 1) / kConvTokens : 1;
  const int64_t units = static_cast<int64_t>(a.tiles) * a.chunks * a.batch;
  const int64_t blocks = (units + kXcds - 1) / kXcds * kXcds;
  const dim3 grid(static_cast<unsigned>(blocks)), block(64);
#define SSM_CONV_CASE(WW)                                                               \
  case WW:                                                                              \
    if (silu)                                                                           \
      hipLaunchKernelGGL((conv_fwd_kernel<TA, WW, V, true>), grid, block, 0, s, a);      \
    else                                                                                \
      hipLaunchKernelGGL((conv_fwd_kernel<TA, WW, V, false>), grid, block, 0, s, a);     \
    break;
  switch (W) {
    SSM_CONV_CASE(2)
    SSM_CONV_CASE(3)
    SSM_CONV_CASE(4)
    default: break;
  }
#undef SSM_CONV_CASE
  return launch_status("ssm_causal_conv1d_fwd");
}

template <typename TA>
int launch_conv_update(const ConvUpdArgs<TA>& a, int W, bool silu, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.batch * a.dim + 255) / 256)), block(256);
#define SSM_CONV_CASE(WW)                                                                   \
  case WW:                                                                                  \
    if (silu)                                                                               \
      hipLaunchKernelGGL((conv_update_kernel<TA, WW, true>), grid, block, 0, s, a);          \
    else                                                                                    \
      hipLaunchKernelGGL((conv_update_kernel<TA, WW, false>), grid, block, 0, s, a);         \
    break;
  switch (W) {
    SSM_CONV_CASE(2)
    SSM_CONV_CASE(3)
    SSM_CONV_CASE(4)
    default: break;
  }
#undef SSM_CONV_CASE
  return launch_status("ssm_causal_conv1d_update");
}

constexpr int64_t kConvMaxDim = int64_t{1} << 24;
constexpr int64_t kConvMaxBlocks = (int64_t{1} << 31) - 1;

}  // namespace ssm

using namespace ssm;

extern "C" {

int ssm_causal_conv1d_fwd(const void* x, const float* weight, const float* bias,
                          const void* initial_conv_state, void* out, void* final_conv_state,
                          int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int silu,
                          int dtype, hipStream_t stream) {
  clear_error();
  const char* fn = "ssm_causal_conv1d_fwd";
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (silu != 0 && silu != 1)
    return fail(SSM_ERR_UNSUPPORTED, "%s: silu must be 0 or 1, got %d", fn, silu);
  if (width < 2 || width > 4)
    return fail(SSM_ERR_UNSUPPORTED, "%s: width must be 2, 3 or 4, got %lld", fn, (long long)width);
  if (batch < 1 || dim < 1 || seqlen < 0 || dim > kConvMaxDim || batch > 65535 ||
      seqlen > (int64_t{1} << 40) / dim)
    return fail(SSM_ERR_SHAPE, "%s: bad sizes batch %lld, seqlen %lld, dim %lld", fn,
                (long long)batch, (long long)seqlen, (long long)dim);
  // one launch: at most 2^25 units of 64 lanes (counted for one channel per lane)
  if (batch * ((seqlen + kConvTokens - 1) / kConvTokens) * ((dim + 63) / 64) >= (int64_t{1} << 25))
    return fail(SSM_ERR_SHAPE, "%s: batch %lld x seqlen %lld x dim %lld exceeds one launch", fn,
                (long long)batch, (long long)seqlen, (long long)dim);
  if (!weight || (seqlen > 0 && (!x || !out)))
    return fail(SSM_ERR_NULL, "%s: weight, x and out are required", fn);
  const size_t es = dtype == SSM_DTYPE_F32 ? 4 : 2;
  const struct { const void* p; size_t k; const char* n; } al[] = {
      {x, es, "x"}, {out, es, "out"}, {weight, 4, "weight"}, {bias, 4, "bias"},
      {initial_conv_state, es, "initial_conv_state"}, {final_conv_state, es, "final_conv_state"}};
  for (const auto& e : al)
    if (e.p && !aligned(e.p, e.k))
      return fail(SSM_ERR_ALIGN, "%s: %s is not %zu-byte aligned", fn, e.n, e.k);
  const size_t tok = static_cast<size_t>(batch) * seqlen * dim * es;
  const size_t st = static_cast<size_t>(batch) * dim * (width - 1) * es;
  const Span ins[] = {{x, tok, "x"}, {weight, static_cast<size_t>(dim) * width * 4, "weight"},
                      {bias, bias ? static_cast<size_t>(dim) * 4 : 0, "bias"},
                      {initial_conv_state, initial_conv_state ? st : 0, "initial_conv_state"}};
  const Span outs[] = {{out, tok, "out"},
                       {final_conv_state, final_conv_state ? st : 0, "final_conv_state"}};
  for (const auto& o : outs)
    for (const auto& i : ins)
      if (overlap(o, i))
        return fail(SSM_ERR_ALIAS, "%s: output %s overlaps input %s", fn, o.name, i.name);
  if (overlap(outs[0], outs[1])) return fail(SSM_ERR_ALIAS, "%s: out overlaps final_conv_state", fn);
  if (seqlen == 0 && !final_conv_state) return SSM_OK;
  // vectors of channels where the layout allows them (float32: 4, bf16: 2)
  const int V = dtype == SSM_DTYPE_F32 ? 4 : kConvVecBf16;
  const bool vec = dim % V == 0 && (seqlen == 0 || (aligned(x, V * es) && aligned(out, V * es)));
  const int64_t tiles = (dim + 64 * (vec ? V : 1) - 1) / (64 * (vec ? V : 1));
  const int64_t chunks = seqlen > 0 ? (seqlen + kConvTokens - 1) / kConvTokens : 1;
  if (tiles * chunks * batch + kXcds > kConvMaxBlocks)
    return fail(SSM_ERR_SHAPE, "%s: problem too large for one launch", fn);
  const bool sl = silu != 0;
  if (dtype == SSM_DTYPE_F32) {
    ConvArgs<float> a{static_cast<const float*>(x), weight, bias,
                      static_cast<const float*>(initial_conv_state), static_cast<float*>(out),
                      static_cast<float*>(final_conv_state), batch, seqlen, static_cast<int>(dim),
                      0, 0};
    return vec ? launch_conv_fwd<float, 4>(a, static_cast<int>(width), sl, stream)
               : launch_conv_fwd<float, 1>(a, static_cast<int>(width), sl, stream);
  }
  ConvArgs<bf16_t> a{static_cast<const bf16_t*>(x), weight, bias,
                     static_cast<const bf16_t*>(initial_conv_state), static_cast<bf16_t*>(out),
                     static_cast<bf16_t*>(final_conv_state), batch, seqlen, static_cast<int>(dim),
                     0, 0};
  return vec ? launch_conv_fwd<bf16_t, kConvVecBf16>(a, static_cast<int>(width), sl, stream)
             : launch_conv_fwd<bf16_t, 1>(a, static_cast<int>(width), sl, stream);
}

int ssm_causal_conv1d_update(void* conv_state, const void* x, const float* weight,
                             const float* bias, void* out, int64_t batch, int64_t dim,
                             int64_t width, int silu, int dtype, hipStream_t stream) {
  clear_error();
  const char* fn = "ssm_causal_conv1d_update";
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (silu != 0 && silu != 1)
    return fail(SSM_ERR_UNSUPPORTED, "%s: silu must be 0 or 1, got %d", fn, silu);
  if (width < 2 || width > 4)
    return fail(SSM_ERR_UNSUPPORTED, "%s: width must be 2, 3 or 4, got %lld", fn, (long long)width);
  if (batch < 1 || dim < 1 || dim > kConvMaxDim || batch > (int64_t{1} << 31) ||
      batch * dim > (int64_t{1} << 31) - 256)  // (batch bounded first: no overflow)
    return fail(SSM_ERR_SHAPE, "%s: bad sizes batch %lld, dim %lld", fn, (long long)batch,
                (long long)dim);
  if (!conv_state || !x || !weight || !out)
    return fail(SSM_ERR_NULL, "%s: conv_state, x, weight and out are required", fn);
  const size_t es = dtype == SSM_DTYPE_F32 ? 4 : 2;
  const struct { const void* p; size_t k; const char* n; } al[] = {
      {x, es, "x"}, {out, es, "out"}, {conv_state, es, "conv_state"}, {weight, 4, "weight"},
      {bias, 4, "bias"}};
  for (const auto& e : al)
    if (e.p && !aligned(e.p, e.k))
      return fail(SSM_ERR_ALIGN, "%s: %s is not %zu-byte aligned", fn, e.n, e.k);
  const size_t tok = static_cast<size_t>(batch) * dim * es;
  const size_t st = static_cast<size_t>(batch) * dim * (width - 1) * es;
  const Span ins[] = {{x, tok, "x"}, {weight, static_cast<size_t>(dim) * width * 4, "weight"},
                      {bias, bias ? static_cast<size_t>(dim) * 4 : 0, "bias"}};
  const Span outs[] = {{out, tok, "out"}, {conv_state, st, "conv_state"}};
  for (const auto& o : outs)
    for (const auto& i : ins)
      if (overlap(o, i))
        return fail(SSM_ERR_ALIAS, "%s: %s overlaps input %s", fn, o.name, i.name);
  if (overlap(outs[0], outs[1])) return fail(SSM_ERR_ALIAS, "%s: out overlaps conv_state", fn);
  const bool sl = silu != 0;
  if (dtype == SSM_DTYPE_F32) {
    ConvUpdArgs<float> a{static_cast<float*>(conv_state), static_cast<const float*>(x), weight,
                         bias, static_cast<float*>(out), batch, static_cast<int>(dim)};
    return launch_conv_update(a, static_cast<int>(width), sl, stream);
  }
  ConvUpdArgs<bf16_t> a{static_cast<bf16_t*>(conv_state), static_cast<const bf16_t*>(x), weight,
                        bias, static_cast<bf16_t*>(out), batch, static_cast<int>(dim)};
  return launch_conv_update(a, static_cast<int>(width), sl, stream);
}

}  // extern "C"
