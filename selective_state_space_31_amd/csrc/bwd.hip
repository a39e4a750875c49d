// bwd.hip -- gradients of the selective scan (the backward pass) for MI355X
// (gfx950), behind the C ABI in include/ssm_scan.h (see there for the
// citation and the definition of every gradient).
//
// The forward keeps no (b, L, D, N) states; neither does this: it recomputes
// them, stripe by stripe (recomputation in the backward pass, as the page
// cited in the header describes for the original kernel).  Plan, for
// stripes of Ls <= 32 tokens:
//   1. summaries, one launch for both: per stripe, the state it reaches
//      from zero with its sum of Delta (the forward's chunk summary), and the
//      adjoint walked from its last token to its first from a zero adjoint,
//      a <- (a + C_t dy_t) * e^(dt_t A); the adjoint recurrence is linear
//      with the same decays as the state, so
//   2. one carry launch folds both chains: the states from the initial
//      state in stripe order, the adjoints from dlast_state in reverse
//      stripe order, giving the state entering every stripe and the
//      adjoint flowing into every stripe's last token from the tokens after
//      it;
//   3. main pass: per stripe, SPL = min(N, 8) states per lane (N/SPL lanes
//      per channel).  The lane runs its stripe forward from the entering
//      state, keeping a checkpoint of its states every SUB = 64/SPL tokens,
//      then takes the sub-chunks from last to first: recompute the
//      sub-chunk's states into registers (64 floats of history), walk it
//      backwards with the adjoint.  Per-token gradients
//      (dx, ddelta, dz) are stored at once; dB and dC, sums over channels,
//      are reduced across the wave's channels by lane shuffles and across
//      the workgroup's 4 waves in LDS into one partial per workgroup;
//      dA, dD, dbias are accumulated per stripe;
//   4. a reduction pass adds the partials in a fixed order (no atomics: the
//      result is bitwise reproducible run to run).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_scan.h"

#include "host_util.hpp"
#include "kernels.hpp"

namespace ssm {

constexpr int kBwdStripe = 32;     // tokens per stripe at most (a multiple of 16)
constexpr int kAdjGroup = 4;      // tokens per load group of the adjoint summary walk
constexpr int kBwdThreads = 256;   // main pass workgroup: 4 waves of the same stripe

// Main-pass shape for a state width: SPL states per lane, G lanes per
// channel, sub-chunks of SUB tokens whose states are recomputed into
// registers (SUB x SPL = 64 floats of history per lane).
template <int NT>
struct BwdShape {
  static constexpr int SPL = NT >= 8 ? 8 : NT;
  static constexpr int G = NT / SPL;
  static constexpr int SUB = 64 / SPL;
  static constexpr int MAXSUB = kBwdStripe / SUB;
  static constexpr int CPB = kBwdThreads / G;
};

template <typename TA>
struct BwdArgs {
  const TA* x;
  const TA* delta;
  const float* bias;
  const float* A;
  const TA* B;
  const TA* C;
  const float* Dsk;
  const TA* z;
  const float* h0;
  const TA* dout;
  const float* dlast;
  TA* dx;
  TA* ddelta;
  TA* dz;
  float* dh0;
  const float* fH;  // (b, K, N, D): slot c = state entering stripe c (c >= 1)
  float* rS;        // (b, K-1, D): slot j = sum of Delta over stripe K-1-j
  float* rH;        // (b, K, N, D): slot K-c <- adjoint summary of stripe c; after the
                    // carry, slot j = adjoint flowing into stripe K-1-j's last token
  float* pB;        // (tiles, b, L, N) partial dB per workgroup tile
  float* pC;        // (tiles, b, L, N) partial dC
  float* pA;        // (b, K, D, N) partial dA per stripe
  float* pD;        // (b, K, D) partial dD
  float* pbias;     // (b, K, D) partial dbias
  int64_t batch;
  int L;
  int Ls;
  int K;
  int dim;
  int tiles;
};

__device__ __forceinline__ float sigmoid_f32(float u) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u * kLog2e));
}

// ----------------------------------------------------------------------------
// 1. adjoint summary of stripe c = 1..K-1 of sequence b (one wave, 64 channels)
// ----------------------------------------------------------------------------
template <typename TA, int NT, bool SP, bool GATE>
__device__ __forceinline__ void bwd_agg_block(const BwdArgs<TA>& a, int tile, int c, int64_t b) {
  const int lane = threadIdx.x;
  const int d = tile * 64 + lane;
  const bool valid = d < a.dim;
  const int dl = valid ? d : a.dim - 1;
  float a2[NT], adj[NT];
  const float A0 = a.A[static_cast<size_t>(dl) * NT];
  bool pow_ok = true;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float An = a.A[static_cast<size_t>(dl) * NT + n];
    a2[n] = An * kLog2e;
    adj[n] = 0.0f;
    pow_ok = pow_ok && (An == static_cast<float>(n + 1) * A0);
  }
  const bool pw = __all(pow_ok);
  const float bias = a.bias ? a.bias[dl] : 0.0f;
  const int s = c * a.Ls;
  const int e = (s + a.Ls < a.L) ? s + a.Ls : a.L;
  float S = 0.0f;
  // A token's inputs: its dt and dy inputs (per lane) and its C row (uniform).
  // The walks take tokens in groups of kAdjGroup whose loads are all issued
  // before the first of them is used, so a group waits for memory once.
  struct Tok {
    TA dl, g, zz;
    float Cv[NT];
  };
  auto fetch = [&](int t, Tok& k) {
    const size_t i = (static_cast<size_t>(b) * a.L + t) * a.dim + dl;
    k.dl = a.delta[i];
    k.g = a.dout[i];
    if constexpr (GATE) k.zz = a.z[i];
    load_row<NT, true>(a.C + (static_cast<size_t>(b) * a.L + t) * NT, NT, k.Cv);
  };
  auto prep = [&](const Tok& k, float& dt, float& dy) {
    const float u = to_f32(k.dl) + bias;
    dt = SP ? softplus_f32(u) : u;
    const float g = to_f32(k.g);
    if constexpr (GATE)
      dy = g * silu_f32(to_f32(k.zz));
    else
      dy = g;
  };
  // The summary is sum_t (prod_{u=s..t} e^(dt_u A)) C_t dy_t.  S4D-real A
  // (every lane of the wave): e^(dt A[n]) = r^(n+1), r = e^(dt A[0]), so walking
  // the stripe forward with P = prod_{u<=t} r_u the weight of state n is
  // dy_t P^(n+1), a chain of multiplies: one multiply and one FMA per state
  // (the mirror of the forward summary pass).  Otherwise the walk runs
  // backwards, a <- (a + C_t dy_t) e^(dt_t A), one exponential per state.
  if (pw) {
    float P = 1.0f;
    for (int t0 = s; t0 < e; t0 += kAdjGroup) {
      Tok k[kAdjGroup];
#pragma unroll
      for (int u = 0; u < kAdjGroup; ++u) fetch(t0 + u < e ? t0 + u : e - 1, k[u]);
#pragma unroll
      for (int u = 0; u < kAdjGroup; ++u) {
        if (t0 + u < e) {
          float dt, dy;
          prep(k[u], dt, dy);
          S += dt;
          P *= __builtin_amdgcn_exp2f(dt * a2[0]);
          float wgt = dy * P;
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            adj[n] = __builtin_fmaf(wgt, k[u].Cv[n], adj[n]);
            wgt *= P;
          }
        }
      }
    }
  } else {
    for (int t1 = e; t1 > s; t1 -= kAdjGroup) {  // tokens t1-1 down to t1-kAdjGroup
      Tok k[kAdjGroup];
#pragma unroll
      for (int u = 0; u < kAdjGroup; ++u) fetch(t1 - 1 - u >= s ? t1 - 1 - u : s, k[u]);
#pragma unroll
      for (int u = 0; u < kAdjGroup; ++u) {
        if (t1 - 1 - u >= s) {
          float dt, dy;
          prep(k[u], dt, dy);
          S += dt;
#pragma unroll
          for (int n = 0; n < NT; ++n)
            adj[n] = __builtin_fmaf(k[u].Cv[n], dy, adj[n]) * __builtin_amdgcn_exp2f(dt * a2[n]);
        }
      }
    }
  }
  if (valid) {
    a.rS[(static_cast<size_t>(b) * (a.K - 1) + (a.K - 1 - c)) * a.dim + d] = S;
    const size_t slot = static_cast<size_t>(b) * a.K + (a.K - c);
#pragma unroll
    for (int n = 0; n < NT; ++n) a.rH[(slot * NT + n) * a.dim + d] = adj[n];
  }
}

// Step 1 in one launch: block (x, stripe, sequence) of one wave; the
// first `tiles` x-blocks summarise the states of stripe y (the forward's
// chunk summary), the others the adjoints of stripe y+1.
template <typename TA, int NT, bool SP, bool GATE>
__global__ void __launch_bounds__(64) bwd_sums_kernel(BwdArgs<TA> a, FwdArgs<TA> f) {
  const int tiles = (a.dim + 63) / 64;
  const int x = static_cast<int>(blockIdx.x);
  if (x < tiles)
    fwd_agg_block<TA, NT, SP>(f, x, static_cast<int>(blockIdx.y), static_cast<int>(blockIdx.z));
  else
    bwd_agg_block<TA, NT, SP, GATE>(a, x - tiles, static_cast<int>(blockIdx.y) + 1, blockIdx.z);
}

// ----------------------------------------------------------------------------
// 3. main pass
// ----------------------------------------------------------------------------
// Sum over the G lanes of one channel (adjacent lanes of a quad): DPP quad
// permutations, no LDS traffic.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm(1,0,3,2)
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm(2,3,0,1)
template <int G>
__device__ __forceinline__ float sum_group(float v) {
  if constexpr (G >= 2)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                             kDppQuadXor1, 0xf, 0xf, false));
  if constexpr (G >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                             kDppQuadXor2, 0xf, 0xf, false));
  return v;
}

// The 8 per-lane values (4 dB and 4 dC terms of the lane's states) summed
// over the wave's channels (the lanes with the same state group), as a
// reduce-scatter: each exchange across lane bit 5, 4, 3 sends half of the
// remaining values and keeps the other half, so 8 values cost 4 + 2 + 1
// exchanges, then full exchanges over the bits from 2 down to the group
// size.  Returns the sum of value ((lane>>5)&1)*4 + ((lane>>4)&1)*2 +
// ((lane>>3)&1) for the lane's state group; lanes differing only in bits
// 2..log2(G) hold the same sum.
//   bits 5 and 4: v_permlane32_swap / v_permlane16_swap (checked on the
//     device): swapping (x, y) leaves a lane of the lower half with its own x
//     and its partner's x, a lane of the upper half with its partner's y and
//     its own y, so x + y is the kept half's pair sum in every lane, with no
//     selects and no LDS;
//   bit 3: DPP row rotate by 8 (the partner within the row of 16);
//   bits 2..: ds_swizzle exchanges (xor within 32 lanes).
__device__ __forceinline__ float sum_swap32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_swap16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
constexpr int kDppRowRor8 = 0x128;
template <int O>
__device__ __forceinline__ float swizzle_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (O << 10) | 0x1F));
}
// Reduce-scatter of V values per lane (V = 8 or 16) over the lanes of the
// same state group: exchanges across lane bits 5, 4, 3 (and 2 for V = 16)
// each keep half of the remaining values, then full exchanges over the
// remaining channel bits.  The lane ends with the sum of value
// scatter_index<V>(lane).
template <int V>
__device__ __forceinline__ int scatter_index(int lane) {
  int vi = ((lane >> 5) & 1) * (V / 2) + ((lane >> 4) & 1) * (V / 4) + ((lane >> 3) & 1) * (V / 8);
  if constexpr (V == 16) vi += (lane >> 2) & 1;
  return vi;
}
template <int V, int G>
__device__ __forceinline__ float reduce_scatter(const float (&v)[V]) {
  static_assert(V == 8 || V == 16, "8 or 16 values");
  const int lane = static_cast<int>(threadIdx.x & 63);
  float w32[V / 2];
#pragma unroll
  for (int j = 0; j < V / 2; ++j) w32[j] = sum_swap32(v[j], v[j + V / 2]);
  float w16[V / 4];
#pragma unroll
  for (int j = 0; j < V / 4; ++j) w16[j] = sum_swap16(w32[j], w32[j + V / 4]);
  const bool b3 = lane & 8;
  float w8[V / 8];
#pragma unroll
  for (int j = 0; j < V / 8; ++j) {
    const float keep = b3 ? w16[j + V / 8] : w16[j], send = b3 ? w16[j] : w16[j + V / 8];
    w8[j] = keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), kDppRowRor8, 0xf,
                                                           0xf, false));
  }
  float w;
  if constexpr (V == 16) {
    const bool b2 = lane & 4;
    const float keep = b2 ? w8[1] : w8[0], send = b2 ? w8[0] : w8[1];
    w = keep + swizzle_xor<4>(send);
    if constexpr (G <= 2) w += swizzle_xor<2>(w);
    if constexpr (G <= 1) w += swizzle_xor<1>(w);
  } else {
    w = w8[0];
    if constexpr (G <= 4) w += swizzle_xor<4>(w);
    if constexpr (G <= 2) w += swizzle_xor<2>(w);
    if constexpr (G <= 1) w += swizzle_xor<1>(w);
  }
  return w;
}

// A compile-time flag passed to a generic lambda.
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

template <typename TA, int NT, bool SP, bool GATE>
__global__ void __launch_bounds__(kBwdThreads) bwd_main_kernel(BwdArgs<TA> a) {
  using Sh = BwdShape<NT>;
  constexpr int SPL = Sh::SPL;  // states per lane
  constexpr int G = Sh::G;      // lanes per channel
  constexpr int SUB = Sh::SUB;  // tokens per recomputed sub-chunk
  constexpr int CPB = Sh::CPB;  // channels per workgroup
  constexpr int V = 2 * SPL;    // dB and dC terms per lane and token
  constexpr int WAVES = kBwdThreads / 64;
  __shared__ float red[WAVES][SUB][2 * NT];
  __shared__ float ckpt[Sh::MAXSUB][SPL][kBwdThreads];  // per-lane checkpoints
  constexpr bool kCacheDt = G > 1;
  __shared__ float dtc[kCacheDt ? kBwdStripe : 1][kCacheDt ? CPB : 1];  // dt per token, channel

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = tid % G;
  const int n0 = SPL * g;
  const int d = blockIdx.x * CPB + tid / G;
  const int c = blockIdx.y;
  const int64_t b = blockIdx.z;
  const bool valid = d < a.dim;
  const int dl = valid ? d : a.dim - 1;
  const int N = NT;
  const int s = c * a.Ls;
  const int e = (s + a.Ls < a.L) ? s + a.Ls : a.L;
  const int len = e - s;

  float Aj[SPL], a2[SPL];
  const float A0 = a.A[static_cast<size_t>(dl) * N];
  bool pow_ok = true;
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    Aj[j] = a.A[static_cast<size_t>(dl) * N + n0 + j];
    a2[j] = Aj[j] * kLog2e;
    pow_ok = pow_ok && (Aj[j] == static_cast<float>(n0 + j + 1) * A0);
  }
  // S4D-real A (every lane of the workgroup): e^(dt A[n]) = r^(n+1),
  // r = e^(dt A[0]); every fourth decay is its own exponential, the three
  // after it follow by multiplying with r (a few ulp).  The choice is made
  // once per workgroup (the walks below hold barriers) and each kind of A
  // runs its own copy of the walks, so no token's work is split by a branch.
  const bool pw = __syncthreads_and(pow_ok) != 0;
  const float a20 = A0 * kLog2e;
  auto run = [&](auto pow_tag) {
  constexpr bool POW = decltype(pow_tag)::value;
  auto decays = [&](float dt, float (&dA)[SPL]) {
    if constexpr (POW) {
      const float r = __builtin_amdgcn_exp2f(dt * a20);
#pragma unroll
      for (int j = 0; j < SPL; ++j)
        dA[j] = (j % 4 == 0) ? __builtin_amdgcn_exp2f(dt * a2[j]) : dA[j > 0 ? j - 1 : 0] * r;
    } else {
#pragma unroll
      for (int j = 0; j < SPL; ++j) dA[j] = __builtin_amdgcn_exp2f(dt * a2[j]);
    }
  };
  const float bias = a.bias ? a.bias[dl] : 0.0f;
  const float dsk = a.Dsk ? a.Dsk[dl] : 0.0f;

  // state entering the stripe
  float h[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    if (c == 0)
      h[j] = a.h0 ? a.h0[(static_cast<size_t>(b) * a.dim + dl) * N + n0 + j] : 0.0f;
    else
      h[j] = a.fH[((static_cast<size_t>(b) * a.K + c) * N + n0 + j) * a.dim + dl];
  }

  // Token rows of a sub-chunk through buffer descriptors based at its first
  // token: the lane's column is a constant offset, the token a scalar one,
  // and rows past the sub-chunk fall outside the range (loads read zero).
  using IO = Io<TA>;
  constexpr uint32_t es = sizeof(TA);
  const uint32_t rowA = static_cast<uint32_t>(a.dim) * es;  // bytes per activation row
  const uint32_t rowN = static_cast<uint32_t>(N) * es;      // bytes per B / C row
  const uint32_t vo_a = static_cast<uint32_t>(dl) * es, vo_n = static_cast<uint32_t>(n0) * es;
  struct Rows {
    rsrc_t x, delta, B;
  };
  auto rows_at = [&](int t0, int t1) {
    const size_t ra = (static_cast<size_t>(b) * a.L + t0) * a.dim;
    const size_t rn = (static_cast<size_t>(b) * a.L + t0) * N;
    const uint32_t n = static_cast<uint32_t>(t1 - t0);
    return Rows{make_rsrc(a.x + ra, n * rowA), make_rsrc(a.delta + ra, n * rowA),
                make_rsrc(a.B + rn, n * rowN)};
  };
  // the lane's SPL consecutive values of a B / C row
  auto loadS = [&](rsrc_t r, uint32_t soff, float (&v)[SPL]) {
    if constexpr (sizeof(TA) == 2) {  // 8-byte loads: B and C rows are 8-byte aligned
#pragma unroll
      for (int q = 0; q < SPL / 4; ++q) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, vo_n + 8 * q, soff, 0);
        v[4 * q] = __uint_as_float(w[0] << 16);
        v[4 * q + 1] = __uint_as_float(w[0] & 0xffff0000u);
        v[4 * q + 2] = __uint_as_float(w[1] << 16);
        v[4 * q + 3] = __uint_as_float(w[1] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < SPL / 4; ++q) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(r, vo_n + 16 * q, soff, 0);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[4 * q + k] = __uint_as_float(w[k]);
      }
    }
  };

  // dt of row i of the sub-chunk
  auto step_dt = [&](const Rows& r, int i) {
    const float u = IO::f32(IO::load(r.delta, vo_a, static_cast<uint32_t>(i) * rowA)) + bias;
    return SP ? softplus_f32(u) : u;
  };
  // one forward token (row i of the sub-chunk): hout = e^(dt A) hin + dt B x
  // (written to its own registers, so that the sub-chunk recompute fills its
  // history without copies)
  auto fwd_step_to = [&](const Rows& r, int i, float dt, const float (&hin)[SPL],
                         float (&hout)[SPL]) {
    const float dx = dt * IO::f32(IO::load(r.x, vo_a, static_cast<uint32_t>(i) * rowA));
    float Bv[SPL], dA[SPL];
    loadS(r.B, static_cast<uint32_t>(i) * rowN, Bv);
    decays(dt, dA);
#pragma unroll
    for (int j = 0; j < SPL; ++j) hout[j] = __builtin_fmaf(dA[j], hin[j], dx * Bv[j]);
  };

  // 3a. forward over the stripe with a checkpoint every SUB tokens (in LDS:
  // each lane reads back only its own); the state after the last sub-chunk
  // is not needed.  With several lanes per channel, every token's dt is also
  // kept in LDS (both lanes write the same value; each reads it back), so
  // the recompute below does not evaluate the softplus again.
  const int nsub = (len + SUB - 1) / SUB;
  const int chw = tid / G;  // the lane's channel within the workgroup
  for (int k = 0; k < nsub; ++k) {
#pragma unroll
    for (int j = 0; j < SPL; ++j) ckpt[k][j][tid] = h[j];
    const int t0 = s + k * SUB;
    if (k == nsub - 1) {
      if constexpr (kCacheDt) {
        const Rows r = rows_at(t0, e);
#pragma unroll 2
        for (int i = 0; i < SUB; ++i) dtc[k * SUB + i][chw] = step_dt(r, i);
      }
      break;
    }
    const Rows r = rows_at(t0, t0 + SUB);
#pragma unroll 2
    for (int i = 0; i < SUB; ++i) {
      const float dt = step_dt(r, i);
      if constexpr (kCacheDt) dtc[k * SUB + i][chw] = dt;
      fwd_step_to(r, i, dt, h, h);
    }
  }

  // 3b. adjoint flowing into the stripe's last token from later tokens
  float adj[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    if (!valid)  // (lanes past the channels: zero adjoint and zero dy keep every sum clean)
      adj[j] = 0.0f;
    else if (c == a.K - 1)
      adj[j] = a.dlast ? a.dlast[(static_cast<size_t>(b) * a.dim + dl) * N + n0 + j] : 0.0f;
    else
      adj[j] = a.rH[((static_cast<size_t>(b) * a.K + (a.K - 1 - c)) * N + n0 + j) * a.dim + dl];
  }
  float dAacc[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) dAacc[j] = 0.0f;
  float dDacc = 0.0f, dbacc = 0.0f;

  // 3c. sub-chunks from last to first (nsub is uniform over the workgroup)
  for (int k = nsub - 1; k >= 0; --k) {
    const int t0 = s + k * SUB;
    const int t1 = (t0 + SUB < e) ? t0 + SUB : e;
    const Rows r = rows_at(t0, t1);
    const size_t ra = (static_cast<size_t>(b) * a.L + t0) * a.dim;
    const uint32_t nbytes = static_cast<uint32_t>(t1 - t0) * rowA;
    const rsrc_t rdo = make_rsrc(a.dout + ra, nbytes);
    const rsrc_t rz = make_rsrc(GATE ? a.z + ra : a.x + ra, nbytes);
    const rsrc_t rC = make_rsrc(a.C + (static_cast<size_t>(b) * a.L + t0) * N,
                                static_cast<uint32_t>(t1 - t0) * rowN);
    // gradients of the per-token rows: only lane 0 of each channel stores
    // (the others store past every descriptor's range, which the hardware
    // drops; byte ranges here stay below 2^30)
    const rsrc_t rdx = make_rsrc(a.dx + ra, nbytes), rdd = make_rsrc(a.ddelta + ra, nbytes);
    const rsrc_t rdz = make_rsrc(GATE ? a.dz + ra : a.dx + ra, GATE ? nbytes : 0);
    const uint32_t vo_st = (g == 0 && valid) ? vo_a : kOutOfRange;
    float ck[SPL], hist[SUB][SPL], dts[SUB];
    {
#pragma unroll
      for (int j = 0; j < SPL; ++j) ck[j] = ckpt[k][j][tid];
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const float(&hin)[SPL] = i == 0 ? ck : hist[i > 0 ? i - 1 : 0];
        if (t0 + i < e) {
          dts[i] = kCacheDt ? dtc[k * SUB + i][chw] : step_dt(r, i);
          fwd_step_to(r, i, dts[i], hin, hist[i]);
        } else {
          dts[i] = 0.0f;
#pragma unroll
          for (int j = 0; j < SPL; ++j) hist[i][j] = hin[j];
        }
      }
    }
#pragma unroll
    for (int i = SUB - 1; i >= 0; --i) {
      const int t = t0 + i;
      // rows past the stripe's end (the last stripe of a ragged length) are
      // skipped: the adjoint passes through them unchanged, and the
      // workgroup's sum below reads no dB / dC slot of theirs
      if (t < e) {
        float pv[V];
        const uint32_t so = static_cast<uint32_t>(i) * rowA, son = static_cast<uint32_t>(i) * rowN;
        const float u = IO::f32(IO::load(r.delta, vo_a, so)) + bias;
        const float dt = dts[i];
        const float xv = IO::f32(IO::load(r.x, vo_a, so));
        float Bv[SPL], Cv[SPL];
        loadS(r.B, son, Bv);
        loadS(rC, son, Cv);
        // readout of this token (all states: sum over the channel's lanes)
        float yp = 0.0f;
#pragma unroll
        for (int j = 0; j < SPL; ++j) yp = __builtin_fmaf(Cv[j], hist[i][j], yp);
        const float y = sum_group<G>(yp) + dsk * xv;
        const float gv = IO::f32(IO::load(rdo, vo_a, so));
        float dy = gv, dzv = 0.0f;
        if constexpr (GATE) {
          const float zv = IO::f32(IO::load(rz, vo_a, so));
          const float sg = sigmoid_f32(zv);
          dy = gv * zv * sg;
          dzv = gv * y * sg * __builtin_fmaf(zv, 1.0f - sg, 1.0f);
        }
        if (!valid) dy = 0.0f;
        const float dtx = dt * xv;
        float s1p = 0.0f, s2p = 0.0f, dAv[SPL];
        decays(dt, dAv);
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
          const float hp = (i > 0) ? hist[i > 0 ? i - 1 : 0][j] : ck[j];
          adj[j] = __builtin_fmaf(Cv[j], dy, adj[j]);  // adjoint of h_t
          pv[SPL + j] = dy * hist[i][j];              // dC term
          const float an = adj[j] * dAv[j];           // adjoint of h_{t-1}
          const float q = an * hp;
          dAacc[j] = __builtin_fmaf(q, dt, dAacc[j]);
          s2p = __builtin_fmaf(Aj[j], q, s2p);
          s1p = __builtin_fmaf(adj[j], Bv[j], s1p);
          pv[j] = adj[j] * dtx;                       // dB term
          adj[j] = an;
        }
        const float s1 = sum_group<G>(s1p), s2 = sum_group<G>(s2p);
        const float ddt = __builtin_fmaf(xv, s1, s2);
        const float dxv = __builtin_fmaf(dt, s1, dsk * dy);
        const float dd = SP ? ddt * sigmoid_f32(u) : ddt;
        IO::store(dxv, rdx, vo_st, so);
        IO::store(dd, rdd, vo_st, so);
        if constexpr (GATE) IO::store(dzv, rdz, vo_st, so);
        dDacc = __builtin_fmaf(dy, xv, dDacc);
        dbacc += dd;
        // dB, dC of this token: sum over the wave's channels
        const float w = reduce_scatter<V, G>(pv);
        if ((lane & (64 / V - 1) & ~(G - 1)) == 0) {
          const int vi = scatter_index<V>(lane);
          red[wave][i][(vi < SPL ? 0 : NT) + n0 + (vi % SPL)] = w;
        }
      }
    }
    // sum over the workgroup's waves; one partial per (tile, b, t, n)
    __syncthreads();
    for (int idx = tid; idx < SUB * 2 * NT; idx += kBwdThreads) {
      const int i = idx / (2 * NT);
      const int rr = idx % (2 * NT);
      const int t = t0 + i;
      if (t < e) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) v += red[w][i][rr];
        float* dst = rr < NT ? a.pB : a.pC;
        dst[((static_cast<size_t>(blockIdx.x) * a.batch + b) * a.L + t) * N + (rr % NT)] = v;
      }
    }
    __syncthreads();
  }

  if (valid) {
    const size_t sc = static_cast<size_t>(b) * a.K + c;
#pragma unroll
    for (int j = 0; j < SPL; ++j) a.pA[(sc * a.dim + d) * N + n0 + j] = dAacc[j];
    if (g == 0) {
      a.pD[sc * a.dim + d] = dDacc;
      a.pbias[sc * a.dim + d] = dbacc;
    }
    if (c == 0 && a.dh0) {
#pragma unroll
      for (int j = 0; j < SPL; ++j)
        a.dh0[(static_cast<size_t>(b) * a.dim + d) * N + n0 + j] = adj[j];
    }
  }
  };
  if (pw)
    run(BoolTag<true>{});
  else
    run(BoolTag<false>{});
}

// ----------------------------------------------------------------------------
// 4. reductions of the partials, in a fixed order
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_reduce_bc_kernel(const float* __restrict__ pB,
                                                           const float* __restrict__ pC,
                                                           float* __restrict__ dB,
                                                           float* __restrict__ dC, int64_t per,
                                                           int tiles) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= per) return;
  // tile order; the loads of four tiles are issued before their adds
  float sb = 0.0f, scv = 0.0f;
  int k = 0;
  for (; k + 4 <= tiles; k += 4) {
    float vb[4], vc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      vb[u] = pB[(k + u) * per + i];
      vc[u] = pC[(k + u) * per + i];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sb += vb[u];
      scv += vc[u];
    }
  }
  for (; k < tiles; ++k) {
    sb += pB[k * per + i];
    scv += pC[k * per + i];
  }
  dB[i] = sb;
  dC[i] = scv;
}

// dA[d,n] = sum over (b, stripe) of pA; dD[d], dbias[d] likewise.  Block
// of 256 = 32 elements x 8 slice groups: group j sums the slices j, j+8, ...
// in order, and the 8 group sums are added in order (a fixed order: the
// result does not depend on scheduling).
constexpr int kRedElems = 32, kRedGroups = 8, kRedBatch = 8;
__global__ void __launch_bounds__(256) bwd_reduce_params_kernel(
    const float* __restrict__ pA, const float* __restrict__ pD, const float* __restrict__ pbias,
    float* __restrict__ dA, float* __restrict__ dD, float* __restrict__ dbias, int dim, int N,
    int64_t slices) {
  __shared__ float part[2][kRedGroups][kRedElems];
  const int e = threadIdx.x % kRedElems, j = threadIdx.x / kRedElems;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kRedElems + e;
  const int64_t nA = static_cast<int64_t>(dim) * N;
  // slice order within the group; the loads of kRedBatch slices are issued
  // before their adds (the latency of one load per add bound this loop)
  float v = 0.0f, vb = 0.0f;
  constexpr int U = kRedBatch;
  if (i < nA) {
    int64_t k = j;
    for (; k + (U - 1) * kRedGroups < slices; k += U * kRedGroups) {
      float t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) t[u] = pA[(k + u * kRedGroups) * nA + i];
#pragma unroll
      for (int u = 0; u < U; ++u) v += t[u];
    }
    for (; k < slices; k += kRedGroups) v += pA[k * nA + i];
  } else if (i < nA + dim) {
    const int64_t d = i - nA;
    int64_t k = j;
    for (; k + (U - 1) * kRedGroups < slices; k += U * kRedGroups) {
      float t[U], tb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        t[u] = pD[(k + u * kRedGroups) * dim + d];
        tb[u] = pbias[(k + u * kRedGroups) * dim + d];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        v += t[u];
        vb += tb[u];
      }
    }
    for (; k < slices; k += kRedGroups) {
      v += pD[k * dim + d];
      vb += pbias[k * dim + d];
    }
  }
  part[0][j][e] = v;
  part[1][j][e] = vb;
  __syncthreads();
  if (j == 0) {
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int g = 0; g < kRedGroups; ++g) {
      s0 += part[0][g][e];
      s1 += part[1][g][e];
    }
    if (i < nA) {
      dA[i] = s0;
    } else if (i < nA + dim) {
      if (dD) dD[i - nA] = s0;
      if (dbias) dbias[i - nA] = s1;
    }
  }
}

// No tokens: parameter gradients are zero, dinitial_state = dlast_state.
__global__ void __launch_bounds__(256) bwd_empty_kernel(const float* __restrict__ dlast,
                                                       float* __restrict__ dh0, int64_t nstate,
                                                       float* __restrict__ dA, float* dD,
                                                       float* dbias, int dim, int N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < nstate && dh0) dh0[i] = dlast ? dlast[i] : 0.0f;
  if (i < static_cast<int64_t>(dim) * N) dA[i] = 0.0f;
  if (i < dim) {
    if (dD) dD[i] = 0.0f;
    if (dbias) dbias[i] = 0.0f;
  }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------
struct BwdPlan {
  int Ls, K, tiles;
};

BwdPlan plan_bwd(int64_t batch, int64_t L, int64_t dim, int64_t N) {
  BwdPlan p;
  const int cpb = N == 16 ? BwdShape<16>::CPB : N == 8 ? BwdShape<8>::CPB : BwdShape<4>::CPB;
  p.tiles = static_cast<int>((dim + cpb - 1) / cpb);
  // enough workgroups for about 3 waves per SIMD; stripes are a multiple of
  // 16 tokens (whole sub-chunks, and whole token pairs-of-groups for the
  // forward summary pass that gives their entering states), at most kBwdStripe
  const int64_t per_stripe = static_cast<int64_t>(p.tiles) * batch * (kBwdThreads / 64);
  const int64_t target = 3LL * 4 * device_cus();
  int64_t K = (target + per_stripe - 1) / per_stripe;
  if (K < 1) K = 1;
  int64_t Ls = L > 0 ? (L + K - 1) / K : 16;
  Ls = (Ls + 15) / 16 * 16;
  if (Ls > kBwdStripe) Ls = kBwdStripe;
  K = L > 0 ? (L + Ls - 1) / Ls : 1;
  p.Ls = static_cast<int>(Ls);
  p.K = static_cast<int>(K);
  return p;
}

struct BwdWs {
  size_t fS, fH, rS, rH, pB, pC, pA, pD, pbias, total;
};

BwdWs bwd_layout(int64_t batch, int64_t L, int64_t dim, int64_t N, const BwdPlan& p) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  BwdWs w{};
  const size_t K = static_cast<size_t>(p.K);
  size_t o = 0;
  w.fS = o; o = up(o + static_cast<size_t>(batch) * (K > 0 ? K - 1 : 0) * dim * 4);
  w.fH = o; o = up(o + static_cast<size_t>(batch) * K * N * dim * 4);
  w.rS = o; o = up(o + static_cast<size_t>(batch) * (K > 0 ? K - 1 : 0) * dim * 4);
  w.rH = o; o = up(o + static_cast<size_t>(batch) * K * N * dim * 4);
  w.pB = o; o = up(o + static_cast<size_t>(p.tiles) * batch * L * N * 4);
  w.pC = o; o = up(o + static_cast<size_t>(p.tiles) * batch * L * N * 4);
  w.pA = o; o = up(o + static_cast<size_t>(batch) * K * dim * N * 4);
  w.pD = o; o = up(o + static_cast<size_t>(batch) * K * dim * 4);
  w.pbias = o; o = up(o + static_cast<size_t>(batch) * K * dim * 4);
  w.total = L > 0 ? o : 0;
  return w;
}

template <typename TA, int NT>
int launch_bwd(const BwdArgs<TA>& a, const FwdArgs<TA>& f, bool sp, bool gate, float* dA,
               float* dB, float* dC, float* dD, float* dbias, hipStream_t s) {
#define SSM_BWD_LAUNCH(KERN, GRID, BLOCK, ...)                                                 \
  do {                                                                                          \
    if (sp && gate) hipLaunchKernelGGL((KERN<TA, NT, true, true>), GRID, BLOCK, 0, s, __VA_ARGS__); \
    else if (sp) hipLaunchKernelGGL((KERN<TA, NT, true, false>), GRID, BLOCK, 0, s, __VA_ARGS__);   \
    else if (gate) hipLaunchKernelGGL((KERN<TA, NT, false, true>), GRID, BLOCK, 0, s, __VA_ARGS__); \
    else hipLaunchKernelGGL((KERN<TA, NT, false, false>), GRID, BLOCK, 0, s, __VA_ARGS__);          \
  } while (0)
  if (a.K > 1) {
    // 1-2. summaries of states and adjoints, then both carries in one launch
    const unsigned tiles = static_cast<unsigned>((a.dim + 63) / 64);
    const dim3 grid(2 * tiles, static_cast<unsigned>(a.K - 1), static_cast<unsigned>(a.batch));
    SSM_BWD_LAUNCH(bwd_sums_kernel, grid, dim3(64), a, f);
    launch_carry(f.A, CarryChain{f.h0, f.ws_S, f.ws_H}, CarryChain{a.dlast, a.rS, a.rH}, a.batch,
                 a.dim, NT, a.K, s);
  }
  // 3. main pass
  {
    const dim3 grid(static_cast<unsigned>(a.tiles), static_cast<unsigned>(a.K),
                    static_cast<unsigned>(a.batch));
    SSM_BWD_LAUNCH(bwd_main_kernel, grid, dim3(kBwdThreads), a);
  }
#undef SSM_BWD_LAUNCH
  // 4. reductions
  const int64_t per = a.batch * a.L * NT;
  hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3(static_cast<unsigned>((per + 255) / 256)), dim3(256),
                     0, s, a.pB, a.pC, dB, dC, per, a.tiles);
  const int64_t np = static_cast<int64_t>(a.dim) * NT + a.dim;
  hipLaunchKernelGGL(bwd_reduce_params_kernel,
                     dim3(static_cast<unsigned>((np + kRedElems - 1) / kRedElems)), dim3(256), 0,
                     s, a.pA, a.pD, a.pbias, dA, dD, dbias, a.dim, NT, a.batch * a.K);
  return launch_status("ssm_scan_bwd");
}

template <typename TA>
int dispatch_bwd(const BwdArgs<TA>& a, const FwdArgs<TA>& f, int N, bool sp, bool gate, float* dA,
                 float* dB, float* dC, float* dD, float* dbias, hipStream_t s) {
  switch (N) {
    case 4: return launch_bwd<TA, 4>(a, f, sp, gate, dA, dB, dC, dD, dbias, s);
    case 8: return launch_bwd<TA, 8>(a, f, sp, gate, dA, dB, dC, dD, dbias, s);
    default: return launch_bwd<TA, 16>(a, f, sp, gate, dA, dB, dC, dD, dbias, s);
  }
}

constexpr int64_t kBwdMaxDim = int64_t{1} << 24;
constexpr int64_t kBwdMaxLen = int64_t{65535} * kBwdStripe;  // stripes fill a grid dimension
constexpr int64_t kBwdMaxLanes = (int64_t{1} << 31) - 256;

}  // namespace ssm

using namespace ssm;

extern "C" {

size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                    int dtype) {
  (void)dtype;
  if (batch < 1 || batch > 65535 || dim < 1 || dim > kBwdMaxDim || seqlen < 0 ||
      seqlen > kBwdMaxLen || (dstate != 4 && dstate != 8 && dstate != 16) ||
      batch * seqlen * dstate > kBwdMaxLanes || batch * dim * dstate > kBwdMaxLanes)
    return 0;
  return bwd_layout(batch, seqlen, dim, dstate, plan_bwd(batch, seqlen, dim, dstate)).total;
}

int ssm_scan_bwd(const void* x, const void* delta, const float* delta_bias, int delta_softplus,
                 const float* A, const void* B, const void* C, const float* D_skip, const void* z,
                 const float* initial_state, const void* dout, const float* dlast_state, void* dx,
                 void* ddelta, void* dz, float* dA, float* dB, float* dC, float* dD,
                 float* ddelta_bias, float* dinitial_state, int64_t batch, int64_t seqlen,
                 int64_t dim, int64_t dstate, int dtype, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  clear_error();
  const char* fn = "ssm_scan_bwd";
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (delta_softplus != 0 && delta_softplus != 1)
    return fail(SSM_ERR_UNSUPPORTED, "%s: delta_softplus must be 0 or 1, got %d", fn,
                delta_softplus);
  if (dstate != 4 && dstate != 8 && dstate != 16)
    return fail(SSM_ERR_UNSUPPORTED, "%s: dstate must be 4, 8 or 16, got %lld", fn,
                (long long)dstate);
  if (batch < 1 || dim < 1 || seqlen < 0 || batch > 65535 || dim > kBwdMaxDim ||
      seqlen > kBwdMaxLen)
    return fail(SSM_ERR_SHAPE, "%s: bad sizes batch %lld, seqlen %lld, dim %lld", fn,
                (long long)batch, (long long)seqlen, (long long)dim);
  // the one-lane-per-element passes (dB/dC sums, the states of an empty call)
  if (batch * seqlen * dstate > kBwdMaxLanes || batch * dim * dstate > kBwdMaxLanes)
    return fail(SSM_ERR_SHAPE, "%s: batch %lld x (seqlen %lld or dim %lld) x dstate %lld exceeds "
                "one launch", fn, (long long)batch, (long long)seqlen, (long long)dim,
                (long long)dstate);
  if (!A || !dA) return fail(SSM_ERR_NULL, "%s: A and dA are required", fn);
  if (seqlen > 0 && (!x || !delta || !B || !C || !dout || !dx || !ddelta || !dB || !dC))
    return fail(SSM_ERR_NULL, "%s: x, delta, B, C, dout, dx, ddelta, dB and dC are required", fn);
  if (seqlen > 0 && z && !dz) return fail(SSM_ERR_NULL, "%s: dz is required with z", fn);
  if (D_skip == nullptr && dD != nullptr)
    return fail(SSM_ERR_NULL, "%s: dD given without D_skip", fn);
  const size_t es = dtype == SSM_DTYPE_F32 ? 4 : 2;
  const struct { const void* p; size_t k; const char* n; } al[] = {
      {x, es, "x"}, {delta, es, "delta"}, {z, es, "z"}, {dout, es, "dout"}, {dx, es, "dx"},
      {ddelta, es, "ddelta"}, {dz, es, "dz"}, {B, 4 * es, "B"}, {C, 4 * es, "C"}, {A, 4, "A"},
      {D_skip, 4, "D_skip"}, {delta_bias, 4, "delta_bias"}, {initial_state, 16, "initial_state"},
      {dlast_state, 16, "dlast_state"}, {dA, 4, "dA"}, {dB, 16, "dB"}, {dC, 16, "dC"},
      {dD, 4, "dD"}, {ddelta_bias, 4, "ddelta_bias"}, {dinitial_state, 16, "dinitial_state"}};
  for (const auto& e : al)
    if (e.p && !aligned(e.p, e.k))
      return fail(SSM_ERR_ALIGN, "%s: %s is not %zu-byte aligned", fn, e.n, e.k);
  const size_t tok = static_cast<size_t>(batch) * seqlen * dim * es;
  const size_t bc = static_cast<size_t>(batch) * seqlen * dstate * es;
  const size_t bc32 = static_cast<size_t>(batch) * seqlen * dstate * 4;
  const size_t st = static_cast<size_t>(batch) * dim * dstate * 4;
  const size_t pd = static_cast<size_t>(dim) * 4;
  const Span ins[] = {{x, tok, "x"}, {delta, tok, "delta"}, {z, z ? tok : 0, "z"},
                      {dout, tok, "dout"}, {B, bc, "B"}, {C, bc, "C"},
                      {A, static_cast<size_t>(dim) * dstate * 4, "A"},
                      {D_skip, D_skip ? pd : 0, "D_skip"},
                      {delta_bias, delta_bias ? pd : 0, "delta_bias"},
                      {initial_state, initial_state ? st : 0, "initial_state"},
                      {dlast_state, dlast_state ? st : 0, "dlast_state"}};
  const Span outs[] = {{dx, tok, "dx"}, {ddelta, tok, "ddelta"}, {dz, dz ? tok : 0, "dz"},
                       {dA, static_cast<size_t>(dim) * dstate * 4, "dA"}, {dB, bc32, "dB"},
                       {dC, bc32, "dC"}, {dD, dD ? pd : 0, "dD"},
                       {ddelta_bias, ddelta_bias ? pd : 0, "ddelta_bias"},
                       {dinitial_state, dinitial_state ? st : 0, "dinitial_state"}};
  for (const auto& o : outs)
    for (const auto& i : ins)
      if (overlap(o, i))
        return fail(SSM_ERR_ALIAS, "%s: output %s overlaps input %s", fn, o.name, i.name);
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i)
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlap(outs[i], outs[j]))
        return fail(SSM_ERR_ALIAS, "%s: outputs %s and %s overlap", fn, outs[i].name, outs[j].name);
  const BwdPlan plan = plan_bwd(batch, seqlen, dim, dstate);
  const BwdWs ws = bwd_layout(batch, seqlen, dim, dstate, plan);
  if (workspace_bytes < ws.total || (ws.total > 0 && !workspace))
    return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, ws.total,
                workspace_bytes);
  if (ws.total > 0 && !aligned(workspace, 256))
    return fail(SSM_ERR_ALIGN, "%s: workspace is not 256-byte aligned", fn);
  const Span wsp{workspace, ws.total, "workspace"};
  for (const auto& i : ins)
    if (overlap(wsp, i)) return fail(SSM_ERR_ALIAS, "%s: workspace overlaps input %s", fn, i.name);
  for (const auto& o : outs)
    if (overlap(wsp, o)) return fail(SSM_ERR_ALIAS, "%s: workspace overlaps output %s", fn, o.name);

  if (seqlen == 0) {
    const int64_t n = static_cast<int64_t>(batch) * dim * dstate;
    hipLaunchKernelGGL(bwd_empty_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                       0, stream, dlast_state, dinitial_state, n, dA, dD, ddelta_bias,
                       static_cast<int>(dim), static_cast<int>(dstate));
    return launch_status(fn);
  }
  char* w = static_cast<char*>(workspace);
  const int K = plan.K;
  auto wf = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  const bool sp = delta_softplus != 0, gate = z != nullptr;
  if (dtype == SSM_DTYPE_F32) {
    FwdArgs<float> f{static_cast<const float*>(x), static_cast<const float*>(delta), delta_bias, A,
                     static_cast<const float*>(B), static_cast<const float*>(C), D_skip, nullptr,
                     nullptr, nullptr, initial_state, wf(ws.fS), wf(ws.fH), nullptr, nullptr, 0,
                     static_cast<int>(seqlen), plan.Ls, K, static_cast<int>(dim),
                     static_cast<int>(dstate)};
    BwdArgs<float> a{static_cast<const float*>(x), static_cast<const float*>(delta), delta_bias,
                     A, static_cast<const float*>(B), static_cast<const float*>(C), D_skip,
                     static_cast<const float*>(z), initial_state, static_cast<const float*>(dout),
                     dlast_state, static_cast<float*>(dx), static_cast<float*>(ddelta),
                     static_cast<float*>(dz), dinitial_state, wf(ws.fH), wf(ws.rS), wf(ws.rH),
                     wf(ws.pB), wf(ws.pC), wf(ws.pA), wf(ws.pD), wf(ws.pbias), batch,
                     static_cast<int>(seqlen), plan.Ls, K, static_cast<int>(dim), plan.tiles};
    return dispatch_bwd(a, f, static_cast<int>(dstate), sp, gate, dA, dB, dC, dD, ddelta_bias,
                        stream);
  }
  FwdArgs<bf16_t> f{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(delta), delta_bias, A,
                    static_cast<const bf16_t*>(B), static_cast<const bf16_t*>(C), D_skip, nullptr,
                    nullptr, nullptr, initial_state, wf(ws.fS), wf(ws.fH), nullptr, nullptr, 0,
                    static_cast<int>(seqlen), plan.Ls, K, static_cast<int>(dim),
                    static_cast<int>(dstate)};
  BwdArgs<bf16_t> a{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(delta), delta_bias,
                    A, static_cast<const bf16_t*>(B), static_cast<const bf16_t*>(C), D_skip,
                    static_cast<const bf16_t*>(z), initial_state, static_cast<const bf16_t*>(dout),
                    dlast_state, static_cast<bf16_t*>(dx), static_cast<bf16_t*>(ddelta),
                    static_cast<bf16_t*>(dz), dinitial_state, wf(ws.fH), wf(ws.rS), wf(ws.rH),
                    wf(ws.pB), wf(ws.pC), wf(ws.pA), wf(ws.pD), wf(ws.pbias), batch,
                    static_cast<int>(seqlen), plan.Ls, K, static_cast<int>(dim), plan.tiles};
  return dispatch_bwd(a, f, static_cast<int>(dstate), sp, gate, dA, dB, dC, dD, ddelta_bias,
                      stream);
}

}  // extern "C"
