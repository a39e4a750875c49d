// ssd.hip -- the state space dual (SSD, Mamba-2) form of the selective scan
// on MFMA, for MI355X (gfx950), behind the C ABI in include/ssm_scan.h (see
// there for the citation and the definition).
//
// With one scalar decay per head the sequence map is 1-semiseparable, so a
// chunk of Q tokens is computed by matrix products (per sequence b, head h,
// with lambda_t = sum of dt A over the chunk up to t):
//   S      = (C B^T) o mask,  mask[t,s] = e^(lambda_t - lambda_s) dt_s for s <= t
//   Y      = S X + diag(e^lambda) (C h^T) + D X,  then the gate
//   h     <- e^(lambda_end) h + X_w^T B,  X_w[s,:] = X[s,:] dt_s e^(lambda_end - lambda_s)
// where h (headdim x dstate) is the state entering the chunk.  The four
// products are bf16 MFMA (v_mfma_f32_32x32x16_bf16) with float32
// accumulation.  One workgroup (4 waves) owns one (b, h) and walks its
// chunks in order; the float32 state lives in the MFMA accumulators of the
// four waves for the whole sequence (no chunk states in memory, no carry
// pass).  Per chunk the operands are staged in LDS: C and B row-major, x
// transposed, the masked S, and a bf16 copy of the state.
//
// MFMA operand layout (32x32x16 bf16; checked on the device): lane l holds
// A[l%32][8*(l/32) + i] and B[8*(l/32) + i][l%32], i = 0..7; accumulator
// element r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_scan.h"

#include "host_util.hpp"
#include "kernels.hpp"

namespace ssm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kSsdQ = 64;        // chunk length (tokens)
constexpr int kSsdP = 64;        // head dimension
constexpr int kSsdThreads = 256;  // 4 waves
constexpr int kSsdPad = 8;       // LDS row padding (bf16 elements)

struct SsdArgs {
  const bf16_t* x;
  const bf16_t* dt;
  const float* dt_bias;
  const float* A;
  const bf16_t* B;
  const bf16_t* C;
  const float* D;
  const bf16_t* z;
  bf16_t* out;
  float* last_state;
  const float* h0;
  int L;
  int H;
  int G;
  int softplus;
};

__device__ __forceinline__ __bf16 to_bf(float v) { return static_cast<__bf16>(v); }
__device__ __forceinline__ float from_bf(__bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float exp_f(float v) { return __builtin_amdgcn_exp2f(v * kLog2e); }

// Row/column of accumulator element r of this lane within a 32x32 tile.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r / 4) + 4 * (lane / 32) + (r % 4); }

template <int NS, bool GATE>
__global__ void __launch_bounds__(kSsdThreads) ssd_fwd_kernel(SsdArgs a) {
  constexpr int Q = kSsdQ, P = kSsdP;
  constexpr int LDC = NS + kSsdPad;  // sC, sB, sH row stride
  constexpr int LDX = Q + kSsdPad;   // sXt, sS row stride
  constexpr int NCT = NS / 32;       // column tiles of the state
  constexpr int TPW = 2 * NCT / 4;   // state tiles per wave
  __shared__ __attribute__((aligned(16))) __bf16 sC[Q * LDC];
  __shared__ __attribute__((aligned(16))) __bf16 sB[Q * LDC];
  __shared__ __attribute__((aligned(16))) __bf16 sH[P * LDC];
  __shared__ __attribute__((aligned(16))) __bf16 sXt[P * LDX];
  __shared__ __attribute__((aligned(16))) __bf16 sS[Q * LDX];
  __shared__ float sdt[Q], slam[Q], sw[Q];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane % 32, hi8 = 8 * (lane / 32);
  const int h = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int L = a.L, H = a.H;
  const int g = h / (H / a.G);
  const float Ah = a.A[h];
  const float Dh = a.D ? a.D[h] : 0.0f;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;

  // the state: tiles k = wave*TPW + i, rows p in 32*(k / NCT), columns n in 32*(k % NCT)
  f32x16 st[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int k = wave * TPW + i, rt = k / NCT, ct = k % NCT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = 32 * rt + acc_row(r, lane), n = 32 * ct + l32;
      st[i][r] = a.h0 ? a.h0[((b * H + h) * P + p) * NS + n] : 0.0f;
    }
  }

  const int nchunks = (L + Q - 1) / Q;
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * Q;
    // ---- 1. stage the chunk (rows past the sequence are zeros) ----
    constexpr int VR = NS / 8;  // 16-byte vectors per B/C row
#pragma unroll
    for (int j = 0; j < Q * VR / kSsdThreads; ++j) {
      const int v = tid + kSsdThreads * j;
      const int t = v / VR, n8 = v % VR;
      uint4 qb = make_uint4(0, 0, 0, 0), qc = make_uint4(0, 0, 0, 0);
      if (t0 + t < L) {
        const size_t row = ((b * L + t0 + t) * a.G + g) * NS + 8 * n8;
        qb = *reinterpret_cast<const uint4*>(a.B + row);
        qc = *reinterpret_cast<const uint4*>(a.C + row);
      }
      *reinterpret_cast<uint4*>(&sB[t * LDC + 8 * n8]) = qb;
      *reinterpret_cast<uint4*>(&sC[t * LDC + 8 * n8]) = qc;
    }
#pragma unroll
    for (int j = 0; j < Q * P / 8 / kSsdThreads; ++j) {
      const int v = tid + kSsdThreads * j;
      const int t = v / (P / 8), p8 = v % (P / 8);
      bf16x8 q = {};
      if (t0 + t < L) q = *reinterpret_cast<const bf16x8*>(a.x + ((b * L + t0 + t) * H + h) * P + 8 * p8);
#pragma unroll
      for (int i = 0; i < 8; ++i) sXt[(8 * p8 + i) * LDX + t] = q[i];
    }
    if (tid < Q) {
      float d = 0.0f;
      if (t0 + tid < L) {
        const float u = to_f32(a.dt[(b * L + t0 + tid) * H + h]) + bias;
        d = a.softplus ? softplus_f32(u) : u;
      }
      sdt[tid] = d;
    }
    __syncthreads();
    if (wave == 0) {  // lambda: inclusive prefix sum of dt A over the chunk
      float v = sdt[lane] * Ah;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float u = __shfl_up(v, o);
        if (lane >= o) v += u;
      }
      slam[lane] = v;
    }
    __syncthreads();
    const float lam_end = slam[Q - 1];
    if (tid < Q) sw[tid] = sdt[tid] * exp_f(lam_end - slam[tid]);

    // ---- 2. S = C B^T, masked: tile (rows t in 32*(wave/2), columns s in 32*(wave%2)) ----
    {
      const int rt = wave / 2, ct = wave % 2;
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < NS / 16; ++kk) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sC[(32 * rt + l32) * LDC + 16 * kk + hi8]);
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&sB[(32 * ct + l32) * LDC + 16 * kk + hi8]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
      }
      const int s = 32 * ct + l32;
      const float lam_s = slam[s], dt_s = sdt[s];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * rt + acc_row(r, lane);
        const float v = (s <= t) ? acc[r] * exp_f(slam[t] - lam_s) * dt_s : 0.0f;
        sS[t * LDX + s] = to_bf(v);
      }
    }
    // ---- 3. bf16 copy of the state entering the chunk ----
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int k = wave * TPW + i, rt = k / NCT, ct = k % NCT;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sH[(32 * rt + acc_row(r, lane)) * LDC + 32 * ct + l32] = to_bf(st[i][r]);
    }
    __syncthreads();

    // ---- 4. Y = S X + diag(e^lambda) (C h^T) + D X: tile (t in 32*(wave/2), p in 32*(wave%2)) ----
    {
      const int rt = wave / 2, ct = wave % 2;
      f32x16 y1 = {}, y2 = {};
#pragma unroll
      for (int kk = 0; kk < Q / 16; ++kk) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sS[(32 * rt + l32) * LDX + 16 * kk + hi8]);
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&sXt[(32 * ct + l32) * LDX + 16 * kk + hi8]);
        y1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, y1, 0, 0, 0);
      }
#pragma unroll
      for (int kk = 0; kk < NS / 16; ++kk) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sC[(32 * rt + l32) * LDC + 16 * kk + hi8]);
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&sH[(32 * ct + l32) * LDC + 16 * kk + hi8]);
        y2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, y2, 0, 0, 0);
      }
      const int p = 32 * ct + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * rt + acc_row(r, lane);
        const int tok = t0 + t;
        if (tok < L) {
          const float xv = from_bf(sXt[p * LDX + t]);
          float y = __builtin_fmaf(exp_f(slam[t]), y2[r], y1[r]);
          y = __builtin_fmaf(Dh, xv, y);
          const size_t o = ((b * L + tok) * H + h) * P + p;
          if constexpr (GATE) y *= silu_f32(to_f32(a.z[o]));
          store_act(a.out + o, y);
        }
      }
    }

    // ---- 5. h <- e^(lambda_end) h + X_w^T B ----
    {
      const float aend = exp_f(lam_end);
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int k = wave * TPW + i, rt = k / NCT, ct = k % NCT;
#pragma unroll
        for (int r = 0; r < 16; ++r) st[i][r] *= aend;
        const int p = 32 * rt + l32, n = 32 * ct + l32;
#pragma unroll
        for (int kk = 0; kk < Q / 16; ++kk) {
          const int s0 = 16 * kk + hi8;
          const bf16x8 xv = *reinterpret_cast<const bf16x8*>(&sXt[p * LDX + s0]);
          bf16x8 av, bv;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            av[j] = to_bf(from_bf(xv[j]) * sw[s0 + j]);
            bv[j] = sB[(s0 + j) * LDC + n];
          }
          st[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, st[i], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the next chunk restages every LDS buffer
  }

  if (a.last_state) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int k = wave * TPW + i, rt = k / NCT, ct = k % NCT;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = 32 * rt + acc_row(r, lane), n = 32 * ct + l32;
        a.last_state[((b * H + h) * P + p) * NS + n] = st[i][r];
      }
    }
  }
}

}  // namespace ssm

using namespace ssm;

extern "C" {

int ssm_ssd_fwd(const void* x, const void* dt, const float* dt_bias, int dt_softplus,
                const float* A, const void* B, const void* C, const float* D, const void* z,
                void* out, float* last_state, const float* initial_state, int64_t batch,
                int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                int dtype, hipStream_t stream) {
  clear_error();
  const char* fn = "ssm_ssd_fwd";
  if (dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "%s: only bf16 activations (dtype %d) are supported", fn,
                SSM_DTYPE_BF16);
  if (dt_softplus != 0 && dt_softplus != 1)
    return fail(SSM_ERR_UNSUPPORTED, "%s: dt_softplus must be 0 or 1", fn);
  if (headdim != kSsdP || (dstate != 64 && dstate != 128))
    return fail(SSM_ERR_UNSUPPORTED, "%s: needs headdim 64 and dstate 64 or 128 (got %lld, %lld)",
                fn, (long long)headdim, (long long)dstate);
  if (batch < 1 || batch > 65535 || seqlen < 0 || seqlen > (int64_t{1} << 30) || nheads < 1 ||
      nheads > 65535 || ngroups < 1 || nheads % ngroups != 0)
    return fail(SSM_ERR_SHAPE, "%s: bad sizes batch %lld, seqlen %lld, nheads %lld, ngroups %lld",
                fn, (long long)batch, (long long)seqlen, (long long)nheads, (long long)ngroups);
  if (!A) return fail(SSM_ERR_NULL, "%s: A is required", fn);
  if (seqlen > 0 && (!x || !dt || !B || !C || !out))
    return fail(SSM_ERR_NULL, "%s: x, dt, B, C and out are required", fn);
  const struct { const void* p; size_t k; const char* n; } al[] = {
      {x, 16, "x"}, {B, 16, "B"}, {C, 16, "C"}, {dt, 2, "dt"}, {z, 2, "z"}, {out, 2, "out"},
      {A, 4, "A"}, {D, 4, "D"}, {dt_bias, 4, "dt_bias"}, {last_state, 4, "last_state"},
      {initial_state, 4, "initial_state"}};
  for (const auto& e : al)
    if (e.p && !aligned(e.p, e.k))
      return fail(SSM_ERR_ALIGN, "%s: %s is not %zu-byte aligned", fn, e.n, e.k);
  const size_t tok = static_cast<size_t>(batch) * seqlen * nheads * headdim * 2;
  const size_t bc = static_cast<size_t>(batch) * seqlen * ngroups * dstate * 2;
  const size_t st = static_cast<size_t>(batch) * nheads * headdim * dstate * 4;
  const size_t ph = static_cast<size_t>(nheads) * 4;
  const Span ins[] = {{x, tok, "x"}, {dt, static_cast<size_t>(batch) * seqlen * nheads * 2, "dt"},
                      {z, z ? tok : 0, "z"}, {B, bc, "B"}, {C, bc, "C"}, {A, ph, "A"},
                      {D, D ? ph : 0, "D"}, {dt_bias, dt_bias ? ph : 0, "dt_bias"},
                      {initial_state, initial_state ? st : 0, "initial_state"}};
  const Span outs[] = {{out, tok, "out"}, {last_state, last_state ? st : 0, "last_state"}};
  for (const auto& o : outs)
    for (const auto& i : ins) {
      if (o.p == last_state && i.p == initial_state && o.p == i.p) continue;  // resume in place
      if (overlap(o, i))
        return fail(SSM_ERR_ALIAS, "%s: output %s overlaps input %s", fn, o.name, i.name);
    }
  if (overlap(outs[0], outs[1])) return fail(SSM_ERR_ALIAS, "%s: out overlaps last_state", fn);
  if (seqlen == 0 && !last_state) return SSM_OK;
  SsdArgs args{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(dt), dt_bias, A,
               static_cast<const bf16_t*>(B), static_cast<const bf16_t*>(C), D,
               static_cast<const bf16_t*>(z), static_cast<bf16_t*>(out), last_state,
               initial_state, static_cast<int>(seqlen), static_cast<int>(nheads),
               static_cast<int>(ngroups), dt_softplus};
  const dim3 grid(static_cast<unsigned>(nheads), static_cast<unsigned>(batch));
  const dim3 block(kSsdThreads);
  if (dstate == 128) {
    if (z) hipLaunchKernelGGL((ssd_fwd_kernel<128, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((ssd_fwd_kernel<128, false>), grid, block, 0, stream, args);
  } else {
    if (z) hipLaunchKernelGGL((ssd_fwd_kernel<64, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((ssd_fwd_kernel<64, false>), grid, block, 0, stream, args);
  }
  return launch_status(fn);
}

}  // extern "C"
