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
// accumulation.  One workgroup (4 waves) owns one (b, h, segment of
// chunks) and walks its chunks in order; the float32 state lives in the
// MFMA accumulators of the four waves (no per-chunk states in memory).  Per
// chunk the operands are staged in LDS: C and B row-major, x transposed,
// the masked S, and a bf16 copy of the state.  When (b, h) pairs alone do
// not fill the chip, the sequence is cut into segments: a state pass runs
// each segment but the last from zero (state update only), a carry pass
// chains the segments' end states, and the output pass starts every
// segment from its entering state.
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
  float* seg_state;  // (batch, nseg, H, P, N): end state of segment s (state pass), then
                     // (after the carry) the state entering segment s
  float* seg_lam;    // (batch, nseg, H): sum of dt A over segment s
  int L;
  int H;
  int G;
  int softplus;
  int cps;   // chunks per segment
  int nseg;
};

__device__ __forceinline__ __bf16 to_bf(float v) { return static_cast<__bf16>(v); }
__device__ __forceinline__ float from_bf(__bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float exp_f(float v) { return __builtin_amdgcn_exp2f(v * kLog2e); }

// Row/column of accumulator element r of this lane within a 32x32 tile.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r / 4) + 4 * (lane / 32) + (r % 4); }

// FULL: outputs (and the last segment's final state); otherwise the state
// pass: only the state update, from zero, leaving the segment's end state
// and total log-decay for the carry.  Block (head, segment, sequence).
template <int NS, bool GATE, bool FULL>
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
  const int seg = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int L = a.L, H = a.H;
  const int g = h / (H / a.G);
  const float Ah = a.A[h];
  const float Dh = a.D ? a.D[h] : 0.0f;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;

  // the state: tiles k = wave*TPW + i, rows p in 32*(k / NCT), columns n in 32*(k % NCT);
  // it enters the segment from the carry (or the initial state), or from
  // zero in the state pass
  const size_t slot = ((static_cast<size_t>(b) * a.nseg + seg) * H + h) * P * NS;
  const float* hin = !FULL ? nullptr : (a.nseg > 1 ? a.seg_state + slot : a.h0 ? a.h0 + (b * H + h) * P * NS : nullptr);
  f32x16 st[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int k = wave * TPW + i, rt = k / NCT, ct = k % NCT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = 32 * rt + acc_row(r, lane), n = 32 * ct + l32;
      st[i][r] = hin ? hin[p * NS + n] : 0.0f;
    }
  }

  const int nchunks = (L + Q - 1) / Q;
  const int c_begin = seg * a.cps;
  const int c_end = (c_begin + a.cps < nchunks) ? c_begin + a.cps : nchunks;
  float lam_seg = 0.0f;

  // The global inputs of a chunk are fetched into registers one chunk ahead,
  // so their latency is covered by the current chunk's work; rows past the
  // sequence read as zeros.  x is fetched token-fastest across lanes (each
  // lane 8 channels of one token) so that its transposed LDS copy is written
  // without bank conflicts.
  constexpr int VR = NS / 8;                    // 16-byte vectors per B/C row
  constexpr int NBC = Q * VR / kSsdThreads;     // B (and C) vectors per thread
  constexpr int NX = Q * P / 8 / kSsdThreads;   // x vectors per thread
  uint4 pb[NBC], pc[NBC];
  bf16x8 px[NX];
  float pdt = 0.0f;
  uint16_t pz[16];
  const int yrt = wave / 2, yct = wave % 2;     // this wave's output tile
  auto fetch = [&](int c) {
    const int t0 = c * Q;
#pragma unroll
    for (int j = 0; j < NBC; ++j) {
      const int v = tid + kSsdThreads * j;
      const int t = v / VR, n8 = v % VR;
      pb[j] = make_uint4(0, 0, 0, 0);
      pc[j] = make_uint4(0, 0, 0, 0);
      if (t0 + t < L) {
        const size_t row = ((b * L + t0 + t) * a.G + g) * NS + 8 * n8;
        pb[j] = *reinterpret_cast<const uint4*>(a.B + row);
        if (FULL) pc[j] = *reinterpret_cast<const uint4*>(a.C + row);
      }
    }
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int v = tid + kSsdThreads * j;
      const int t = v % Q, p8 = v / Q;
      px[j] = bf16x8{};
      if (t0 + t < L) px[j] = *reinterpret_cast<const bf16x8*>(a.x + ((b * L + t0 + t) * H + h) * P + 8 * p8);
    }
    if (tid < Q) {
      pdt = 0.0f;
      if (t0 + tid < L) {
        const float u = to_f32(a.dt[(b * L + t0 + tid) * H + h]) + bias;
        pdt = a.softplus ? softplus_f32(u) : u;
      }
    }
    if constexpr (FULL && GATE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = t0 + 32 * yrt + acc_row(r, lane);
        pz[r] = 0;
        if (tok < L) pz[r] = a.z[((b * L + tok) * H + h) * P + 32 * yct + l32].bits;
      }
    }
  };
  if (c_begin < c_end) fetch(c_begin);

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * Q;
    // ---- 1. stage the chunk fetched ahead, then fetch the next ----
#pragma unroll
    for (int j = 0; j < NBC; ++j) {
      const int v = tid + kSsdThreads * j;
      const int t = v / VR, n8 = v % VR;
      *reinterpret_cast<uint4*>(&sB[t * LDC + 8 * n8]) = pb[j];
      if (FULL) *reinterpret_cast<uint4*>(&sC[t * LDC + 8 * n8]) = pc[j];
    }
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int v = tid + kSsdThreads * j;
      const int t = v % Q, p8 = v / Q;
#pragma unroll
      for (int i = 0; i < 8; ++i) sXt[(8 * p8 + i) * LDX + t] = px[j][i];
    }
    if (tid < Q) sdt[tid] = pdt;
    uint16_t zc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) zc[r] = pz[r];
    if (c + 1 < c_end) fetch(c + 1);
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
    lam_seg += lam_end;
    if (tid < Q) sw[tid] = sdt[tid] * exp_f(lam_end - slam[tid]);
    if constexpr (!FULL) __syncthreads();  // (the full pass has barriers before sw is read)

    if constexpr (FULL) {
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
          if constexpr (GATE) y *= silu_f32(__uint_as_float(static_cast<uint32_t>(zc[r]) << 16));
          store_act(a.out + o, y);
        }
      }
    }
    }  // FULL

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

  // the state pass leaves its segment's end state; the full pass of the
  // last segment leaves the final state
  float* dst = !FULL ? a.seg_state + slot
                     : (seg == a.nseg - 1 && a.last_state ? a.last_state + (b * H + h) * P * NS
                                                          : nullptr);
  if (dst) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int k = wave * TPW + i, rt = k / NCT, ct = k % NCT;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = 32 * rt + acc_row(r, lane), n = 32 * ct + l32;
        dst[p * NS + n] = st[i][r];
      }
    }
  }
  if (!FULL && tid == 0) a.seg_lam[(static_cast<size_t>(b) * a.nseg + seg) * H + h] = lam_seg;
}

// Carry over segments: one lane per (sequence, head, p, n).  h runs from the
// initial state through the segments' end states, h <- e^(lambda_s) h + H_s,
// and each slot is overwritten with the state entering that segment.
__global__ void __launch_bounds__(256) ssd_carry_kernel(SsdArgs a, int PN) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_b = static_cast<int64_t>(a.H) * PN;
  if (idx >= per_b) return;
  const int64_t b = blockIdx.y;
  const int h = static_cast<int>(idx / PN);
  const int e = static_cast<int>(idx % PN);
  float hv = a.h0 ? a.h0[(b * a.H + h) * PN + e] : 0.0f;
  for (int s = 0; s < a.nseg; ++s) {
    float* sp = a.seg_state + ((b * a.nseg + s) * a.H + h) * static_cast<int64_t>(PN) + e;
    const float Hs = (s < a.nseg - 1) ? *sp : 0.0f;
    *sp = hv;
    if (s < a.nseg - 1) {
      float unused;
      hv = __builtin_fmaf(exp_acc(a.seg_lam[(b * a.nseg + s) * a.H + h], unused), hv, Hs);
    }
  }
}

struct SsdPlan {
  int cps, nseg;
};

// Segments: enough (head, segment, sequence) workgroups for about four per
// compute unit, at least two chunks per segment.
SsdPlan plan_ssd(int64_t batch, int64_t L, int64_t H) {
  const int64_t nchunks = (L + kSsdQ - 1) / kSsdQ;
  const int64_t target = 4LL * device_cus();
  int64_t nseg = (target + batch * H - 1) / (batch * H);
  if (nseg > nchunks / 2) nseg = nchunks / 2;
  if (nseg < 1) nseg = 1;
  int64_t cps = (nchunks + nseg - 1) / nseg;
  if (cps < 1) cps = 1;
  nseg = nchunks > 0 ? (nchunks + cps - 1) / cps : 1;
  return SsdPlan{static_cast<int>(cps), static_cast<int>(nseg)};
}

size_t ssd_workspace(int64_t batch, int64_t H, int64_t P, int64_t N, const SsdPlan& p) {
  if (p.nseg <= 1) return 0;
  const size_t states = static_cast<size_t>(batch) * p.nseg * H * P * N * 4;
  return (states + 255) / 256 * 256 + static_cast<size_t>(batch) * p.nseg * H * 4;
}

}  // namespace ssm

using namespace ssm;

extern "C" {

size_t ssm_ssd_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int64_t ngroups) {
  (void)ngroups;
  if (batch < 1 || batch > 65535 || seqlen < 0 || seqlen > (int64_t{1} << 30) || nheads < 1 ||
      nheads > 65535 || headdim != kSsdP || (dstate != 64 && dstate != 128))
    return 0;
  return ssd_workspace(batch, nheads, headdim, dstate, plan_ssd(batch, seqlen, nheads));
}

int ssm_ssd_fwd(const void* x, const void* dt, const float* dt_bias, int dt_softplus,
                const float* A, const void* B, const void* C, const float* D, const void* z,
                void* out, float* last_state, const float* initial_state, int64_t batch,
                int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
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
  const SsdPlan plan = plan_ssd(batch, seqlen, nheads);
  const size_t need = ssd_workspace(batch, nheads, headdim, dstate, plan);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace_bytes);
  if (need > 0 && !aligned(workspace, 256))
    return fail(SSM_ERR_ALIGN, "%s: workspace is not 256-byte aligned", fn);
  const Span wsp{workspace, need, "workspace"};
  for (const auto& i : ins)
    if (overlap(wsp, i)) return fail(SSM_ERR_ALIAS, "%s: workspace overlaps input %s", fn, i.name);
  for (const auto& o : outs)
    if (overlap(wsp, o)) return fail(SSM_ERR_ALIAS, "%s: workspace overlaps output %s", fn, o.name);
  if (seqlen == 0 && !last_state) return SSM_OK;
  const size_t sbytes = static_cast<size_t>(batch) * plan.nseg * nheads * headdim * dstate * 4;
  float* seg_state = need ? static_cast<float*>(workspace) : nullptr;
  float* seg_lam = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                   (sbytes + 255) / 256 * 256)
                        : nullptr;
  SsdArgs args{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(dt), dt_bias, A,
               static_cast<const bf16_t*>(B), static_cast<const bf16_t*>(C), D,
               static_cast<const bf16_t*>(z), static_cast<bf16_t*>(out), last_state,
               initial_state, seg_state, seg_lam, static_cast<int>(seqlen),
               static_cast<int>(nheads), static_cast<int>(ngroups), dt_softplus, plan.cps,
               plan.nseg};
  const dim3 block(kSsdThreads);
  const bool big = dstate == 128;
  if (plan.nseg > 1) {
    // state pass over every segment but the last, then the carry
    const dim3 g1(static_cast<unsigned>(nheads), static_cast<unsigned>(plan.nseg - 1),
                  static_cast<unsigned>(batch));
    if (big) hipLaunchKernelGGL((ssd_fwd_kernel<128, false, false>), g1, block, 0, stream, args);
    else hipLaunchKernelGGL((ssd_fwd_kernel<64, false, false>), g1, block, 0, stream, args);
    const int PN = static_cast<int>(headdim * dstate);
    const int64_t lanes = nheads * PN;
    hipLaunchKernelGGL(ssd_carry_kernel,
                       dim3(static_cast<unsigned>((lanes + 255) / 256), static_cast<unsigned>(batch)),
                       dim3(256), 0, stream, args, PN);
  }
  const dim3 grid(static_cast<unsigned>(nheads), static_cast<unsigned>(plan.nseg),
                  static_cast<unsigned>(batch));
  if (big) {
    if (z) hipLaunchKernelGGL((ssd_fwd_kernel<128, true, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((ssd_fwd_kernel<128, false, true>), grid, block, 0, stream, args);
  } else {
    if (z) hipLaunchKernelGGL((ssd_fwd_kernel<64, true, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((ssd_fwd_kernel<64, false, true>), grid, block, 0, stream, args);
  }
  return launch_status(fn);
}

}  // extern "C"
