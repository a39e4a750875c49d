// rates.hip -- gfx950 rate microbenchmarks behind the roofline figures:
// vector fp32 FMA / MUL and v_exp_f32 issue rates at several occupancies and
// by operand kind (an SGPR operand vs VGPR operands only), the scan's
// per-state step with the token's B/C values read from SGPRs, from VGPRs or
// through a DPP row broadcast, LDS access patterns of the SSD kernel's B/C
// rows (bank conflicts: the 64 banks of 4 bytes, 256 bytes per cycle), and
// HBM streaming rates (copy, read, in-place update) on buffers larger than
// the MALL.  Standalone executable; prints one line per measurement.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <utility>

#define CK(x)                                                                          \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);      \
      std::exit(1);                                                                    \
    }                                                                                  \
  } while (0)

template <int CH>
__global__ void __launch_bounds__(256) k_fma(float* out, int iters, float a, float b) {
  float v[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) v[i] = 1e-3f * (i + threadIdx.x);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < CH; ++i) v[i] = __builtin_fmaf(v[i], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i) s += v[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// as k_fma with the multiplier and addend in per-lane registers (VGPRs)
template <int CH>
__global__ void __launch_bounds__(256) k_fma_v(float* out, int iters, float a, float b) {
  float v[CH];
  const float va = a + 1e-9f * threadIdx.x, vb = b + 1e-9f * threadIdx.x;
#pragma unroll
  for (int i = 0; i < CH; ++i) v[i] = 1e-3f * (i + threadIdx.x);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < CH; ++i) v[i] = __builtin_fmaf(v[i], va, vb);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i) s += v[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The scan's per-state step over 16 states, per token: decay chain
// d <- d*r, h <- d*h + (x*b), y <- y + c*h, with the token's b/c read
//   SRC 0: from SGPRs (scalar loads of a row per token, as the scan does),
//   SRC 1: from VGPRs (per-lane constants: no load, the bound without SGPRs),
//   SRC 2: from lanes 0-15 of a VGPR through DPP row_newbcast.
// The asm barrier keeps x*b a separate multiply, as in the scan.
typedef const __attribute__((address_space(4))) float mb_cfloat_t;
constexpr int kMixStates = 16, kMixTokens = 1024;
template <int n>
__device__ __forceinline__ float mb_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + n,
                                                               0xF, 0xF, false));
}
template <int SRC, int n>
__device__ __forceinline__ void mb_state(float (&h)[kMixStates], const float (&vb)[kMixStates],
                                         const float (&vc)[kMixStates], mb_cfloat_t* q, float lb,
                                         float lc, float x, float r, float& d, float& y) {
  float b, c;
  if constexpr (SRC == 0) { b = q[n]; c = q[kMixStates + n]; }
  if constexpr (SRC == 1) { b = vb[n]; c = vc[n]; }
  if constexpr (SRC == 2) { b = mb_bcast<n>(lb); c = mb_bcast<n>(lc); }
  float u = x * b;
  __asm__ volatile("" : "+v"(u));
  h[n] = __builtin_fmaf(d, h[n], u);
  y = __builtin_fmaf(c, h[n], y);
  d *= r;
}
template <int SRC, int... ns>
__device__ __forceinline__ void mb_states(std::integer_sequence<int, ns...>, float (&h)[kMixStates],
                                          const float (&vb)[kMixStates], const float (&vc)[kMixStates],
                                          mb_cfloat_t* q, float lb, float lc, float x, float r, float& d,
                                          float& y) {
  (mb_state<SRC, ns>(h, vb, vc, q, lb, lc, x, r, d, y), ...);
}
template <int SRC>
__global__ void __launch_bounds__(256) k_step(float* out, const float* bc) {
  float h[kMixStates], vb[kMixStates], vc[kMixStates];
#pragma unroll
  for (int n = 0; n < kMixStates; ++n) {
    h[n] = 0.f;
    vb[n] = 0.01f * n + 1e-7f * threadIdx.x;
    vc[n] = 0.02f * n - 1e-7f * threadIdx.x;
  }
  float x = 0.3f + 1e-6f * threadIdx.x, r = 0.97f + 1e-8f * threadIdx.x, acc = 0.f;
  const int lane = threadIdx.x & 63;
  for (int t = 0; t < kMixTokens; ++t) {
    const float* g = bc + (t & 63) * 2 * kMixStates;  // 64 rows of b then c
    float lb = 0.f, lc = 0.f;
    if constexpr (SRC == 2) {
      lb = g[lane & 15];
      lc = g[kMixStates + (lane & 15)];
    }
    r = __builtin_fmaf(r, 0.99999f, 1e-7f);
    float d = r, y = 0.f;
    x = __builtin_fmaf(x, 0.9999f, 1e-5f);
    mb_states<SRC>(std::make_integer_sequence<int, kMixStates>{}, h, vb, vc, (mb_cfloat_t*)g, lb, lc,
                   x, r, d, y);
    acc += y;
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

template <int CH>
__global__ void __launch_bounds__(256) k_mul(float* out, int iters, float a, float) {
  float v[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) v[i] = 1e-3f * (i + threadIdx.x);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < CH; ++i) v[i] = v[i] * a;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i) s += v[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int CH>
__global__ void __launch_bounds__(256) k_exp(float* out, int iters, float, float) {
  float v[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) v[i] = 1e-3f * (i + threadIdx.x);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < CH; ++i) v[i] = __builtin_amdgcn_exp2f(-v[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i) s += v[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// --- LDS access patterns.  Per-lane byte offsets of the SSD kernel's B/C
// rows (64 rows of 256 bytes: 128 bf16 states per token), for one wave
// instruction each (index i), in the earlier layout (the 16-byte piece index
// XOR-swizzled by the row within each 128-byte half) and the current one
// (the half also flipped by bit 3 of the row).
__device__ __forceinline__ int lds_swz(int r) { return (r & 1) | ((r & 2) << 1) | ((r & 4) >> 1); }
template <int P>
__device__ int lds_addr(int lane, int tid, int i) {
  const int m = lane & 15, q = lane >> 4, k4 = m >> 2, bq = m & 3;
  if (P == 0 || P == 1) return (lane * 8 + i * 512) & 16383;  // contiguous 8 bytes per lane
  if (P == 4) return (lane * 16 + i * 1024) & 16383;          // contiguous 16 bytes per lane
  if (P == 2 || P == 3) {  // B^T transposes (tr16_b64): i = 4 tile + 2 k-step + f
    const int nb = i >> 2, kk = (i >> 1) & 1, f = i & 1;
    const int r = 8 * q + k4 + 4 * f, piece = (4 * ((nb >> 1) & 1) + bq) ^ lds_swz(r & 7);
    const int hb = (nb >> 2) ^ (P == 3 ? (r >> 3) & 1 : 0);
    return r * 256 + 32 * 256 * kk + 128 * hb + piece * 16 + 8 * (nb & 1);
  }
  if (P == 5 || P == 6) {  // 16-byte row reads of the products: i = 4 k-step + row block
    const int kk = (i >> 2) & 3, sb = i & 3, row = 16 * sb + m;
    const int piece = (4 * (kk & 1) + q) ^ lds_swz(m & 7);
    const int hb = (kk >> 1) ^ (P == 6 ? (row >> 3) & 1 : 0);
    return row * 256 + 128 * hb + piece * 16;
  }
  // staging writes of the rows: thread tid owns piece tid % 16 of rows tid / 16 + 16 j
  const int j = P == 7 ? (i >> 1) & 3 : i & 3, row = tid / 16 + 16 * j;
  const int piece = ((tid % 16) ^ lds_swz(row & 7)) ^ (P == 8 ? 8 * ((row >> 3) & 1) : 0);
  return row * 256 + piece * 16 + (P == 7 ? 8 * ((i & 1) ^ (tid & 1)) : 0);
}
template <int P>
constexpr int lds_n() { return (P == 5 || P == 6) ? 16 : (P == 7 ? 8 : (P == 8 ? 4 : 32)); }
typedef __attribute__((ext_vector_type(4))) short lds_s16x4_t;
typedef __attribute__((address_space(3))) lds_s16x4_t lds_tr_t;
typedef __attribute__((ext_vector_type(2))) unsigned lds_u2_t;
typedef __attribute__((ext_vector_type(4))) unsigned lds_u4_t;
typedef __attribute__((address_space(3))) volatile lds_u2_t lds_u2_p;
typedef __attribute__((address_space(3))) volatile lds_u4_t lds_u4_p;
template <int P>
__global__ void __launch_bounds__(256) k_lds(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char buf[32768];
  for (int i = threadIdx.x; i < 8192; i += 256) reinterpret_cast<unsigned*>(buf)[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  constexpr int N = lds_n<P>();
  int a[N];
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = lds_addr<P>(lane, threadIdx.x, i);
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
    const int off = (it & 1) << 14;  // alternate the two 16 KB halves (the same banks)
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (P == 1 || P == 2 || P == 3) {
        const lds_s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr_t*)(buf + a[i] + off));
        acc += static_cast<unsigned>(v[0]) ^ static_cast<unsigned>(v[3]);
      } else if constexpr (P == 0) {
        const lds_u2_t v = *(lds_u2_p*)(buf + a[i] + off);
        acc += v[0] ^ v[1];
      } else if constexpr (P == 7) {
        *(lds_u2_p*)(buf + a[i] + off) = lds_u2_t{acc, acc + 1u};
        acc += 3u;
      } else if constexpr (P == 8) {
        *(lds_u4_p*)(buf + a[i] + off) = lds_u4_t{acc, acc + 1u, acc + 2u, acc + 3u};
        acc += 5u;
      } else {
        const lds_u4_t v = *(lds_u4_p*)(buf + a[i] + off);
        acc += v[0] ^ v[3];
      }
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] = static_cast<float>(acc & 1u);
}

__global__ void __launch_bounds__(256) k_copy(const float4* __restrict__ in, float4* __restrict__ out,
                                              size_t n) {
  const size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  if (i < n) out[i] = in[i];
}

__global__ void __launch_bounds__(256) k_read(const float4* __restrict__ in, float* __restrict__ out,
                                              size_t n) {
  const size_t T = static_cast<size_t>(gridDim.x) * blockDim.x;
  float s = 0.f;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n; i += T) {
    const float4 v = in[i];
    s += v.x + v.y + v.z + v.w;
  }
  if (s == 1234.5f) out[0] = s;  // keeps the loads
}

__global__ void __launch_bounds__(256) k_inplace(float4* __restrict__ io, size_t n) {
  const size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  if (i < n) {
    float4 v = io[i];
    v.x = v.x * 1.0001f + 1.f;
    v.y *= 0.999f;
    v.z += 1.f;
    v.w -= 1.f;
    io[i] = v;
  }
}

int main() {
  hipDeviceProp_t p;
  CK(hipGetDeviceProperties(&p, 0));
  const int cus = p.multiProcessorCount;
  std::printf("device %s, %d CUs, clock %d kHz\n", p.gcnArchName, cus, p.clockRate);
  float* out;
  CK(hipMalloc(&out, static_cast<size_t>(cus) * 16 * 256 * sizeof(float)));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  // best of 5 timed launches, each right behind about 10 ms of untimed
  // launches of the same kernel: the device is in its loaded steady state
  // (right after an idle period it runs slower for several milliseconds)
  auto timed = [&](auto launch) {
    CK(hipEventRecord(e0));
    launch();
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    float once;
    CK(hipEventElapsedTime(&once, e0, e1));
    const int pre = static_cast<int>(10.0f / (once > 1e-3f ? once : 1e-3f)) + 1;
    float best = 1e30f;
    for (int r = 0; r < 5; ++r) {
      for (int i = 0; i < pre; ++i) launch();
      CK(hipEventRecord(e0));
      launch();
      CK(hipEventRecord(e1));
      CK(hipEventSynchronize(e1));
      float ms;
      CK(hipEventElapsedTime(&ms, e0, e1));
      if (ms < best) best = ms;
    }
    return best;
  };
  // --- vector ALU rates: 32 independent chains per lane
  auto valu = [&](const char* name, void (*k)(float*, int, float, float), int waves_per_simd) {
    const int iters = 2048, chains = 32;
    const int blocks = cus * waves_per_simd;  // 256 threads = one wave per SIMD
    const float ms = timed([&] {
      hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, out, iters, 0.999f, 1e-4f);
    });
    const double ops = static_cast<double>(blocks) * 256 * iters * chains;
    const double rate = ops / (ms * 1e-3);
    const double lanes_per_clk = rate / (cus * 4.0) / 2.4e9;
    std::printf("valu %-4s waves/SIMD=%d  %.3e lane-ops/s  %.2f lanes/clk/SIMD  %.2f clk per wave64 op\n",
                name, waves_per_simd, rate, lanes_per_clk, 64.0 / lanes_per_clk);
  };
  for (int w : {1, 2, 4, 8}) valu("fma", k_fma<32>, w);  // multiplier in an SGPR
  for (int w : {4, 8}) valu("fma-v", k_fma_v<32>, w);   // VGPR operands only
  valu("mul", k_mul<32>, 8);
  valu("exp", k_exp<32>, 8);
  // --- per-state step, b/c from SGPRs / VGPRs / DPP broadcast
  float* bc;
  CK(hipMalloc(&bc, 64 * 2 * kMixStates * sizeof(float)));
  CK(hipMemset(bc, 0, 64 * 2 * kMixStates * sizeof(float)));
  auto step = [&](const char* name, void (*k)(float*, const float*), int waves_per_simd) {
    const int blocks = cus * waves_per_simd;
    const float ms = timed([&] { hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, out, bc); });
    const double wave_tokens = static_cast<double>(blocks) * 4 * kMixTokens;
    const double clk = ms * 1e-3 * 2.4e9 * cus * 4.0 / wave_tokens;
    std::printf("step %-5s waves/SIMD=%d  %.1f clk per wave-token per SIMD, %.2f per state\n", name,
                waves_per_simd, clk, clk / kMixStates);
  };
  for (int w : {6, 8}) {
    step("sgpr", k_step<0>, w);
    step("vgpr", k_step<1>, w);
    step("dpp", k_step<2>, w);
  }
  // --- LDS access patterns: cycles of one CU per wave instruction
  auto lds = [&](const char* name, void (*k)(float*, int), int n) {
    const int blocks = cus * 8, iters = 2000;
    const float ms = timed([&] { hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, out, iters); });
    const double inst_per_cu = blocks * 4.0 / cus * iters * n;
    std::printf("lds  %-52s %6.2f clk per wave-instruction per CU\n", name,
                ms * 1e-3 * 2.4e9 / inst_per_cu);
  };
  lds("read b64, contiguous", k_lds<0>, lds_n<0>());
  lds("read tr16_b64, contiguous", k_lds<1>, lds_n<1>());
  lds("read tr16_b64, B^T of the SSD, earlier layout", k_lds<2>, lds_n<2>());
  lds("read tr16_b64, B^T of the SSD, half flipped by row bit 3", k_lds<3>, lds_n<3>());
  lds("read b128, contiguous", k_lds<4>, lds_n<4>());
  lds("read b128, SSD product rows, earlier layout", k_lds<5>, lds_n<5>());
  lds("read b128, SSD product rows, half flipped by row bit 3", k_lds<6>, lds_n<6>());
  lds("write b64, SSD row staging in 8-byte halves (earlier)", k_lds<7>, lds_n<7>());
  lds("write b128, SSD row staging in 16-byte pieces (current)", k_lds<8>, lds_n<8>());
  // --- HBM streams on 2 GiB buffers (8x the MALL)
  const size_t bytes = static_cast<size_t>(2) << 30, n = bytes / 16;
  float4 *a, *b;
  CK(hipMalloc(&a, bytes));
  CK(hipMalloc(&b, bytes));
  CK(hipMemset(a, 1, bytes));
  CK(hipMemset(b, 0, bytes));
  auto hbm = [&](const char* name, double moved, auto launch) {
    const float ms = timed(launch);
    std::printf("hbm  %-40s %8.3f ms  %7.1f GB/s\n", name, ms, moved / (ms * 1e-3) / 1e9);
  };
  hbm("copy 2 GiB (read+write)", 2.0 * bytes, [&] {
    hipLaunchKernelGGL(k_copy, dim3((n + 255) / 256), dim3(256), 0, 0, a, b, n);
  });
  hbm("read 2 GiB", 1.0 * bytes, [&] {
    hipLaunchKernelGGL(k_read, dim3(cus * 16), dim3(256), 0, 0, a, out, n);
  });
  hbm("in-place 2 GiB (read+write)", 2.0 * bytes, [&] {
    hipLaunchKernelGGL(k_inplace, dim3((n + 255) / 256), dim3(256), 0, 0, a, n);
  });
  const size_t nl = static_cast<size_t>(84) * 1000 * 1000 / 16;  // one decode layer's state
  int layer = 0;
  hbm("in-place 84 MB, 4 rotating buffers", 2.0 * nl * 16, [&] {
    float4* base = a + static_cast<size_t>(layer++ % 4) * nl * 2;
    hipLaunchKernelGGL(k_inplace, dim3((nl + 255) / 256), dim3(256), 0, 0, base, nl);
  });
  CK(hipDeviceSynchronize());
  std::printf("done\n");
  return 0;
}
