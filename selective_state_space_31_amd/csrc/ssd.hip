// ssd.hip -- the state space dual (SSD, Mamba-2) form of the selective scan
// on MFMA, for MI355X (gfx950), behind the C ABI in include/ssm_scan.h (see
// there for the citation and the definition).
//
// With one scalar decay per head the sequence map is 1-semiseparable, so a
// chunk of Q = 64 tokens is computed by matrix products (per sequence b,
// head h, with lambda_t = sum of dt A over the chunk up to t):
//   S      = (C B^T) o mask,  mask[t,s] = e^(lambda_t - lambda_s) dt_s for s <= t
//   Y      = S X + diag(e^lambda) (C h^T) + D X,  then the gate
//   h     <- e^(lambda_end) h + X_w^T B,  X_w[s,:] = X[s,:] dt_s e^(lambda_end - lambda_s)
// where h (headdim x dstate) is the state entering the chunk.  The products
// are bf16 MFMA (v_mfma_f32_16x16x32_bf16) with float32 accumulation.
//
// Work split.  One workgroup (4 waves) owns one (b, h, segment of chunks)
// and walks its chunks in order.  Wave w owns the 16 head channels
// p in [16w, 16w+16): it keeps the float32 state h[p][:] for those channels
// in its MFMA accumulators (as h^T tiles of 16 state rows x 16 channels),
// computes Y^T for them (Y^T = X^T S^T + H C^T ...) and updates their state.
// Because the readout term H C^T takes H as the A operand straight from the
// wave's own accumulators, the state never goes through LDS.  The masked S
// is the one product the waves share: its ten non-zero 16x16 tiles (s <= t)
// are split over the waves and staged in LDS as bf16.
//
// LDS holds the chunk's B, C and x row-major (token rows) as they arrive
// from HBM, with the 16-byte pieces of each row XOR-swizzled by the row
// index so that the MFMA operand reads hit distinct banks.  The operands
// that need a token-contiguous layout (B^T and X^T, whose contraction index
// is the token) are read with the gfx950 transpose load ds_read_b64_tr_b16.
// All global traffic goes through buffer descriptors based at the chunk's
// first row: per-lane offsets are loop constants, the row stride steps are
// scalar offsets, and rows past the sequence end fall outside the
// descriptor's range (loads read zero, stores are dropped).  The next
// chunk's inputs are fetched into registers while the current one is
// computed.  A wave's outputs cover only 32 bytes of each token row, so they
// are staged (float32, before the gate) in the LDS that C and S used, and
// every wave then gates and stores 16 whole 128-byte rows: a quarter of the
// memory requests that storing the accumulator layout directly would make.
//
// When (b, h) pairs alone do not fill the chip, the sequence is cut into
// segments: a state pass runs every segment but the last (state update
// only; segment 0 from the initial state, the others from zero) and leaves
// its end state and total log-decay; the output pass of segment s starts
// from the state entering it, composed from the end states of segments
// 0..s-1 (segment 0 from a copy of the initial state the state pass left).
//
// MFMA operand layout (16x16x32 bf16; checked on the device): lane l holds
// A[l%16][8*(l/16) + i] and B[8*(l/16) + i][l%16], i = 0..7; accumulator
// element r of lane l is D[4*(l/16) + r][l%16].  ds_read_b64_tr_b16 (checked
// on the device, arbitrary per-lane addresses): within each 16-lane group,
// lane 4b+j receives element j of the 8 bytes addressed by lane 4k+b, as its
// element k (k, b, j = 0..3).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_scan.h"

#include "host_util.hpp"
#include "kernels.hpp"

namespace ssm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kSsdQ = 64;         // chunk length (tokens)
constexpr int kSsdP = 64;         // head dimension
constexpr int kSsdThreads = 256;  // 4 waves

// Workgroups per compute unit the segment plan aims for.  On the 2.7B-shaped
// layer (320 (sequence, head) pairs, 32 chunks each) this gives 4 segments;
// 1 to 16 segments measured 134, 125, 125, 119, 126, 137, 135, 134, 149 and
// 187 us for 1, 2, 3, 4, 5, 6, 8, 10, 12, 16.
constexpr int kSsdWgPerCu = 4;

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
  float* seg_state;  // (batch, nseg-1, H) blocks of P*N floats: end state of segment s
                     // (segment 0 from the initial state, the others from zero), in
                     // the waves' accumulator order
  float* h0_copy;    // (batch, H) blocks of P*N floats: the initial state in the same
                     // order, for the output pass of segment 0
  float* seg_lam;    // (batch, nseg-1, H): sum of dt A over segment s
  int L;
  int H;
  int G;
  int softplus;
  int cps;  // chunks per segment
  int nseg;
};

// v shifted across lanes by a DPP pattern; lanes without a source read 0
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}

// inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// inside each row of 16, then the row totals (row_bcast15 to rows 1 and 3,
// row_bcast31 to rows 2 and 3)
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_or_zero<0x111, 0xf>(v);
  v += dpp_or_zero<0x112, 0xf>(v);
  v += dpp_or_zero<0x114, 0xf>(v);
  v += dpp_or_zero<0x118, 0xf>(v);
  v += dpp_or_zero<0x142, 0xa>(v);
  v += dpp_or_zero<0x143, 0xc>(v);
  return v;
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ bf16x8 lds_b128(const unsigned char* base, int byte) {
  return *reinterpret_cast<const bf16x8*>(base + byte);
}

// transpose load (see the header comment for its lane mapping)
__device__ __forceinline__ s16x4 lds_tr(unsigned char* base, int byte) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + byte));
}

__device__ __forceinline__ bf16x8 cat8(s16x4 lo, s16x4 hi) {
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// LDS layout of the B and C rows (token rows of NS bf16 states): rows of 128
// bytes, 64 states each, so that consecutive rows fall on the two halves of
// the 64 banks of 4 bytes (256 bytes per cycle); with 128 states the row's
// second 64 states are in a second plane of Q such rows (kBcPlane bytes
// further), which the operand reads reach by an immediate offset.  (Rows of
// 256 bytes all start at bank 0: a wave's transpose loads of B^T and 16-byte
// row reads then fell on a quarter to a half of the banks, 8.1 cycles per
// wave instruction against 4.4 now.)  The 16-byte pieces of a 128-byte row
// are XOR-swizzled by the row: bits 1 and 2 of (row % 8) swapped, so eight
// consecutive rows get distinct pieces, and rows 4i..4i+3 get {0,1,4,5} or
// {2,3,6,7}.
constexpr int kBcRow = 128;                 // bytes per row of a plane
constexpr int kBcPlane = kSsdQ * kBcRow;    // bytes per plane
__device__ __forceinline__ int swz_bc(int r) { return (r & 1) | ((r & 2) << 1) | ((r & 4) >> 1); }
// byte offset of the 16-byte piece P (states 8P..8P+7) of row r
__device__ __forceinline__ int bc_addr(int r, int P) {
  return (P >> 3) * kBcPlane + r * kBcRow + (((P & 7) ^ swz_bc(r & 7)) << 4);
}
//  x rows (128 bytes): 2 (row % 4) + bit 2 of the row, for the transpose loads of X^T.
__device__ __forceinline__ int swz_x(int r) { return 2 * (r & 3) + ((r >> 2) & 1); }
//  S rows (128 bytes): row % 8.
__device__ __forceinline__ int swz_s(int r) { return r & 7; }

// State tile nb of a wave holds h^T rows n = nmap(nb, q) + r for the lanes
// of group q (accumulator elements r = 0..3): the two tiles 2i, 2i+1 of a
// group cover the eight consecutive n = 32i + 8q .. +7, the lower four in
// tile 2i for even q and in tile 2i+1 for odd q.  B and C rows hold the
// 8-byte halves of odd 16-byte pieces swapped, so the k-step order of the
// readout H C^T (tile 2i's values first) matches C's 16-byte row reads
// without a per-lane select, and the transpose loads of B^T for tile nb
// read half nb % 2 of every piece.
__device__ __forceinline__ int nmap(int nb, int q) {
  return 32 * (nb >> 1) + 8 * q + 4 * ((nb & 1) ^ (q & 1));
}

// Row-read offset of k-step kk (16 states: pieces 4 kk + q) from the bases
// of the two piece parities in the first plane.
__device__ __forceinline__ int bc_off(const int (&bc_kp)[2], int kk) {
  return bc_kp[kk & 1] + kBcPlane * (kk >> 1);
}

// Tiles (sb, tb0..tb0+NTB-1) of S^T (rows s in 16 sb, columns t in 16 tb):
// S^T = B C^T masked and scaled, written to sS as S[t][s] in bf16.
template <int NS, int NTB>
__device__ __forceinline__ void ssd_s_tiles(const unsigned char* sB, const unsigned char* sC,
                                            unsigned char* sS, const float* slam,
                                            const float* sdt, const int (&bc_kp)[2], int lane,
                                            int sb, int tb0) {
  const int m = lane & 15, q = lane >> 4;
  f32x4 acc[NTB];
#pragma unroll
  for (int i = 0; i < NTB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NS / 32; ++kk) {
    const int off = bc_off(bc_kp, kk);
    const bf16x8 av = lds_b128(sB, off + 16 * kBcRow * sb);
#pragma unroll
    for (int i = 0; i < NTB; ++i) {
      const bf16x8 bv = lds_b128(sC, off + 16 * kBcRow * (tb0 + i));
      acc[i] = mfma16(av, bv, acc[i]);
    }
  }
  const int s0 = 16 * sb + 4 * q;
  const f32x4 ls = *reinterpret_cast<const f32x4*>(&slam[s0]);
  const f32x4 ds = *reinterpret_cast<const f32x4*>(&sdt[s0]);
#pragma unroll
  for (int i = 0; i < NTB; ++i) {
    const int tb = tb0 + i, t = 16 * tb + m;
    const float lt = slam[t];
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = acc[i][r] * __builtin_amdgcn_exp2f(lt - ls[r]) * ds[r];
      v[r] = (tb > sb || 4 * q + r <= m) ? e : 0.0f;
    }
    const u32x2 pk = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    *reinterpret_cast<u32x2*>(sS + t * 128 + (((2 * sb + (q >> 1)) ^ swz_s(t)) << 4) +
                              8 * (q & 1)) = pk;
  }
}

// Zero tile (sb, tb), sb > tb, of S: above the diagonal, read by the products
// of the k-steps that straddle the diagonal.
__device__ __forceinline__ void ssd_s_zero(unsigned char* sS, int lane, int sb, int tb) {
  const int m = lane & 15, q = lane >> 4, t = 16 * tb + m;
  *reinterpret_cast<u32x2*>(sS + t * 128 + (((2 * sb + (q >> 1)) ^ swz_s(t)) << 4) + 8 * (q & 1)) =
      u32x2{0u, 0u};
}

// FULL: outputs (and the last segment's final state); otherwise the state
// pass: only the state update, from zero, leaving the segment's end state
// and total log-decay.  Block (head, segment, sequence).
template <int NS, bool GATE, bool FULL>
__global__ void __launch_bounds__(kSsdThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
ssd_fwd_kernel(SsdArgs a) {
  constexpr int Q = kSsdQ, P = kSsdP;
  constexpr int NT = NS / 16;                  // state tiles per wave
  constexpr int NK = NS / 32;                  // k-steps over the state dimension
  constexpr int RB = NS * 2;                   // sB / sC row bytes
  constexpr int PPR = NS / 8;                  // 16-byte pieces per B / C row
  constexpr int NBC = Q * PPR / kSsdThreads;   // B (and C) pieces per thread
  constexpr int RPJ = kSsdThreads / PPR;       // rows between a thread's B / C pieces
  constexpr int NX = Q * P / 8 / kSsdThreads;  // x pieces per thread
  static_assert(RB <= 2 * kBcRow, "B/C rows span at most two planes");
  static_assert(RPJ % 8 == 0 && NX == 2, "layout");
  __shared__ __attribute__((aligned(16))) unsigned char sB[Q * RB];
  // C and S share one region: once every wave has formed its products, the
  // region holds the float32 outputs before the gate (Q x P x 4 bytes)
  static_assert(Q * RB + Q * Q * 2 >= Q * P * 4, "output staging fits");
  __shared__ __attribute__((aligned(16))) unsigned char sCS[FULL ? Q * RB + Q * Q * 2 : 16];
  __shared__ __attribute__((aligned(16))) unsigned char sX[Q * P * 2];
  unsigned char* const sC = sCS;
  unsigned char* const sS = sCS + (FULL ? Q * RB : 0);
  unsigned char* const sY = sCS;
  __shared__ __attribute__((aligned(16))) float slam[Q], sel[Q], sw[Q], sdt[Q];  // slam: lambda log2(e)

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int m = lane & 15, q = lane >> 4;
  const int h = blockIdx.x, seg = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int L = a.L, H = a.H;
  const int grp = h / (H / a.G);
  const float Ah = a.A[h];
  const float Dh = a.D ? a.D[h] : 0.0f;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const uint32_t rowX = static_cast<uint32_t>(H) * P * 2;      // bytes per token row of x, z, out
  const uint32_t rowBC = static_cast<uint32_t>(a.G) * NS * 2;  // bytes per token row of B, C
  const int64_t bh = b * H + h;

  // ---- the state entering the segment ----
  // With one segment, its workgroup reads the initial state and writes the
  // final state itself (in place is safe).  With several, the initial state
  // is read only by the state pass (segment 0 starts from it and leaves a
  // copy for the output pass), which finishes before the output pass writes
  // the final state: the output pass never reads the caller's initial_state,
  // which may be the last_state buffer.
  f32x4 st[NT];
#pragma unroll
  for (int nb = 0; nb < NT; ++nb) st[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool h0_direct = a.h0 && (FULL ? a.nseg == 1 : seg == 0);
  if (h0_direct) {
    const float* src = a.h0 + (bh * P + 16 * w + m) * NS;
#pragma unroll
    for (int nb = 0; nb < NT; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[nb][r] = src[nmap(nb, q) + r];
    if (!FULL) {
      f32x4* cp = reinterpret_cast<f32x4*>(a.h0_copy + static_cast<size_t>(bh) * P * NS) + w * NT * 64;
#pragma unroll
      for (int nb = 0; nb < NT; ++nb) cp[nb * 64 + lane] = st[nb];
    }
  }
  if constexpr (FULL) {
    if (a.h0 && a.nseg > 1 && seg == 0) {
      const f32x4* cp =
          reinterpret_cast<const f32x4*>(a.h0_copy + static_cast<size_t>(bh) * P * NS) + w * NT * 64;
#pragma unroll
      for (int nb = 0; nb < NT; ++nb) st[nb] = cp[nb * 64 + lane];
    }
    for (int j = 0; j < seg; ++j) {
      const size_t slot = (static_cast<size_t>(b) * (a.nseg - 1) + j) * H + h;
      float lo;
      const float e = exp_acc(a.seg_lam[slot], lo);
      const f32x4* hs = reinterpret_cast<const f32x4*>(a.seg_state + slot * P * NS) + w * NT * 64;
#pragma unroll
      for (int nb = 0; nb < NT; ++nb) {
        const f32x4 v = hs[nb * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) st[nb][r] = __builtin_fmaf(e, st[nb][r], v[r]);
      }
    }
  }

  const int nchunks = (L + Q - 1) / Q;
  const int c_begin = seg * a.cps;
  const int c_end = (c_begin + a.cps < nchunks) ? c_begin + a.cps : nchunks;
  float lam_seg = 0.0f;

  // per-lane offsets (loop constants)
  const uint32_t vo_bc = (tid / PPR) * rowBC + (tid % PPR) * 16;
  // B and C rows: the two 8-byte halves of every odd 16-byte piece are
  // stored swapped (see the state tiles' n mapping); each thread writes
  // whole 16-byte pieces (as two 8-byte halves the writes conflicted 4-way)
  const int lds_bc = bc_addr(tid / PPR, tid % PPR);
  const bool bc_odd = (tid & 1) != 0;  // (PPR is even: the piece's parity)
  const uint32_t vo_x = (tid >> 3) * rowX + (tid & 7) * 16;
  const int lds_x = (tid >> 3) * 128 + (((tid & 7) ^ swz_x(tid >> 3)) << 4);
  // z, out: whole 128-byte rows; lane -> token 16 w + 8 i + lane / 8, channels 8 (lane % 8) .. +7
  const uint32_t vo_r = (lane >> 3) * rowX + (lane & 7) * 16;
  const uint32_t vo_dt = lane * static_cast<uint32_t>(H) * 2;
  // LDS address bases of the operand reads; the loop indices (k-step, row
  // block, tile) enter as immediate offsets
  const int k4 = m >> 2, bq = m & 3;
  int bc_kp[2];   // B, C rows 16 blk + m, pieces 4 kk + q (kk parity kp), first half
  int s_base[2];   // S rows 16 tb + m, pieces 4 kk + q
#pragma unroll
  for (int kp = 0; kp < 2; ++kp)
    bc_kp[kp] = bc_addr(m, 4 * kp + q);
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) s_base[kp] = m * 128 + (((4 * kp + q) ^ swz_s(m)) << 4);
  const int x_ep = m * 128 + (((2 * w + (q >> 1)) ^ swz_x(m)) << 4) + 8 * (q & 1);
  int xt_base[2];        // X^T transpose loads: rows 32 kk + 8 q + k4 + 4 f
  int bt_base[2][2];  // B^T transpose loads: [f][tile pair parity], first 128-byte half
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int r = 8 * q + k4 + 4 * f;
    xt_base[f] = r * 128 + (((2 * w + (bq >> 1)) ^ swz_x(r)) << 4) + 8 * (bq & 1);
#pragma unroll
    for (int c1 = 0; c1 < 2; ++c1)
      bt_base[f][c1] = bc_addr(r, 4 * c1 + bq);
  }

  u32x4 pb[NBC], pc[NBC], px[NX];
  u32x4 pz[2];
  uint32_t pdt = 0;
  // Every global access of the chunk loop is issued unconditionally, so the
  // compiler's counts of outstanding loads are exact and a wait for one
  // chunk's data never drains the next chunk's prefetch; a chunk outside the
  // segment gets a descriptor of zero bytes (its loads read zero and touch
  // no memory).
  // (the clamp is taken back to a scalar register: descriptors are scalar,
  // and a count the compiler leaves in a vector register would wrap every
  // load in a loop over lanes)
  auto rows_of = [&](int c) {
    const int t0 = c * Q;
    const int v = (L - t0 < Q) ? L - t0 : Q;
    return __builtin_amdgcn_readfirstlane((c < c_end && v > 0) ? v : 0);
  };
  // B and C (shared by the heads of a group, mostly served by L2) are
  // fetched after the current chunk's readout, x and dt one whole chunk ahead
  auto fetch_bc = [&](int c) {
    const int valid = rows_of(c);
    const int64_t rbc = (b * L + c * Q) * a.G + grp;
    const rsrc_t rB = make_rsrc(a.B + rbc * NS, valid * rowBC);
#pragma unroll
    for (int j = 0; j < NBC; ++j)
      pb[j] = __builtin_amdgcn_raw_buffer_load_b128(rB, vo_bc, j * RPJ * rowBC, 0);
    if constexpr (FULL) {
      const rsrc_t rC = make_rsrc(a.C + rbc * NS, valid * rowBC);
#pragma unroll
      for (int j = 0; j < NBC; ++j)
        pc[j] = __builtin_amdgcn_raw_buffer_load_b128(rC, vo_bc, j * RPJ * rowBC, 0);
    }
  };
  auto fetch_x = [&](int c) {
    const int valid = rows_of(c);
    const int64_t rx = (b * L + c * Q) * H + h;
    const rsrc_t rX = make_rsrc(a.x + rx * P, valid * rowX);
#pragma unroll
    for (int j = 0; j < NX; ++j)
      px[j] = __builtin_amdgcn_raw_buffer_load_b128(rX, vo_x, j * 32 * rowX, 0);
    // (only wave 0 uses dt: the other waves' descriptor has no bytes)
    pdt = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(a.dt + rx, w == 0 ? valid * H * 2 : 0),
                                               vo_dt, 0, 0);
  };
  // the gate of a chunk is fetched after the previous chunk's outputs are written
  auto fetch_z = [&](int c) {
    const int t0 = c * Q;
    const int valid = rows_of(c);
    const rsrc_t rZ = make_rsrc(a.z + ((b * L + t0) * H + h) * P, valid * rowX);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      pz[i] = __builtin_amdgcn_raw_buffer_load_b128(rZ, vo_r, (16 * w + 8 * i) * rowX, 0);
  };
  if (c_begin < c_end) {
    fetch_bc(c_begin);
    fetch_x(c_begin);
    if constexpr (FULL && GATE) fetch_z(c_begin);
  }

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * Q;
    // ---- 1. stage the chunk fetched ahead; wave 0 forms lambda and the weights ----
#pragma unroll
    for (int j = 0; j < NBC; ++j) {
      const int o = j * RPJ * kBcRow;
      *reinterpret_cast<u32x4*>(sB + lds_bc + o) =
          bc_odd ? u32x4{pb[j][2], pb[j][3], pb[j][0], pb[j][1]} : pb[j];
      if constexpr (FULL) {
        *reinterpret_cast<u32x4*>(sC + lds_bc + o) =
            bc_odd ? u32x4{pc[j][2], pc[j][3], pc[j][0], pc[j][1]} : pc[j];
      }
    }
#pragma unroll
    for (int j = 0; j < NX; ++j) *reinterpret_cast<u32x4*>(sX + lds_x + j * 32 * 128) = px[j];
    if (w == 0) {
      const float u = bf_lo(pdt) + bias;
      float dtv = a.softplus ? softplus_f32(u) : u;
      if (t0 + lane >= L) dtv = 0.0f;  // past the end: no decay, no input
      // lambda in log2 units: exponentials below are exp2 of differences
      const float v = wave_prefix_sum(dtv * (Ah * kLog2e));
      const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
      slam[lane] = v;
      sel[lane] = __builtin_amdgcn_exp2f(v);
      sw[lane] = dtv * __builtin_amdgcn_exp2f(lend - v);
      sdt[lane] = dtv;
    }
    fetch_x(c + 1);
    if constexpr (!FULL) fetch_bc(c + 1);
    __syncthreads();

    // X^T operand of this wave's channels: lane (q, m) holds x[s = 32 kk + 8 q + i][16 w + m]
    bf16x8 xa[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      xa[kk] = cat8(lds_tr(sX, xt_base[0] + 32 * 128 * kk), lds_tr(sX, xt_base[1] + 32 * 128 * kk));

    if constexpr (FULL) {
      // ---- 2. the ten non-zero tiles of S, split over the waves ----
      // (the two zero tiles are rewritten every chunk: the outputs staged
      // at the end of a chunk may cover S)
      if (w == 0) {
        ssd_s_tiles<NS, 3>(sB, sC, sS, slam, sdt, bc_kp, lane, 0, 0);
        ssd_s_zero(sS, lane, 1, 0);
      } else if (w == 1) {
        ssd_s_tiles<NS, 3>(sB, sC, sS, slam, sdt, bc_kp, lane, 1, 1);
      } else if (w == 2) {
        ssd_s_tiles<NS, 2>(sB, sC, sS, slam, sdt, bc_kp, lane, 2, 2);
        ssd_s_zero(sS, lane, 3, 2);
      } else {
        ssd_s_tiles<NS, 1>(sB, sC, sS, slam, sdt, bc_kp, lane, 0, 3);
        ssd_s_tiles<NS, 1>(sB, sC, sS, slam, sdt, bc_kp, lane, 3, 3);
      }
      // bf16 copy of the entering state as the A operand of H C^T: lane (q, m)
      // holds h[16 w + m][n] for the n of its tiles 2 kk, 2 kk + 1 in that order
      bf16x8 hA[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const f32x4 lo = st[2 * kk], hi = st[2 * kk + 1];
        hA[kk] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]),
                                                   pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3])});
      }
      __syncthreads();

      // ---- 3. Y^T = X^T S^T + (H C^T) diag(e^lambda) + D X^T, per 16 tokens ----
      // products of token block tb (the masked intra-chunk part and the readout)
      auto products = [&](int tb, f32x4& y1, f32x4& y2) {
        y1 = f32x4{0.f, 0.f, 0.f, 0.f};
        y2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < (tb >= 2 ? 2 : 1); ++kk)
          y1 = mfma16(xa[kk], lds_b128(sS, s_base[kk] + 16 * 128 * tb), y1);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          y2 = mfma16(hA[kk], lds_b128(sC, bc_off(bc_kp, kk) + 16 * kBcRow * tb), y2);
      };
      // y before the gate: lane (q, m) holds channels 16 w + 4 q .. +3 of token 16 tb + m
      auto combine = [&](int tb, const f32x4& y1, const f32x4& y2) {
        const float el = sel[16 * tb + m];
        const u32x2 xr = *reinterpret_cast<const u32x2*>(sX + x_ep + 16 * 128 * tb);
        const float xv[4] = {bf_lo(xr[0]), bf_hi(xr[0]), bf_lo(xr[1]), bf_hi(xr[1])};
        f32x4 y;
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = __builtin_fmaf(Dh, xv[r], __builtin_fmaf(el, y2[r], y1[r]));
        return y;
      };
      f32x4 yp[4];
      {
        f32x4 ya1, ya2, yb1, yb2;
        products(0, ya1, ya2);
        products(1, yb1, yb2);
        yp[0] = combine(0, ya1, ya2);
        products(2, ya1, ya2);
        yp[1] = combine(1, yb1, yb2);
        products(3, yb1, yb2);
        yp[2] = combine(2, ya1, ya2);
        yp[3] = combine(3, yb1, yb2);
      }
      __syncthreads();  // every wave is done with C and S
      // float32 rows of 64 channels, 16-byte pieces swizzled by token % 16
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        *reinterpret_cast<f32x4*>(sY + (16 * tb + m) * 256 + (((4 * w + q) ^ m) << 4)) = yp[tb];
      fetch_bc(c + 1);
    }

    // ---- 4. h <- e^(lambda_end) h + X_w^T B ----
    {
      bf16x8 xw[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(&sw[32 * kk + 8 * q]);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(&sw[32 * kk + 8 * q + 4]);
        const float f[8] = {static_cast<float>(xa[kk][0]) * w0[0], static_cast<float>(xa[kk][1]) * w0[1],
                            static_cast<float>(xa[kk][2]) * w0[2], static_cast<float>(xa[kk][3]) * w0[3],
                            static_cast<float>(xa[kk][4]) * w1[0], static_cast<float>(xa[kk][5]) * w1[1],
                            static_cast<float>(xa[kk][6]) * w1[2], static_cast<float>(xa[kk][7]) * w1[3]};
        xw[kk] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]),
                                                   pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])});
      }
      const float aend = sel[Q - 1];
      if constexpr (!FULL) lam_seg += slam[Q - 1] * kLn2;
      // A operands (B^T) of tile nb for both k-steps, read one tile ahead
      auto bt_read = [&](int nb, int kk) {
        // (tiles nb >= 4 hold states 64..127: the second plane)
        const int imm = 32 * kBcRow * kk + 8 * (nb & 1) + kBcPlane * (nb >> 2);
        const int c1 = (nb >> 1) & 1;
        return cat8(lds_tr(sB, bt_base[0][c1] + imm), lds_tr(sB, bt_base[1][c1] + imm));
      };
      bf16x8 an0 = bt_read(0, 0), an1 = bt_read(0, 1);
#pragma unroll
      for (int nb = 0; nb < NT; ++nb) {
        const bf16x8 a0 = an0, a1 = an1;
        if (nb + 1 < NT) {
          an0 = bt_read(nb + 1, 0);
          an1 = bt_read(nb + 1, 1);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) st[nb][r] *= aend;
        st[nb] = mfma16(a0, xw[0], st[nb]);
        st[nb] = mfma16(a1, xw[1], st[nb]);
      }
    }
    if constexpr (FULL) {
      __syncthreads();  // the outputs before the gate are complete
      // ---- 5. gate and store: wave w writes tokens 16 w .. 16 w + 15, whole rows ----
      const int valid = (L - t0 < Q) ? L - t0 : Q;
      const rsrc_t rO = make_rsrc(a.out + ((b * L + t0) * H + h) * P, valid * rowX);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = 16 * w + 8 * i + (lane >> 3), pc0 = 2 * (lane & 7);
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(sY + t * 256 + ((pc0 ^ (t & 15)) << 4));
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(sY + t * 256 + (((pc0 + 1) ^ (t & 15)) << 4));
        float y[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
        if constexpr (GATE) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            y[2 * j] *= silu_f32(bf_lo(pz[i][j]));
            y[2 * j + 1] *= silu_f32(bf_hi(pz[i][j]));
          }
        }
        const u32x4 o = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]),
                         pack_bf16(y[6], y[7])};
        __builtin_amdgcn_raw_buffer_store_b128(o, rO, vo_r, (16 * w + 8 * i) * rowX, kStoreStream);
      }
      if constexpr (GATE) fetch_z(c + 1);
    }
    __syncthreads();  // the next chunk restages every LDS buffer
  }

  if constexpr (FULL) {
    if (seg == a.nseg - 1 && a.last_state) {
      float* dst = a.last_state + (bh * P + 16 * w + m) * NS;
#pragma unroll
      for (int nb = 0; nb < NT; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[nmap(nb, q) + r] = st[nb][r];
    }
  } else {
    const size_t slot = (static_cast<size_t>(b) * (a.nseg - 1) + seg) * H + h;
    f32x4* hs = reinterpret_cast<f32x4*>(a.seg_state + slot * P * NS) + w * NT * 64;
#pragma unroll
    for (int nb = 0; nb < NT; ++nb) hs[nb * 64 + lane] = st[nb];
    if (tid == 0) a.seg_lam[slot] = lam_seg;
  }
}

struct SsdPlan {
  int cps, nseg;
};

// Segments: enough (head, segment, sequence) workgroups for the resident
// workgroups of every compute unit, at least two chunks per segment.
SsdPlan plan_ssd(int64_t batch, int64_t L, int64_t H) {
  const int64_t nchunks = (L + kSsdQ - 1) / kSsdQ;
  const int64_t target = static_cast<int64_t>(kSsdWgPerCu) * device_cus();
  int64_t nseg = (target + batch * H - 1) / (batch * H);
  if (nseg > nchunks / 2) nseg = nchunks / 2;
  if (nseg < 1) nseg = 1;
  int64_t cps = (nchunks + nseg - 1) / nseg;
  if (cps < 1) cps = 1;
  nseg = nchunks > 0 ? (nchunks + cps - 1) / cps : 1;
  return SsdPlan{static_cast<int>(cps), static_cast<int>(nseg)};
}

// Workspace (only with several segments): the segments' end states
// (nseg - 1 per (sequence, head)), a copy of the initial state per
// (sequence, head), then the segments' log-decays.
size_t ssd_workspace(int64_t batch, int64_t H, int64_t P, int64_t N, const SsdPlan& p) {
  if (p.nseg <= 1) return 0;
  const size_t states = static_cast<size_t>(batch) * p.nseg * H * P * N * 4;
  return (states + 255) / 256 * 256 + static_cast<size_t>(batch) * (p.nseg - 1) * H * 4;
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
      {x, 16, "x"}, {B, 16, "B"}, {C, 16, "C"}, {dt, 2, "dt"}, {z, 8, "z"}, {out, 8, "out"},
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
  const size_t slot_floats = static_cast<size_t>(batch) * nheads * headdim * dstate;
  const size_t sbytes = slot_floats * plan.nseg * 4;
  float* seg_state = need ? static_cast<float*>(workspace) : nullptr;
  float* h0_copy = need ? seg_state + slot_floats * (plan.nseg - 1) : nullptr;
  float* seg_lam = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                   (sbytes + 255) / 256 * 256)
                        : nullptr;
  SsdArgs args{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(dt), dt_bias, A,
               static_cast<const bf16_t*>(B), static_cast<const bf16_t*>(C), D,
               static_cast<const bf16_t*>(z), static_cast<bf16_t*>(out), last_state,
               initial_state, seg_state, h0_copy, seg_lam, static_cast<int>(seqlen),
               static_cast<int>(nheads), static_cast<int>(ngroups), dt_softplus, plan.cps,
               plan.nseg};
  const dim3 block(kSsdThreads);
  const bool big = dstate == 128;
  if (plan.nseg > 1) {
    // state pass over every segment but the last
    const dim3 g1(static_cast<unsigned>(nheads), static_cast<unsigned>(plan.nseg - 1),
                  static_cast<unsigned>(batch));
    if (big) hipLaunchKernelGGL((ssd_fwd_kernel<128, false, false>), g1, block, 0, stream, args);
    else hipLaunchKernelGGL((ssd_fwd_kernel<64, false, false>), g1, block, 0, stream, args);
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
