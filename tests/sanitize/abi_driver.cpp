// abi_driver.cpp -- host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure).
//
// Linked against host-only builds of the library's units (no device code:
// nothing here may reach a kernel launch).  Every call below carries an
// argument the library must reject before it touches the device, and the
// workspace queries run over grids of edge and extreme sizes, where the size
// arithmetic would overflow if it were not checked.  Pointers are distinct
// host blocks: the host code compares their values (alignment, overlap) and
// must never dereference them.  Exit status: the number of calls that were
// not rejected.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "ssm_scan.h"

namespace {

int g_bad = 0;

void expect_reject(int rc, const char* what) {
  if (rc >= 0) {
    std::printf("NOT REJECTED (rc %d): %s\n", rc, what);
    ++g_bad;
  }
}

// Distinct, generously spaced blocks standing in for device buffers.
struct Blocks {
  std::vector<char*> v;
  char* get(size_t bytes = size_t{1} << 16) {
    char* p = static_cast<char*>(std::aligned_alloc(256, bytes));
    v.push_back(p);
    return p;
  }
  ~Blocks() {
    for (char* p : v) std::free(p);
  }
};

const int64_t kEdge[] = {INT64_MIN, -1, 0, 1, 2, 3, 63, 64, 65, 4096, 65535, 65536,
                         int64_t{1} << 31, int64_t{1} << 40, INT64_MAX};
const int64_t kStates[] = {INT64_MIN, -1, 0, 1, 3, 4, 8, 16, 17, 64, 65, 128, 129, INT64_MAX};

}  // namespace

int main() {
  Blocks m;
  const hipStream_t s = nullptr;
  void *x = m.get(), *dl = m.get(), *B = m.get(), *C = m.get(), *z = m.get(), *out = m.get();
  float *A = reinterpret_cast<float*>(m.get()), *bias = reinterpret_cast<float*>(m.get());
  float *Ds = reinterpret_cast<float*>(m.get()), *last = reinterpret_cast<float*>(m.get());
  float* h0 = reinterpret_cast<float*>(m.get());
  void* ws = m.get();
  char* xm = static_cast<char*>(x) + 1;  // misaligned

  // ---- workspace queries over edge sizes (must never overflow) ----
  size_t acc = 0;
  for (int64_t b : kEdge)
    for (int64_t L : kEdge)
      for (int64_t d : kEdge)
        for (int64_t n : kStates)
          for (int dt = 0; dt < 3; ++dt) {
            acc += ssm_scan_fwd_workspace_bytes(b, L, d, n, dt);
            acc += ssm_scan_fwd_varlen_workspace_bytes(b, L, d, n, dt);
            acc += ssm_scan_bwd_workspace_bytes(b, L, d, n, dt);
            acc += ssm_scan_fwd_chunked_workspace_bytes(b, L, d, n, dt, 64);
          }
  for (int64_t cl : kEdge) acc += ssm_scan_fwd_chunked_workspace_bytes(4, 2048, 1536, 16, 1, cl);
  for (int64_t b : kEdge)
    for (int64_t L : kEdge)
      for (int64_t h : kEdge)
        for (int64_t n : kStates)
          for (int64_t g : {int64_t{-1}, int64_t{0}, int64_t{1}, int64_t{2}, int64_t{3}}) {
            acc += ssm_ssd_fwd_workspace_bytes(b, L, h, 64, n, g);
            acc += ssm_ssd_fwd_workspace_bytes(b, L, h, n, 128, g);
          }
  std::printf("workspace queries done (%zu)\n", acc & 0xffff);

  // ---- forward: dense, chunked, no-alloc ----
  auto fwd = [&](const void* xx, const void* dd, const float* AA, const void* BB, const void* CC,
                 void* oo, int sp, int64_t b, int64_t L, int64_t d, int64_t n, int dt,
                 size_t wsb, const char* what) {
    expect_reject(ssm_scan_fwd(xx, dd, bias, sp, AA, BB, CC, Ds, z, oo, last, h0, b, L, d, n, dt,
                               ws, wsb, s),
                  what);
    expect_reject(ssm_scan_fwd_chunked(xx, dd, bias, sp, AA, BB, CC, Ds, z, oo, last, h0, b, L, d,
                                       n, dt, 64, ws, wsb, s),
                  what);
    expect_reject(ssm_scan_fwd_noalloc(xx, dd, bias, sp, AA, BB, CC, Ds, z, oo, last, h0, b, L, d,
                                       n, dt, s),
                  what);
  };
  fwd(nullptr, dl, A, B, C, out, 1, 1, 16, 64, 16, 1, 1 << 16, "fwd: null x");
  fwd(x, nullptr, A, B, C, out, 1, 1, 16, 64, 16, 1, 1 << 16, "fwd: null delta");
  fwd(x, dl, nullptr, B, C, out, 1, 1, 16, 64, 16, 1, 1 << 16, "fwd: null A");
  fwd(x, dl, A, nullptr, C, out, 1, 1, 16, 64, 16, 1, 1 << 16, "fwd: null B");
  fwd(x, dl, A, B, C, nullptr, 1, 1, 16, 64, 16, 1, 1 << 16, "fwd: null out");
  for (int64_t v : kEdge) {
    if (v < 1) {
      fwd(x, dl, A, B, C, out, 1, v, 16, 64, 16, 1, 1 << 16, "fwd: batch < 1");
      fwd(x, dl, A, B, C, out, 1, 1, 16, v, 16, 1, 1 << 16, "fwd: dim < 1");
    }
    if (v < 0) fwd(x, dl, A, B, C, out, 1, 1, v, 64, 16, 1, 1 << 16, "fwd: seqlen < 0");
    if (v > (int64_t{1} << 35)) {
      fwd(x, dl, A, B, C, out, 1, v, v, v, 16, 1, 1 << 16, "fwd: sizes beyond any device");
      fwd(x, dl, A, B, C, out, 1, 1, v, 64, 16, 1, 1 << 16, "fwd: seqlen beyond any device");
    }
  }
  for (int64_t n : kStates)
    if (n < 1 || n > 64) fwd(x, dl, A, B, C, out, 1, 1, 16, 64, n, 1, 1 << 16, "fwd: dstate");
  fwd(x, dl, A, B, C, out, 1, 1, 16, 64, 16, 7, 1 << 16, "fwd: dtype");
  fwd(x, dl, A, B, C, out, 2, 1, 16, 64, 16, 1, 1 << 16, "fwd: softplus flag");
  fwd(xm, dl, A, B, C, out, 1, 1, 16, 64, 16, 1, 1 << 16, "fwd: misaligned x");
  fwd(x, dl, A, B, C, x, 1, 1, 16, 64, 16, 1, 1 << 16, "fwd: out aliases x");
  fwd(x, dl, A, B, C, static_cast<char*>(dl) + 64, 1, 1, 16, 64, 16, 1, 1 << 16,
      "fwd: out overlaps delta");
  expect_reject(ssm_scan_fwd(x, dl, bias, 1, A, B, C, Ds, z, out, last, h0, 1, 1 << 16, 64, 16, 1,
                             ws, 1, s),
                "fwd: workspace too small");
  for (int64_t cl : kEdge)
    if (cl < 0 || cl > (int64_t{1} << 35))
      expect_reject(ssm_scan_fwd_chunked(x, dl, bias, 1, A, B, C, Ds, z, out, last, h0, 1, 4096,
                                         64, 16, 1, cl, ws, 1 << 16, s),
                    "fwd chunked: chunk_len");

  // ---- packed sequences ----
  const int32_t* cu = reinterpret_cast<const int32_t*>(m.get());
  auto var = [&](const int32_t* cc, int64_t nseq, int64_t T, int64_t d, int64_t n, size_t wsb,
                 const char* what) {
    expect_reject(ssm_scan_fwd_varlen(x, dl, bias, 1, A, B, C, Ds, z, out, last, h0, cc, nseq, T,
                                      d, n, 1, ws, wsb, s),
                  what);
  };
  var(nullptr, 2, 64, 64, 16, 1 << 16, "varlen: null offsets");
  for (int64_t v : kEdge) {
    if (v < 1) var(cu, v, 64, 64, 16, 1 << 16, "varlen: nseq < 1");
    if (v < 0) var(cu, 2, v, 64, 16, 1 << 16, "varlen: total < 0");
    if (v > (int64_t{1} << 35)) var(cu, v, v, v, 16, 1 << 16, "varlen: huge");
  }
  var(cu, 2, 1 << 16, 64, 16, 1, "varlen: workspace too small");

  // ---- decode ----
  auto dec = [&](float* st, const void* xx, const float* AA, void* oo, int64_t b, int64_t d,
                 int64_t n, const char* what) {
    expect_reject(ssm_state_update(st, xx, dl, bias, 1, AA, B, C, Ds, z, oo, b, d, n, 1, s), what);
  };
  dec(nullptr, x, A, out, 4, 64, 16, "decode: null state");
  dec(h0, x, A, x, 4, 64, 16, "decode: out aliases x");
  dec(h0, x, A, h0, 4, 64, 16, "decode: out aliases state");
  dec(h0, x, reinterpret_cast<float*>(reinterpret_cast<char*>(A) + 4), out, 4, 64, 16,
      "decode: A not 16-byte aligned with dstate % 4 == 0");
  for (int64_t v : kEdge)
    if (v < 1 || v > (int64_t{1} << 35)) {
      dec(h0, x, A, out, v, 64, 16, "decode: batch");
      dec(h0, x, A, out, 4, v, 16, "decode: dim");
    }
  for (int64_t n : kStates)
    if (n < 1 || n > 64) dec(h0, x, A, out, 4, 64, n, "decode: dstate");

  // ---- convolution ----
  float* w = reinterpret_cast<float*>(m.get());
  for (int64_t W : {int64_t{-1}, int64_t{0}, int64_t{1}, int64_t{5}, INT64_MAX})
    expect_reject(ssm_causal_conv1d_fwd(x, w, bias, nullptr, out, nullptr, 1, 16, 64, W, 1, 1, s),
                  "conv: width");
  expect_reject(ssm_causal_conv1d_fwd(x, w, bias, nullptr, out, nullptr, 1, 16, 64, 4, 2, 1, s),
                "conv: silu flag");
  expect_reject(ssm_causal_conv1d_fwd(x, w, bias, nullptr, x, nullptr, 1, 16, 64, 4, 1, 1, s),
                "conv: out aliases x");
  for (int64_t v : kEdge)
    if (v < 0 || v > (int64_t{1} << 35)) {
      expect_reject(ssm_causal_conv1d_fwd(x, w, bias, nullptr, out, nullptr, v, 16, 64, 4, 1, 1, s),
                    "conv: batch");
      expect_reject(ssm_causal_conv1d_fwd(x, w, bias, nullptr, out, nullptr, 1, v, 64, 4, 1, 1, s),
                    "conv: seqlen");
      expect_reject(ssm_causal_conv1d_fwd(x, w, bias, nullptr, out, nullptr, 1, 16, v, 4, 1, 1, s),
                    "conv: dim");
      expect_reject(ssm_causal_conv1d_update(z, x, w, bias, out, v, 64, 4, 1, 1, s),
                    "conv update: batch");
    }
  expect_reject(ssm_causal_conv1d_update(nullptr, x, w, bias, out, 4, 64, 4, 1, 1, s),
                "conv update: null state");
  expect_reject(ssm_causal_conv1d_update(z, x, w, bias, out, 4, 64, 1, 1, 1, s),
                "conv update: width");

  // ---- backward ----
  void *dx = m.get(), *ddl = m.get(), *dz = m.get(), *dout = m.get();
  float *dA = reinterpret_cast<float*>(m.get()), *dB = reinterpret_cast<float*>(m.get());
  float *dC = reinterpret_cast<float*>(m.get()), *dD = reinterpret_cast<float*>(m.get());
  float *dbias = reinterpret_cast<float*>(m.get()), *dh0 = reinterpret_cast<float*>(m.get());
  auto bwd = [&](void* dxx, int64_t b, int64_t L, int64_t d, int64_t n, size_t wsb,
                 const char* what) {
    expect_reject(ssm_scan_bwd(x, dl, bias, 1, A, B, C, Ds, z, h0, dout, nullptr, dxx, ddl, dz, dA,
                               dB, dC, dD, dbias, dh0, b, L, d, n, 1, ws, wsb, s),
                  what);
  };
  bwd(nullptr, 1, 64, 64, 16, 1 << 16, "bwd: null dx");
  bwd(x, 1, 64, 64, 16, 1 << 16, "bwd: dx aliases x");
  bwd(dx, 1, 1 << 16, 64, 16, 1, "bwd: workspace too small");
  for (int64_t n : kStates)
    if (n != 4 && n != 8 && n != 16) bwd(dx, 1, 64, 64, n, 1 << 16, "bwd: dstate");
  for (int64_t v : kEdge)
    if (v < 1 || v > (int64_t{1} << 35)) {
      bwd(dx, v, 64, 64, 16, 1 << 16, "bwd: batch");
      bwd(dx, 1, 64, v, 16, 1 << 16, "bwd: dim");
      if (v != 0) bwd(dx, 1, v, 64, 16, 1 << 16, "bwd: seqlen");
    }

  // ---- SSD ----
  auto ssd = [&](void* oo, int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                 int dt, size_t wsb, const char* what) {
    expect_reject(ssm_ssd_fwd(x, dl, bias, 1, A, B, C, Ds, z, oo, last, h0, b, L, H, P, N, G, dt,
                              ws, wsb, s),
                  what);
  };
  ssd(out, 1, 128, 8, 32, 128, 1, 1, 1 << 16, "ssd: headdim");
  ssd(out, 1, 128, 8, 64, 96, 1, 1, 1 << 16, "ssd: dstate");
  ssd(out, 1, 128, 8, 64, 128, 3, 1, 1 << 16, "ssd: groups do not divide heads");
  ssd(out, 1, 128, 8, 64, 128, 1, 0, 1 << 16, "ssd: float32 activations");
  ssd(x, 1, 128, 8, 64, 128, 1, 1, 1 << 16, "ssd: out aliases x");
  ssd(out, 1, 1 << 14, 8, 64, 128, 1, 1, 1, "ssd: workspace too small");
  for (int64_t v : kEdge)
    if (v < 1 || v > (int64_t{1} << 35)) {
      ssd(out, v, 128, 8, 64, 128, 1, 1, 1 << 16, "ssd: batch");
      ssd(out, 1, 128, v, 64, 128, 1, 1, 1 << 16, "ssd: heads");
      if (v != 0) ssd(out, 1, v, 8, 64, 128, 1, 1, 1 << 16, "ssd: seqlen");
    }

  std::printf("abi driver: %d call(s) not rejected; last message: %s\n", g_bad, ssm_last_error());
  return g_bad;
}
