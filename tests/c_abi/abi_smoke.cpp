// The C ABI used from a plain host program: device buffers from hipMalloc,
// one stream, no Python and no torch.  Each call is checked against values
// fixed by hand (closed forms of the operations on tiny inputs):
//   route    p_t = (1 - cos(q_t, k_{t-1})) / 2, p = 1 at the sequence start
//   compact  the positions with p >= 1/2 and their rows
//   dechunk  P = 1 gives each byte its chunk's row
//   coding   orthogonal rows: Delta R_t = 1/2 log(1 + alpha |h_t|^2); a batch
//            split over two streams equals its sequences computed alone
//   top-k    BOS plus the K - 1 largest scores, in time order
//   upsample g = 0 leaves the residual h unchanged
// Prints "abi smoke ok" and exits 0 on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/bllm.h"

#define CK(x)                                                                               \
  do {                                                                                      \
    hipError_t e_ = (x);                                                                    \
    if (e_ != hipSuccess) {                                                                 \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);            \
      return 1;                                                                             \
    }                                                                                       \
  } while (0)
#define OK(x)                                                                               \
  do {                                                                                      \
    int r_ = (x);                                                                           \
    if (r_ != BLLM_OK) {                                                                    \
      std::printf("%s returned %d (%s) at line %d\n", #x, r_, bllm_status_string(r_), __LINE__); \
      return 1;                                                                             \
    }                                                                                       \
  } while (0)
#define EXPECT(c, msg)                        \
  do {                                        \
    if (!(c)) {                               \
      std::printf("FAIL: %s\n", msg);         \
      return 1;                               \
    }                                         \
  } while (0)

template <class T>
static T* to_dev(const std::vector<T>& h) {
  T* p = nullptr;
  if (hipMalloc(&p, h.size() * sizeof(T) + 16) != hipSuccess) return nullptr;
  if (hipMemcpy(p, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
  return p;
}

template <class T>
static std::vector<T> to_host(const T* d, size_t n) {
  std::vector<T> h(n);
  if (hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost) != hipSuccess) h.clear();
  return h;
}

static void* dev_bytes(size_t n) {
  void* p = nullptr;
  return hipMalloc(&p, n > 0 ? n : 16) == hipSuccess ? p : nullptr;
}

static uint16_t bf16(float x) {  // exact for the small integers used here
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return static_cast<uint16_t>(u >> 16);
}

int main() {
  hipStream_t st;
  CK(hipStreamCreate(&st));
  EXPECT(bllm_version() > 0, "version");

  // ---- route, compact, dechunk: one sequence of 4 rows, d = 4, fp32
  const int64_t d = 4, T = 4;
  // k_0 = e0, k_1 = e1, k_2 = e0; q_1 = e0 (cos 1), q_2 = e0 (cos 0 with k_1), q_3 = -e0 (cos -1)
  std::vector<float> q = {1, 0, 0, 0, 1, 0, 0, 0, 1, 0, 0, 0, -1, 0, 0, 0};
  std::vector<float> k = {1, 0, 0, 0, 0, 1, 0, 0, 1, 0, 0, 0, 0, 0, 1, 0};
  std::vector<int64_t> off = {0, T};
  float* dq = to_dev(q);
  float* dk = to_dev(k);
  int64_t* doff = to_dev(off);
  float* dp = static_cast<float*>(dev_bytes(T * 4));
  uint8_t* db = static_cast<uint8_t*>(dev_bytes(T));
  float* dtau = static_cast<float*>(dev_bytes(4));
  EXPECT(dq && dk && doff && dp && db && dtau, "alloc");
  OK(bllm_route(dq, dk, BLLM_F32, d, doff, 1, T, 0.5f, -1.0, dp, db, dtau, nullptr, nullptr, 0, st));
  CK(hipStreamSynchronize(st));
  const std::vector<float> p = to_host(dp, T);
  const std::vector<uint8_t> b = to_host(db, T);
  const float p_want[4] = {1.f, 0.f, 0.5f, 1.f};
  for (int t = 0; t < 4; ++t) EXPECT(std::fabs(p[t] - p_want[t]) < 1e-6f, "route p");
  const uint8_t b_want[4] = {1, 0, 1, 1};
  for (int t = 0; t < 4; ++t) EXPECT(b[t] == b_want[t], "route b");

  std::vector<float> rows(T * d);
  for (int i = 0; i < T * d; ++i) rows[i] = static_cast<float>(i);
  float* drows = to_dev(rows);
  int32_t* didx = static_cast<int32_t*>(dev_bytes(T * 4));
  int64_t* dcoff = static_cast<int64_t*>(dev_bytes(2 * 8));
  float* dz = static_cast<float*>(dev_bytes(T * d * 4));
  float* dP = static_cast<float*>(dev_bytes(T * 4));
  int32_t* dstat = static_cast<int32_t*>(dev_bytes(4));
  const size_t wsc = bllm_compact_workspace(T);
  void* ws = dev_bytes(wsc);
  EXPECT(drows && didx && dcoff && dz && dP && dstat && ws, "alloc");
  CK(hipMemset(dstat, 0, 4));
  OK(bllm_compact(db, dp, drows, BLLM_F32, d, doff, 1, T, T, didx, dcoff, dz, dP, dstat, ws, wsc, st));
  CK(hipStreamSynchronize(st));
  const std::vector<int32_t> idx = to_host(didx, 3);
  const std::vector<int64_t> coff = to_host(dcoff, 2);
  EXPECT(idx[0] == 0 && idx[1] == 2 && idx[2] == 3, "compact idx");
  EXPECT(coff[0] == 0 && coff[1] == 3, "compact chunk offsets");
  const std::vector<float> z = to_host(dz, 3 * d);
  for (int c = 0; c < 3; ++c)
    for (int f = 0; f < d; ++f) EXPECT(z[c * d + f] == rows[idx[c] * d + f], "compact rows");

  std::vector<float> ones(3, 1.f);
  float* dones = to_dev(ones);
  float* dout = static_cast<float*>(dev_bytes(T * d * 4));
  const size_t wsd = bllm_dechunk_workspace(d);
  void* ws2 = dev_bytes(wsd);
  EXPECT(dones && dout && ws2, "alloc");
  OK(bllm_dechunk_ema(dz, dones, BLLM_F32, d, didx, dcoff, doff, 1, T, 3, dout, ws2, wsd, st));
  CK(hipStreamSynchronize(st));
  const std::vector<float> out = to_host(dout, T * d);
  const int chunk_of[4] = {0, 0, 1, 2};
  for (int t = 0; t < 4; ++t)
    for (int f = 0; f < d; ++f) EXPECT(out[t * d + f] == z[chunk_of[t] * d + f], "dechunk rows");

  // ---- coding rate: 3 orthogonal rows h_t = s_t e_t, d = 4, eps^2 = 0.5
  const double eps2 = 0.5, alpha = 4.0 / eps2;
  const float s3[3] = {0.5f, 1.5f, 0.25f};
  std::vector<float> h(3 * d, 0.f);
  for (int t = 0; t < 3; ++t) h[t * d + t] = s3[t];
  float* dh = to_dev(h);
  float* ddr = static_cast<float*>(dev_bytes(3 * 4));
  const size_t wsr = bllm_coding_rate_workspace(1, 3, d);
  void* ws3 = dev_bytes(wsr);
  EXPECT(dh && ddr && ws3, "alloc");
  CK(hipMemset(dstat, 0, 4));
  OK(bllm_coding_rate(dh, BLLM_F32, 1, 3, d, eps2, ddr, dstat, ws3, wsr, st));
  CK(hipStreamSynchronize(st));
  const std::vector<float> dr = to_host(ddr, 3);
  for (int t = 0; t < 3; ++t) {
    const double want = 0.5 * std::log1p(alpha * s3[t] * s3[t]);
    EXPECT(std::fabs(dr[t] - want) <= 1e-5 * want, "coding rate closed form");
  }
  EXPECT(to_host(dstat, 1)[0] == 0, "coding rate status");

  // ---- coding rate of a batch (2 sequences x 16384 rows, d 64: 2 x 256 row
  // blocks): the batch's Delta R equals that of each sequence alone, bit for bit
  {
    const int64_t Tb = 16384, db2 = 64, nb = 2;
    std::vector<float> hb(nb * Tb * db2);
    uint32_t x = 12345u;
    for (auto& v : hb) {  // small integers / 64: exact in fp32
      x = x * 1664525u + 1013904223u;
      v = static_cast<float>(static_cast<int>(x >> 27) - 16) / 64.f;
    }
    float* dhb = to_dev(hb);
    float* dall = static_cast<float*>(dev_bytes(nb * Tb * 4));
    float* done = static_cast<float*>(dev_bytes(Tb * 4));
    const size_t wsb = bllm_coding_rate_workspace(nb, Tb, db2);
    void* wsbuf = dev_bytes(wsb);
    EXPECT(dhb && dall && done && wsbuf, "alloc");
    CK(hipMemset(dstat, 0, 4));
    OK(bllm_coding_rate(dhb, BLLM_F32, nb, Tb, db2, 0.5, dall, dstat, wsbuf, wsb, st));
    CK(hipStreamSynchronize(st));
    const std::vector<float> all = to_host(dall, nb * Tb);
    for (int64_t q = 0; q < nb; ++q) {
      OK(bllm_coding_rate(dhb + q * Tb * db2, BLLM_F32, 1, Tb, db2, 0.5, done, dstat, wsbuf, wsb, st));
      CK(hipStreamSynchronize(st));
      const std::vector<float> one = to_host(done, Tb);
      EXPECT(std::memcmp(one.data(), all.data() + q * Tb, Tb * 4) == 0, "batch = single sequences");
    }
    EXPECT(to_host(dstat, 1)[0] == 0, "batch status");
  }

  // ---- top-k: scores of one sequence, K = 2 -> {0, argmax of the rest}
  std::vector<float> sc = {5.f, 1.f, 7.f, 3.f};
  float* dsc = to_dev(sc);
  int32_t* dsel = static_cast<int32_t*>(dev_bytes(2 * 4));
  EXPECT(dsc && dsel, "alloc");
  OK(bllm_topk_select(dsc, 1, 4, 2, dsel, nullptr, nullptr, st));
  CK(hipStreamSynchronize(st));
  const std::vector<int32_t> sel = to_host(dsel, 2);
  EXPECT(sel[0] == 0 && sel[1] == 2, "top-k set");

  // ---- upsample with g = 0: s = h, bf16, T = 4, K = 2, d_global 32, d_local 8
  const int64_t Tu = 4, Ku = 2, dg = 32, dl = 8, nb = 16;
  std::vector<uint16_t> g(Ku * dg, 0), W(nb * dg * dl), hu(Tu * dl);
  for (size_t i = 0; i < W.size(); ++i) W[i] = bf16(static_cast<float>(i % 7) - 3.f);
  for (size_t i = 0; i < hu.size(); ++i) hu[i] = bf16(static_cast<float>(i % 11) - 5.f);
  std::vector<int32_t> uidx = {0, 2};
  uint16_t* dg_ = to_dev(g);
  uint16_t* dW = to_dev(W);
  uint16_t* dhu = to_dev(hu);
  int32_t* duidx = to_dev(uidx);
  uint16_t* ds = static_cast<uint16_t*>(dev_bytes(Tu * dl * 2));
  const size_t wsu = bllm_upsample_workspace(1, Tu, Ku, dg, dl, nb);
  void* ws4 = dev_bytes(wsu);
  EXPECT(dg_ && dW && dhu && duidx && ds && ws4, "alloc");
  OK(bllm_upsample_bins(dg_, dW, duidx, dhu, BLLM_BF16, 1, Tu, Ku, dg, dl, nb, ds, ws4, wsu, st));
  CK(hipStreamSynchronize(st));
  const std::vector<uint16_t> s = to_host(ds, Tu * dl);
  for (size_t i = 0; i < s.size(); ++i) EXPECT(s[i] == hu[i], "upsample residual");

  // ---- argument errors come back before anything is enqueued
  EXPECT(bllm_topk_select(dsc, 1, 4, 5, dsel, nullptr, nullptr, st) == BLLM_E_INVAL, "K > T");
  EXPECT(bllm_coding_rate(dh, BLLM_F32, 1, 3, d, 0.0, ddr, nullptr, ws3, wsr, st) == BLLM_E_INVAL, "eps2");

  CK(hipStreamDestroy(st));
  std::printf("abi smoke ok\n");
  return 0;
}
