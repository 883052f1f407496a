// ByteFlow Top-K boundary selection.
//
// ByteFlow paper page, method step details, stage 2 (and the paper notes, key
// design 2): the first position is always kept (BOS); the K-1 positions with
// the largest marginal coding rate among the rest are added; the set is
// returned in time order.  A fixed K keeps every output the same size.
//
// A later window of a stream (the local Top-K of a streaming chunker, which
// the paper page's weakness analysis suggests for autoregressive inference)
// forces no position: its K largest scores are kept.
//
// One workgroup (1024 threads) per sequence.  Scores become order-preserving
// uint32 keys (NaN -> 0, the lowest; -0 -> +0), an 8-bit radix select finds
// the key of the (K-1)-th largest, ties at that key are resolved by time order
// with a block scan, and a second block scan compacts the chosen positions in
// time order.  Up to kLdsKeys positions the keys are kept in LDS; longer
// sequences (up to 64 positions per thread) recompute them from the scores,
// which stay in L2, in every pass.
#include <algorithm>

#include "common.h"

namespace bllm {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kLdsKeys = 16384;                 // keys kept in LDS (64 KB) up to this length
constexpr int kMaxT = 64 * kTopkThreads;        // one 64-bit selection word per thread

__device__ inline uint32_t order_key(float x, bool* nan) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) { *nan = true; return 0u; }
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive scan over the 1024 threads of one int each
__device__ inline int block_excl_scan1024(int v, int* sh, int* tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int wt;
  const int x = wave_incl_scan(v, wt);
  if (lane == 63) sh[w] = x;
  __syncthreads();
  if (w == 0) {
    const int y = lane < 16 ? sh[lane] : 0;
    int all;
    const int inc = wave_incl_scan(y, all);
    if (lane < 16) sh[16 + lane] = inc - y;
    if (lane == 15) sh[32] = inc;
  }
  __syncthreads();
  const int r = sh[16 + w] + x - v;
  *tot = sh[32];
  __syncthreads();
  return r;
}

template <bool kInLds>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ score, int T,
                                                            int K, int bos, int32_t* __restrict__ idx_out,
                                                            uint8_t* __restrict__ mask_out,
                                                            int32_t* __restrict__ status) {
  extern __shared__ uint32_t lkeys[];  // [T] when kInLds
  __shared__ uint32_t hist[256];
  __shared__ int scan_sh[40];
  __shared__ uint32_t sel_prefix, sel_want;
  const int s = blockIdx.x;
  const float* sc = score + static_cast<int64_t>(s) * T;
  bool nan = false;
  for (int t = threadIdx.x; t < T; t += blockDim.x) {
    const uint32_t k = t == 0 && bos ? 0u : order_key(sc[t], &nan);
    if (kInLds) lkeys[t] = k;
  }
  if (nan && status) atomicOr(status, BLLM_S_NONFINITE);
  auto key = [&](int t) {
    if (kInLds) return lkeys[t];
    bool ignored = false;
    return t == 0 && bos ? 0u : order_key(sc[t], &ignored);
  };
  const int per = (T + kTopkThreads - 1) / kTopkThreads;
  const int t0 = threadIdx.x * per;
  const int t1 = min(t0 + per, T);
  const int want0 = K - bos;  // positions chosen by score; 0 is forced when bos
  if (threadIdx.x == 0) { sel_prefix = 0; sel_want = static_cast<uint32_t>(want0); }
  __syncthreads();
  uint32_t kth = 0xFFFFFFFFu, take_eq = 0;
  if (want0 > 0) {
    uint32_t mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
      __syncthreads();
      const uint32_t prefix = sel_prefix;
      // each wave takes 64 consecutive keys at a time (no LDS bank
      // conflicts); the scores crowd into few digits, so the lanes that
      // share the first active lane's digit add with one atomic
      const int lane = threadIdx.x & 63;
      for (int base = bos + static_cast<int>(threadIdx.x) - lane; base < T; base += kTopkThreads) {
        const int t = base + lane;
        const uint32_t kt = t < T ? key(t) : 0u;
        const bool act = t < T && (kt & mask) == prefix;
        const uint32_t dg = act ? (kt >> shift) & 0xFFu : 0u;
        const uint64_t am = __ballot(act);
        if (am == 0) continue;
        const int fl = __ffsll(static_cast<unsigned long long>(am)) - 1;
        const uint32_t d0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dg), fl));
        const uint64_t m0 = __ballot(act && dg == d0);
        if (lane == fl) atomicAdd(&hist[d0], static_cast<uint32_t>(__popcll(m0)));
        if (act && dg != d0) atomicAdd(&hist[dg], 1u);
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        // lane l owns digits 255-4l .. 252-4l (descending)
        const int l = threadIdx.x;
        uint32_t c[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { c[q] = hist[255 - 4 * l - q]; sum += c[q]; }
        int all;  // counts of at most kMaxT keys: the int scan is exact
        const uint32_t inc = static_cast<uint32_t>(wave_incl_scan(static_cast<int>(sum), all));
        const uint32_t want = sel_want;
        const uint32_t above = inc - sum;
        if (above < want && want <= inc) {
          uint32_t cum = above;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (cum < want && want <= cum + c[q]) {
              sel_want = want - cum;
              sel_prefix = prefix | (static_cast<uint32_t>(255 - 4 * l - q) << shift);
            }
            cum += c[q];
          }
        }
      }
      mask |= 0xFFu << shift;
      __syncthreads();
    }
    kth = sel_prefix;
    take_eq = sel_want;  // how many keys equal to kth are taken (earliest first)
  }
  // rank of each equal key in time order
  int neq = 0;
  for (int t = max(t0, bos); t < t1; ++t) neq += key(t) == kth;
  int tot;
  int eq_rank = block_excl_scan1024(neq, scan_sh, &tot);
  int nsel = 0;
  uint64_t selbits = 0;  // per <= 64
  for (int t = t0; t < t1; ++t) {
    bool sel;
    const uint32_t kt = key(t);
    if (t == 0 && bos) sel = true;
    else if (want0 <= 0) sel = false;
    else if (kt > kth) sel = true;
    else if (kt == kth) sel = static_cast<uint32_t>(eq_rank++) < take_eq;
    else sel = false;
    if (sel) { selbits |= uint64_t(1) << (t - t0); ++nsel; }
  }
  int pos = block_excl_scan1024(nsel, scan_sh, &tot);
  int32_t* out = idx_out + static_cast<int64_t>(s) * K;
  for (int t = t0; t < t1; ++t) {
    const bool sel = (selbits >> (t - t0)) & 1u;
    if (sel && pos < K) out[pos++] = t;
    if (mask_out) mask_out[static_cast<int64_t>(s) * T + t] = sel;
  }
}

// z = the hidden states at the selected positions, per sequence in time
// order (the paper page's stage 2 gather, before the global model): one
// group of G lanes per output row, 16-byte copies, grid-stride over rows.
// An index outside [0, T) is clamped into it, so no read leaves h.
__global__ __launch_bounds__(256) void gather_topk_kernel(const uint8_t* __restrict__ h, int64_t T, int64_t K,
                                                          int64_t nrows, int row_bytes, int gshift,
                                                          const int32_t* __restrict__ idx,
                                                          uint8_t* __restrict__ z) {
  const int G = 1 << gshift;
  const int g = threadIdx.x & (G - 1);
  const int64_t groups = static_cast<int64_t>(gridDim.x) * (blockDim.x >> gshift);
  const int nvec = row_bytes / 16;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> gshift) + (threadIdx.x >> gshift); r < nrows;
       r += groups) {
    const int64_t t = min(max(static_cast<int64_t>(idx[r]), int64_t(0)), T - 1);
    const int64_t src = (r / K) * T + t;
    const uint4* sp = reinterpret_cast<const uint4*>(h + src * row_bytes);
    uint4* o = reinterpret_cast<uint4*>(z + r * row_bytes);
    for (int v = g; v < nvec; v += G) o[v] = sp[v];
  }
}

}  // namespace
}  // namespace bllm

using namespace bllm;

static int topk_entry(const float* score, int64_t nseq, int64_t T, int64_t K, int bos, int32_t* idx_out,
                      uint8_t* mask_out, int32_t* status, void* stream) {
  if (!score || !idx_out || nseq < 1 || T < 1 || K < 1 || K > T) return BLLM_E_INVAL;
  if (T > kMaxT || nseq > 0x7FFFFFFF) return BLLM_E_NOTSUP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (T <= kLdsKeys)
    hipLaunchKernelGGL(topk_kernel<true>, dim3(static_cast<unsigned>(nseq)), dim3(kTopkThreads),
                       static_cast<size_t>(T) * 4, st, score, static_cast<int>(T), static_cast<int>(K), bos,
                       idx_out, mask_out, status);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3(static_cast<unsigned>(nseq)), dim3(kTopkThreads), 0, st,
                       score, static_cast<int>(T), static_cast<int>(K), bos, idx_out, mask_out, status);
  return launch_status();
}

extern "C" int bllm_topk_select(const float* score, int64_t nseq, int64_t T, int64_t K,
                                int32_t* idx_out, uint8_t* mask_out, int32_t* status,
                                void* stream) {
  return topk_entry(score, nseq, T, K, 1, idx_out, mask_out, status, stream);
}

extern "C" int bllm_topk_select_window(const float* score, int64_t nseq, int64_t W, int64_t K, int first,
                                       int32_t* idx_out, uint8_t* mask_out, int32_t* status, void* stream) {
  return topk_entry(score, nseq, W, K, first ? 1 : 0, idx_out, mask_out, status, stream);
}

extern "C" int bllm_gather_topk(const void* h, int dtype, int64_t nseq, int64_t T, int64_t d, int64_t K,
                                const int32_t* idx, void* z_out, void* stream) {
  if (!h || !idx || !z_out || nseq < 1 || T < 1 || d < 1 || K < 1 || K > T) return BLLM_E_INVAL;
  if (!valid_dtype(dtype)) return BLLM_E_NOTSUP;
  const int64_t row_bytes = d * elem_size(dtype);
  if (row_bytes % 16 != 0 || row_bytes > (int64_t(1) << 20) || !aligned16(h) || !aligned16(z_out))
    return BLLM_E_NOTSUP;
  if (nseq * T >= (int64_t(1) << 31)) return BLLM_E_NOTSUP;
  const int nvec = static_cast<int>(row_bytes / 16);
  int gshift = 0;
  while ((1 << gshift) < nvec && gshift < 6) ++gshift;
  const int64_t nrows = nseq * K;
  const int rows_per_block = 256 >> gshift;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(ceil_div(nrows, rows_per_block), 16384));
  hipLaunchKernelGGL(gather_topk_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(h), T, K, nrows, static_cast<int>(row_bytes), gshift, idx,
                     static_cast<uint8_t*>(z_out));
  return launch_status();
}
