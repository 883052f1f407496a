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
// uint32 keys in LDS (NaN -> 0, the lowest; -0 -> +0), an 8-bit radix select
// finds the key of the (K-1)-th largest, ties at that key are resolved by time
// order with a block scan, and a second block scan compacts the chosen
// positions in time order.
#include "common.h"

namespace bllm {
namespace {

constexpr int kTopkThreads = 1024;

__device__ inline uint32_t order_key(float x, bool* nan) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) { *nan = true; return 0u; }
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive scan over the 1024 threads of one int each
__device__ inline int block_excl_scan1024(int v, int* sh, int* tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  if (w == 0) {
    int y = lane < 16 ? sh[lane] : 0;
    int inc = y;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int z = __shfl_up(inc, off, 64);
      if (lane >= off) inc += z;
    }
    if (lane < 16) sh[16 + lane] = inc - y;
    if (lane == 15) sh[32] = inc;
  }
  __syncthreads();
  const int r = sh[16 + w] + x - v;
  *tot = sh[32];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ score, int T,
                                                            int K, int bos, int32_t* __restrict__ idx_out,
                                                            uint8_t* __restrict__ mask_out,
                                                            int32_t* __restrict__ status) {
  extern __shared__ uint32_t keys[];  // [T]
  __shared__ uint32_t hist[256];
  __shared__ int scan_sh[40];
  __shared__ uint32_t sel_prefix, sel_want;
  const int s = blockIdx.x;
  const float* sc = score + static_cast<int64_t>(s) * T;
  bool nan = false;
  for (int t = threadIdx.x; t < T; t += blockDim.x) keys[t] = t == 0 && bos ? 0u : order_key(sc[t], &nan);
  if (nan && status) atomicOr(status, BLLM_S_NONFINITE);
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
        const bool act = t < T && (keys[t] & mask) == prefix;
        const uint32_t dg = act ? (keys[t] >> shift) & 0xFFu : 0u;
        const uint64_t am = __ballot(act);
        if (am == 0) continue;
        const int fl = __ffsll(static_cast<unsigned long long>(am)) - 1;
        const uint32_t d0 = __shfl(dg, fl, 64);
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
        uint32_t inc = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t z = __shfl_up(inc, off, 64);
          if (l >= off) inc += z;
        }
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
  for (int t = max(t0, bos); t < t1; ++t) neq += keys[t] == kth;
  int tot;
  int eq_rank = block_excl_scan1024(neq, scan_sh, &tot);
  int nsel = 0;
  uint32_t selbits = 0;  // per <= 32
  for (int t = t0; t < t1; ++t) {
    bool sel;
    if (t == 0 && bos) sel = true;
    else if (want0 <= 0) sel = false;
    else if (keys[t] > kth) sel = true;
    else if (keys[t] == kth) sel = static_cast<uint32_t>(eq_rank++) < take_eq;
    else sel = false;
    if (sel) { selbits |= 1u << (t - t0); ++nsel; }
  }
  int pos = block_excl_scan1024(nsel, scan_sh, &tot);
  int32_t* out = idx_out + static_cast<int64_t>(s) * K;
  for (int t = t0; t < t1; ++t) {
    const bool sel = (selbits >> (t - t0)) & 1u;
    if (sel && pos < K) out[pos++] = t;
    if (mask_out) mask_out[static_cast<int64_t>(s) * T + t] = sel;
  }
}

}  // namespace
}  // namespace bllm

using namespace bllm;

static int topk_entry(const float* score, int64_t nseq, int64_t T, int64_t K, int bos, int32_t* idx_out,
                      uint8_t* mask_out, int32_t* status, void* stream) {
  if (!score || !idx_out || nseq < 1 || T < 1 || K < 1 || K > T) return BLLM_E_INVAL;
  if (T > 16384 || nseq > 0x7FFFFFFF) return BLLM_E_NOTSUP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t shmem = static_cast<size_t>(T) * 4;
  hipLaunchKernelGGL(topk_kernel, dim3(static_cast<unsigned>(nseq)), dim3(kTopkThreads), shmem, st,
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
