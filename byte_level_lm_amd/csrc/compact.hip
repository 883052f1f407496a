// Boundary compaction over a packed ragged batch.
//
// ByteGen report, section 2.3: the chosen boundary positions are kept and the
// rest dropped, giving a shorter ragged sequence per stream (nested tensors,
// no padding).  The same call performs ByteFlow's gather z = [h_{s_1}..h_{s_K}]
// (paper page, method step details, stage 2) when the mask is the Top-K mask.
//
// Three launches: per-tile counts, per-tile wave-ballot prefix + scatter of
// idx/P/chunk offsets, then a row gather with one lane group per kept row.
// The scatter finds the number of kept positions before its tile by a
// look-back over the tile words: the count kernel stores every tile's count,
// and a scatter block replaces its tile's word by the inclusive prefix (flag
// bit set) as soon as it knows it; a block sums the counts of the tiles
// before it, 64 words per step, back to the nearest inclusive prefix.  Every
// count is in memory before the scatter starts, so no block ever waits on
// another, and the look-back is short because tiles finish roughly in order.
// HBM-bound: 1 byte read per position, then (M/N)(8 + 2*d*e) bytes per position.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.h"

namespace bllm {
namespace {

constexpr int kTile = 4096;  // positions per tile: 256 threads x 16 bytes

__device__ inline uint32_t load_flags16(const uint8_t* mask, int64_t pos0, int64_t total) {
  uint32_t f = 0;
  if (pos0 + 16 <= total) {
    const uint4 v = *reinterpret_cast<const uint4*>(mask + pos0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((w[i] >> (8 * j)) & 0xFFu) f |= 1u << (4 * i + j);
  } else {
    for (int e = 0; e < 16; ++e)
      if (pos0 + e < total && mask[pos0 + e]) f |= 1u << e;
  }
  return f;
}

// first s in [0, n] with a[s] >= x
__device__ inline int lower_seq(const int64_t* a, int n, int64_t x) {
  int lo = 0, hi = n + 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// exclusive block scan of one int per thread (blockDim = 256); returns the block total in *tot
__device__ inline int block_excl_scan256(int v, int* sh, int* tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int wt;
  const int x = wave_incl_scan(v, wt);
  if (lane == 63) sh[w] = x;
  __syncthreads();
  int wbase = 0, all = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) wbase += sh[i];
    all += sh[i];
  }
  __syncthreads();
  *tot = all;
  return wbase + x - v;
}

constexpr uint64_t kInclusive = uint64_t(1) << 63;  // tile word holds the inclusive prefix

__global__ __launch_bounds__(256) void compact_count(const uint8_t* __restrict__ mask,
                                                     int64_t total, uint64_t* __restrict__ words) {
  __shared__ int sh[4];
  const int64_t pos0 = static_cast<int64_t>(blockIdx.x) * kTile + threadIdx.x * 16;
  const int c = __popc(load_flags16(mask, pos0, total));
  int tot;
  block_excl_scan256(c, sh, &tot);
  if (threadIdx.x == 0) words[blockIdx.x] = static_cast<uint64_t>(tot);
}

// number of kept positions in tiles [0, tile): the first wave walks the tile
// words backwards 64 at a time (lane j reads tile t - j) and stops at the
// nearest word that holds an inclusive prefix (tiles below 0 count as an
// inclusive 0); every tile's count is already in memory, so nothing waits
__device__ inline int64_t tiles_before(const uint64_t* words, int64_t tile) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  for (int64_t t = tile - 1;; t -= 64) {
    const int64_t i = t - lane;
    const uint64_t w = i >= 0 ? __hip_atomic_load(words + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : kInclusive;
    const uint64_t incl = __ballot((w & kInclusive) != 0);
    const int stop = incl ? __builtin_ctzll(incl) : 64;
    int64_t v = lane <= stop ? static_cast<int64_t>(w & ~kInclusive) : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    base += v;
    if (incl) return base;
  }
}

__global__ __launch_bounds__(256) void compact_scatter(
    const uint8_t* __restrict__ mask, const float* __restrict__ p, const int64_t* __restrict__ offsets,
    int nseq, int64_t total, int64_t capacity, uint64_t* __restrict__ words,
    int32_t* __restrict__ idx_out, int64_t* __restrict__ chunk_offsets, float* __restrict__ P_out,
    int64_t* __restrict__ m_out, int32_t* __restrict__ status) {
  __shared__ int sh[4];
  __shared__ int64_t sbase;
  const int tile = blockIdx.x;
  const int64_t pos0 = static_cast<int64_t>(tile) * kTile + threadIdx.x * 16;
  const uint32_t f = load_flags16(mask, pos0, total);
  if (threadIdx.x < 64) {
    const int64_t b = tiles_before(words, tile);
    if (threadIdx.x == 0) sbase = b;
  }
  int tile_tot;
  const int64_t local = block_excl_scan256(__popc(f), sh, &tile_tot);  // its barriers also publish sbase
  const int64_t base = sbase;
  if (threadIdx.x == 0)
    __hip_atomic_store(words + tile, kInclusive | static_cast<uint64_t>(base + tile_tot), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  const int64_t mine = base + local;
  uint32_t rest = f;
  int64_t r = mine;
  while (rest) {
    const int e = __ffs(rest) - 1;
    rest &= rest - 1;
    if (r < capacity) {
      idx_out[r] = static_cast<int32_t>(pos0 + e);
      if (P_out) P_out[r] = p[pos0 + e];
    }
    ++r;
  }
  if (pos0 < total) {
    for (int s = lower_seq(offsets, nseq, pos0); s < nseq && offsets[s] < pos0 + 16 && offsets[s] < total; ++s) {
      const int e = static_cast<int>(offsets[s] - pos0);
      chunk_offsets[s] = mine + __popc(f & ((1u << e) - 1u));
    }
  }
  if (tile == static_cast<int>(gridDim.x) - 1 && threadIdx.x == 0) {
    const int64_t M = base + tile_tot;
    *m_out = M;
    for (int s = lower_seq(offsets, nseq, total); s <= nseq; ++s) chunk_offsets[s] = M;
    if (M > capacity && status) atomicOr(status, BLLM_S_CAPACITY);
  }
}

// copy kept rows: one group of G lanes per row, grid-stride over rows
__global__ __launch_bounds__(256) void compact_gather(const uint8_t* __restrict__ rows, int row_bytes,
                                                      int gshift, const int32_t* __restrict__ idx,
                                                      const int64_t* __restrict__ m_in, int64_t capacity,
                                                      uint8_t* __restrict__ rows_out) {
  const int G = 1 << gshift;
  const int g = threadIdx.x & (G - 1);
  const int64_t M = min(*m_in, capacity);
  const int64_t groups = static_cast<int64_t>(gridDim.x) * (blockDim.x >> gshift);
  const int nvec = row_bytes / 16;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> gshift) + (threadIdx.x >> gshift);
       r < M; r += groups) {
    const int64_t src = idx[r];
    const uint4* s = reinterpret_cast<const uint4*>(rows + src * row_bytes);
    uint4* o = reinterpret_cast<uint4*>(rows_out + r * row_bytes);
    for (int v = g; v < nvec; v += G) o[v] = s[v];
  }
}

// workspace: the tile words, then the total count M
constexpr size_t compact_ws_bytes(int64_t total) {
  return (static_cast<size_t>((total + kTile - 1) / kTile + 1) * 8 + 255) / 256 * 256 + 256;
}

// ------------------------------------------------------------- no-allocation variant
// bllm_compact_noalloc runs the same kernels on a scratch array of this file
// (device memory of the library, one copy per GPU, held until the process
// ends) instead of a workspace argument, for callers that cannot allocate.
// The kernels write every word of the scratch they later read (the count
// kernel stores each tile's word, the scatter stores M), so nothing needs
// clearing between calls.  Calls that overlap on one GPU share the array and
// race.
constexpr int64_t kNoAllocMaxTotal = int64_t(1) << 27;  // 134M positions
constexpr size_t kNoAllocScratchBytes = compact_ws_bytes(kNoAllocMaxTotal);  // 262,656 bytes
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch[kMaxDevices];

// The device address of `scratch` on the GPU that runs `st`, looked up once
// per device with that device current; nullptr if it cannot be found.
void* scratch_for(hipStream_t st) {
  int dev = 0;
  if (st ? hipStreamGetDevice(st, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch[dev].load(std::memory_order_relaxed);
  if (ptr) return ptr;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  bool ok = cur == dev || hipSetDevice(dev) == hipSuccess;
  ok = ok && hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr != nullptr;
  if (cur != dev && hipSetDevice(cur) != hipSuccess) ok = false;
  if (!ok) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace
}  // namespace bllm

using namespace bllm;

extern "C" size_t bllm_compact_workspace(int64_t total) { return compact_ws_bytes(total); }

// argument checks shared by both entry points (host only, before any HIP call)
static int compact_args(const uint8_t* mask, const float* p, const void* rows, int dtype, int64_t d,
                        const int64_t* offsets, int64_t nseq, int64_t total, int64_t capacity,
                        const int32_t* idx_out, const int64_t* chunk_offsets_out, const void* rows_out,
                        const float* P_out) {
  if (!offsets || !chunk_offsets_out || nseq < 1 || total < 0 || capacity < 0) return BLLM_E_INVAL;
  if (total > 0 && (!mask || (capacity > 0 && !idx_out))) return BLLM_E_INVAL;  // NULL allowed when empty
  if ((rows && !rows_out) || (p && !P_out)) return BLLM_E_INVAL;
  if (rows) {
    if (d < 1) return BLLM_E_INVAL;
    if (!valid_dtype(dtype)) return BLLM_E_NOTSUP;
    if ((d * elem_size(dtype)) % 16 != 0 || !aligned16(rows) || !aligned16(rows_out))
      return BLLM_E_NOTSUP;
  }
  if (!aligned16(mask)) return BLLM_E_NOTSUP;
  if (total >= (int64_t(1) << 31) || nseq >= (int64_t(1) << 30)) return BLLM_E_NOTSUP;
  return BLLM_OK;
}

extern "C" int bllm_compact(const uint8_t* mask, const float* p, const void* rows, int dtype,
                            int64_t d, const int64_t* offsets, int64_t nseq, int64_t total,
                            int64_t capacity, int32_t* idx_out, int64_t* chunk_offsets_out,
                            void* rows_out, float* P_out, int32_t* status, void* ws,
                            size_t ws_bytes, void* stream) {
  const int rc = compact_args(mask, p, rows, dtype, d, offsets, nseq, total, capacity, idx_out,
                              chunk_offsets_out, rows_out, P_out);
  if (rc != BLLM_OK) return rc;
  if (!ws || ws_bytes < bllm_compact_workspace(total) || !aligned16(ws)) return BLLM_E_WS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t ntiles = ceil_div(total, kTile);
  uint64_t* words = static_cast<uint64_t*>(ws);
  int64_t* m_dev = reinterpret_cast<int64_t*>(static_cast<char*>(ws) +
                                              align_up(static_cast<size_t>(ntiles + 1) * 8, 256));
  if (total == 0) {
    hipLaunchKernelGGL(fill_i64, dim3(1), dim3(256), 0, st, chunk_offsets_out, nseq + 1, int64_t(0));
    hipLaunchKernelGGL(fill_i64, dim3(1), dim3(64), 0, st, m_dev, int64_t(1), int64_t(0));
    return launch_status();
  }
  hipLaunchKernelGGL(compact_count, dim3(static_cast<unsigned>(ntiles)), dim3(256), 0, st, mask,
                     total, words);
  hipLaunchKernelGGL(compact_scatter, dim3(static_cast<unsigned>(ntiles)), dim3(256), 0, st, mask, p,
                     offsets, static_cast<int>(nseq), total, capacity, words, idx_out,
                     chunk_offsets_out, P_out, m_dev, status);
  if (rows && capacity > 0) {
    const int row_bytes = static_cast<int>(d * elem_size(dtype));
    const int nvec = row_bytes / 16;
    int gshift = 0;
    while ((1 << gshift) < nvec && gshift < 6) ++gshift;
    const int rows_per_block = 256 >> gshift;
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>(ceil_div(capacity, rows_per_block), 16384));
    hipLaunchKernelGGL(compact_gather, dim3(grid), dim3(256), 0, st,
                       static_cast<const uint8_t*>(rows), row_bytes, gshift, idx_out, m_dev, capacity,
                       static_cast<uint8_t*>(rows_out));
  }
  return launch_status();
}

extern "C" int bllm_compact_noalloc(const uint8_t* mask, const float* p, const void* rows, int dtype,
                                    int64_t d, const int64_t* offsets, int64_t nseq, int64_t total,
                                    int64_t capacity, int32_t* idx_out, int64_t* chunk_offsets_out,
                                    void* rows_out, float* P_out, int32_t* status, void* stream) {
  const int rc = compact_args(mask, p, rows, dtype, d, offsets, nseq, total, capacity, idx_out,
                              chunk_offsets_out, rows_out, P_out);
  if (rc != BLLM_OK) return rc;
  if (total > kNoAllocMaxTotal) return BLLM_E_WS;  // the scratch holds the tile words of 2^27 positions
  void* ws = scratch_for(static_cast<hipStream_t>(stream));
  if (!ws) return BLLM_E_HIP;
  return bllm_compact(mask, p, rows, dtype, d, offsets, nseq, total, capacity, idx_out, chunk_offsets_out,
                      rows_out, P_out, status, ws, kNoAllocScratchBytes, stream);
}
