// ByteFlow multi-linear upsampling with the large residual.
//
// ByteFlow paper page, method step details, stage 4, and the paper notes, key
// design 4: every byte position t falls in chunk c(t) (the last selected
// position at or before t) and, by its relative position inside that chunk,
// in one of B bins whose matrix W_b is shared by all chunks;
// s_t = h_t + g_{c(t)} W_{bin(t)}.  bin(t) = floor(B (t - s_c) / L_c).
//
// Positions of one chunk that share a bin need the same product, so the work
// items are the distinct (chunk, bin) pairs, each covering a run of
// consecutive positions.  Items are bucketed by bin (counting sort with wave
// ballots), then one grouped GEMM per bin on bf16 MFMA (v_mfma_f32_32x32x16_bf16):
// A rows are gathered from g by chunk, B = W_b (transposed once into the
// workspace so both operands are contiguous along the reduction), and the
// epilogue adds h_t and writes every position of the item's run.
#include <algorithm>

#include "common.h"

namespace bllm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChunksPerBlock = 256;
constexpr int kBM = 128, kBN = 128, kBK = 32;

struct UpGeom {
  int nseq, T, K, dg, dl, nbins, nblk;
};

// first position offset of bin b in a chunk of length L: ceil(b L / B)
__device__ inline int bin_lo(int b, int L, int B) { return (b * L + B - 1) / B; }

__device__ inline uint64_t present_bins(int L, int B) {
  uint64_t m = 0;
  for (int b = 0; b < B; ++b)
    if (bin_lo(b, L, B) < bin_lo(b + 1, L, B)) m |= uint64_t(1) << b;
  return m;
}

__device__ inline int chunk_len(const int32_t* idx, const UpGeom& g, int64_t cg) {
  const int i = static_cast<int>(cg % g.K);
  const int64_t s = cg / g.K;
  const int cur = idx[cg];
  const int nxt = i + 1 < g.K ? idx[cg + 1] : g.T;
  (void)s;
  return nxt - cur;
}

__global__ __launch_bounds__(kChunksPerBlock) void up_count(const int32_t* __restrict__ idx, UpGeom g,
                                                            int32_t* __restrict__ counts) {
  __shared__ int wc[4][64];
  const int64_t cg = static_cast<int64_t>(blockIdx.x) * kChunksPerBlock + threadIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t m = cg < static_cast<int64_t>(g.nseq) * g.K ? present_bins(chunk_len(idx, g, cg), g.nbins) : 0;
  for (int b = 0; b < g.nbins; ++b) {
    const uint64_t bal = __ballot((m >> b) & 1);
    if (lane == 0) wc[w][b] = __popcll(bal);
  }
  __syncthreads();
  if (threadIdx.x < g.nbins)
    counts[static_cast<int64_t>(blockIdx.x) * g.nbins + threadIdx.x] =
        wc[0][threadIdx.x] + wc[1][threadIdx.x] + wc[2][threadIdx.x] + wc[3][threadIdx.x];
}

// single block: per-bin totals, item offsets, tile offsets, per-block bases
__global__ __launch_bounds__(64) void up_offsets(const int32_t* __restrict__ counts, UpGeom g,
                                                 int32_t* __restrict__ base, int32_t* __restrict__ bin_off,
                                                 int32_t* __restrict__ bin_cnt, int32_t* __restrict__ tile_off) {
  __shared__ int tot[64];
  const int b = threadIdx.x;
  int sum = 0;
  if (b < g.nbins) {
    for (int k = 0; k < g.nblk; ++k) sum += counts[static_cast<int64_t>(k) * g.nbins + b];
    tot[b] = sum;
  }
  __syncthreads();
  if (b == 0) {
    int io = 0, to = 0;
    for (int q = 0; q < g.nbins; ++q) {
      bin_off[q] = io;
      bin_cnt[q] = tot[q];
      tile_off[q] = to;
      io += tot[q];
      to += (tot[q] + kBM - 1) / kBM;
    }
    tile_off[g.nbins] = to;
  }
  __syncthreads();
  if (b < g.nbins) {
    int run = bin_off[b];
    for (int k = 0; k < g.nblk; ++k) {
      base[static_cast<int64_t>(k) * g.nbins + b] = run;
      run += counts[static_cast<int64_t>(k) * g.nbins + b];
    }
  }
}

__global__ __launch_bounds__(kChunksPerBlock) void up_items(const int32_t* __restrict__ idx, UpGeom g,
                                                            const int32_t* __restrict__ base,
                                                            int4* __restrict__ items) {
  __shared__ int wc[4][64];
  const int64_t cg = static_cast<int64_t>(blockIdx.x) * kChunksPerBlock + threadIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool valid = cg < static_cast<int64_t>(g.nseq) * g.K;
  const int L = valid ? chunk_len(idx, g, cg) : 0;
  const uint64_t m = valid ? present_bins(L, g.nbins) : 0;
  int below[64];
  for (int b = 0; b < g.nbins; ++b) {
    const uint64_t bal = __ballot((m >> b) & 1);
    below[b] = lanes_below(bal);
    if (lane == 0) wc[w][b] = __popcll(bal);
  }
  __syncthreads();
  if (!valid) return;
  const int64_t s = cg / g.K;
  const int64_t row0 = s * g.T + idx[cg];
  for (int b = 0; b < g.nbins; ++b) {
    if (!((m >> b) & 1)) continue;
    int slot = base[static_cast<int64_t>(blockIdx.x) * g.nbins + b] + below[b];
    for (int q = 0; q < w; ++q) slot += wc[q][b];
    const int lo = bin_lo(b, L, g.nbins), hi = bin_lo(b + 1, L, g.nbins);
    items[slot] = make_int4(static_cast<int>(cg), static_cast<int>(row0 + lo), hi - lo, 0);
  }
}

// Wt[b][n][k] = W[b][k][n], 32x32 tiles through LDS
__global__ __launch_bounds__(256) void up_transpose(const uint16_t* __restrict__ W, int dg, int dl,
                                                    uint16_t* __restrict__ Wt) {
  __shared__ uint16_t t[32][33];
  const int b = blockIdx.z;
  const int k0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  const uint16_t* src = W + static_cast<int64_t>(b) * dg * dl;
  uint16_t* dst = Wt + static_cast<int64_t>(b) * dg * dl;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8)
    if (k0 + r < dg && n0 + tx < dl) t[r][tx] = src[static_cast<int64_t>(k0 + r) * dl + n0 + tx];
  __syncthreads();
  for (int r = ty; r < 32; r += 8)
    if (n0 + r < dl && k0 + tx < dg) dst[static_cast<int64_t>(n0 + r) * dg + k0 + tx] = t[tx][r];
}

// grouped gather-GEMM: one 128 x 128 output tile (items x d_local) per block
__global__ __launch_bounds__(256) void up_gemm(const uint16_t* __restrict__ gmat,
                                               const uint16_t* __restrict__ Wt,
                                               const uint16_t* __restrict__ h, UpGeom g,
                                               const int32_t* __restrict__ bin_off,
                                               const int32_t* __restrict__ bin_cnt,
                                               const int32_t* __restrict__ tile_off,
                                               const int4* __restrict__ items,
                                               uint16_t* __restrict__ out) {
  constexpr int LDK = kBK + 8;  // padded row (bf16 elements)
  __shared__ __attribute__((aligned(16))) uint16_t sA[kBM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kBN * LDK];
  __shared__ int4 sItem[kBM];
  const int tau = blockIdx.x;
  if (tau >= tile_off[g.nbins]) return;
  int b = 0;
  while (tile_off[b + 1] <= tau) ++b;
  const int first = (tau - tile_off[b]) * kBM;
  const int mcount = min(kBM, bin_cnt[b] - first);
  const int n0 = blockIdx.y * kBN;
  const int tid = threadIdx.x;
  if (tid < kBM) sItem[tid] = tid < mcount ? items[bin_off[b] + first + tid] : make_int4(0, 0, 0, 0);
  __syncthreads();
  const int w = tid >> 6, lane = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  floatx16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;
  // loader geometry: each thread moves 32 bytes (16 bf16) of A and of B per K step
  const int lrow = tid >> 1, lhalf = tid & 1;
  const bool arow_ok = lrow < mcount;
  const uint16_t* arow = gmat + static_cast<int64_t>(sItem[lrow].x) * g.dg + 16 * lhalf;
  const uint16_t* brow = Wt + (static_cast<int64_t>(b) * g.dl + n0 + lrow) * g.dg + 16 * lhalf;
  const bool brow_ok = n0 + lrow < g.dl;
  for (int k0 = 0; k0 < g.dg; k0 += kBK) {
    uint4 a0 = make_uint4(0, 0, 0, 0), a1 = a0, b0 = a0, b1 = a0;
    if (arow_ok) {
      a0 = *reinterpret_cast<const uint4*>(arow + k0);
      a1 = *reinterpret_cast<const uint4*>(arow + k0 + 8);
    }
    if (brow_ok) {
      b0 = *reinterpret_cast<const uint4*>(brow + k0);
      b1 = *reinterpret_cast<const uint4*>(brow + k0 + 8);
    }
    __syncthreads();
    *reinterpret_cast<uint4*>(sA + lrow * LDK + 16 * lhalf) = a0;
    *reinterpret_cast<uint4*>(sA + lrow * LDK + 16 * lhalf + 8) = a1;
    *reinterpret_cast<uint4*>(sB + lrow * LDK + 16 * lhalf) = b0;
    *reinterpret_cast<uint4*>(sB + lrow * LDK + 16 * lhalf + 8) = b1;
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ar = 64 * wm + 32 * t + (lane & 31);
        const int br = 64 * wn + 32 * t + (lane & 31);
        af[t] = *reinterpret_cast<const bf16x8*>(sA + ar * LDK + ks + 8 * (lane >> 5));
        bfr[t] = *reinterpret_cast<const bf16x8*>(sB + br * LDK + ks + 8 * (lane >> 5));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[c], acc[a][c], 0, 0, 0);
    }
  }
  // epilogue: s_t = h_t + acc for every position of the item's run
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 64 * wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int n = n0 + 64 * wn + 32 * c + (lane & 31);
        if (m >= mcount || n >= g.dl) continue;
        const int4 it = sItem[m];
        for (int e = 0; e < it.z; ++e) {
          const int64_t o = static_cast<int64_t>(it.y + e) * g.dl + n;
          out[o] = f32_to_bf16(acc[a][c][r] + bf16_to_f32(h[o]));
        }
      }
}

struct UpWs {
  int32_t *counts, *base, *bin_off, *bin_cnt, *tile_off;
  int4* items;
  uint16_t* Wt;
};

UpWs up_carve(void* ws, const UpGeom& g) {
  char* p = static_cast<char*>(ws);
  UpWs u;
  const size_t cb = align_up(static_cast<size_t>(g.nblk) * g.nbins * 4, 256);
  u.counts = reinterpret_cast<int32_t*>(p); p += cb;
  u.base = reinterpret_cast<int32_t*>(p); p += cb;
  u.bin_off = reinterpret_cast<int32_t*>(p); p += 256;
  u.bin_cnt = reinterpret_cast<int32_t*>(p); p += 256;
  u.tile_off = reinterpret_cast<int32_t*>(p); p += 512;
  u.items = reinterpret_cast<int4*>(p); p += align_up(static_cast<size_t>(g.nseq) * g.T * 16, 256);
  u.Wt = reinterpret_cast<uint16_t*>(p);
  return u;
}

size_t up_ws_bytes(const UpGeom& g) {
  const size_t cb = align_up(static_cast<size_t>(g.nblk) * g.nbins * 4, 256);
  return 2 * cb + 1024 + align_up(static_cast<size_t>(g.nseq) * g.T * 16, 256) +
         static_cast<size_t>(g.nbins) * g.dg * g.dl * 2 + 256;
}

}  // namespace
}  // namespace bllm

using namespace bllm;

extern "C" size_t bllm_upsample_workspace(int64_t nseq, int64_t T, int64_t K, int64_t d_global,
                                          int64_t d_local, int64_t nbins) {
  if (nseq < 1 || T < 1 || K < 1 || nbins < 1 || d_global < 1 || d_local < 1) return 0;
  UpGeom g{static_cast<int>(nseq), static_cast<int>(T), static_cast<int>(K), static_cast<int>(d_global),
           static_cast<int>(d_local), static_cast<int>(nbins),
           static_cast<int>(ceil_div(nseq * K, kChunksPerBlock))};
  return up_ws_bytes(g);
}

extern "C" int bllm_upsample_bins(const void* gm, const void* W, const int32_t* idx, const void* h,
                                  int dtype, int64_t nseq, int64_t T, int64_t K, int64_t d_global,
                                  int64_t d_local, int64_t nbins, void* s_out, void* ws,
                                  size_t ws_bytes, void* stream) {
  if (!gm || !W || !idx || !h || !s_out || nseq < 1 || T < 1 || K < 1 || K > T || d_global < 1 ||
      d_local < 1 || nbins < 1)
    return BLLM_E_INVAL;
  if (dtype != BLLM_BF16) return BLLM_E_NOTSUP;
  if (nbins > 64 || d_global % kBK != 0 || d_local % 8 != 0 || nseq * T >= (int64_t(1) << 31) ||
      !aligned16(gm) || !aligned16(W) || !aligned16(h) || !aligned16(s_out))
    return BLLM_E_NOTSUP;
  UpGeom g{static_cast<int>(nseq), static_cast<int>(T), static_cast<int>(K), static_cast<int>(d_global),
           static_cast<int>(d_local), static_cast<int>(nbins),
           static_cast<int>(ceil_div(nseq * K, kChunksPerBlock))};
  if (!ws || ws_bytes < up_ws_bytes(g) || !aligned16(ws)) return BLLM_E_WS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  UpWs u = up_carve(ws, g);
  hipLaunchKernelGGL(up_transpose, dim3(static_cast<unsigned>(ceil_div(d_local, 32)),
                                        static_cast<unsigned>(ceil_div(d_global, 32)),
                                        static_cast<unsigned>(nbins)),
                     dim3(256), 0, st, static_cast<const uint16_t*>(W), g.dg, g.dl, u.Wt);
  hipLaunchKernelGGL(up_count, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.counts);
  hipLaunchKernelGGL(up_offsets, dim3(1), dim3(64), 0, st, u.counts, g, u.base, u.bin_off, u.bin_cnt,
                     u.tile_off);
  hipLaunchKernelGGL(up_items, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.base, u.items);
  const int64_t max_tiles = ceil_div(nseq * T, kBM) + nbins;
  hipLaunchKernelGGL(up_gemm, dim3(static_cast<unsigned>(max_tiles), static_cast<unsigned>(ceil_div(d_local, kBN))),
                     dim3(256), 0, st, static_cast<const uint16_t*>(gm), u.Wt,
                     static_cast<const uint16_t*>(h), g, u.bin_off, u.bin_cnt, u.tile_off, u.items,
                     static_cast<uint16_t*>(s_out));
  return launch_status();
}
