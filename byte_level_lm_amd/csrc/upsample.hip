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
// consecutive positions; runs longer than kMaxRun positions (long chunks) are
// split into several items, so no GEMM tile's epilogue carries much more than
// 128 * kMaxRun positions.  Items are bucketed by bin (counting sort with wave
// ballots; a deterministic order), then one grouped GEMM per bin on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16): A rows are gathered from g by chunk, B = W_b
// (transposed once into the workspace so both operands are contiguous along
// the reduction), and the epilogue adds h_t and writes every position of the
// item's run with 16-byte loads and stores.
#include <algorithm>

#include "common.h"

namespace bllm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChunksPerBlock = 256;
constexpr int kMaxRun = 16;
constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLDK = kBK + 8;  // LDS row stride (bf16) of the operand tiles

// row of element r held by `lane` in a 32x32 MFMA accumulator
__device__ inline int crow_of(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

struct UpGeom {
  int nseq, T, K, dg, dl, nbins, nblk;
};

// first position offset of bin b in a chunk of length L: ceil(b L / B)
__device__ inline int bin_lo(int b, int L, int B) { return (b * L + B - 1) / B; }


__device__ inline int chunk_len(const int32_t* idx, const UpGeom& g, int64_t cg) {
  const int i = static_cast<int>(cg % g.K);
  const int nxt = i + 1 < g.K ? idx[cg + 1] : g.T;
  return nxt - idx[cg];
}

// items of bin b of a chunk of length L: its run split into pieces of at most kMaxRun
__device__ inline int bin_pieces(int b, int L, int B) {
  return (bin_lo(b + 1, L, B) - bin_lo(b, L, B) + kMaxRun - 1) / kMaxRun;
}

__device__ inline int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ inline int wave_excl_i(int v, int lane) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x - v;
}

// per-block, per-bin item counts
__global__ __launch_bounds__(kChunksPerBlock) void up_count(const int32_t* __restrict__ idx, UpGeom g,
                                                            int32_t* __restrict__ counts) {
  __shared__ int wc[4][64];
  const int64_t cg = static_cast<int64_t>(blockIdx.x) * kChunksPerBlock + threadIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool valid = cg < static_cast<int64_t>(g.nseq) * g.K;
  const int L = valid ? chunk_len(idx, g, cg) : 0;
  for (int b = 0; b < g.nbins; ++b) {
    const int n = wave_sum_i(valid ? bin_pieces(b, L, g.nbins) : 0);
    if (lane == 0) wc[w][b] = n;
  }
  __syncthreads();
  if (threadIdx.x < g.nbins)
    counts[static_cast<int64_t>(blockIdx.x) * g.nbins + threadIdx.x] =
        wc[0][threadIdx.x] + wc[1][threadIdx.x] + wc[2][threadIdx.x] + wc[3][threadIdx.x];
}

// single block: per-bin running offsets of every count block, bin offsets and
// tile offsets.  Counts are staged through LDS in chunks of 64 blocks.
__global__ __launch_bounds__(256) void up_offsets(const int32_t* __restrict__ counts, UpGeom g,
                                                  int32_t* __restrict__ base, int32_t* __restrict__ bin_off,
                                                  int32_t* __restrict__ bin_cnt, int32_t* __restrict__ tile_off) {
  constexpr int CB = 64;
  __shared__ int sc[CB][65];
  __shared__ int tot[64];
  const int tid = threadIdx.x;
  int run = 0;
  for (int k0 = 0; k0 < g.nblk; k0 += CB) {
    const int nk = min(CB, g.nblk - k0);
    __syncthreads();
    for (int e = tid; e < nk * g.nbins; e += blockDim.x)
      sc[e / g.nbins][e % g.nbins] = counts[static_cast<int64_t>(k0) * g.nbins + e];
    __syncthreads();
    if (tid < g.nbins) {
      for (int k = 0; k < nk; ++k) {
        base[static_cast<int64_t>(k0 + k) * g.nbins + tid] = run;
        run += sc[k][tid];
      }
    }
  }
  if (tid < g.nbins) tot[tid] = run;
  __syncthreads();
  if (tid == 0) {
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
  for (int64_t e = tid; e < static_cast<int64_t>(g.nblk) * g.nbins; e += blockDim.x)
    base[e] += bin_off[e % g.nbins];
}

// items grouped by bin, in chunk order inside each bin
__global__ __launch_bounds__(kChunksPerBlock) void up_items(const int32_t* __restrict__ idx, UpGeom g,
                                                            const int32_t* __restrict__ base,
                                                            int4* __restrict__ items) {
  __shared__ int wc[4][64];
  const int64_t cg = static_cast<int64_t>(blockIdx.x) * kChunksPerBlock + threadIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool valid = cg < static_cast<int64_t>(g.nseq) * g.K;
  const int L = valid ? chunk_len(idx, g, cg) : 0;
  for (int b = 0; b < g.nbins; ++b) {
    const int n = wave_sum_i(valid ? bin_pieces(b, L, g.nbins) : 0);
    if (lane == 0) wc[w][b] = n;
  }
  __syncthreads();
  const int64_t row0 = valid ? (cg / g.K) * g.T + idx[cg] : 0;
  for (int b = 0; b < g.nbins; ++b) {
    const int np = valid ? bin_pieces(b, L, g.nbins) : 0;
    int slot = base[static_cast<int64_t>(blockIdx.x) * g.nbins + b] + wave_excl_i(np, lane);
    for (int q = 0; q < w; ++q) slot += wc[q][b];
    const int lo = bin_lo(b, L, g.nbins), hi = bin_lo(b + 1, L, g.nbins);
    for (int e = 0; e < np; ++e) {
      const int a = lo + e * kMaxRun;
      items[slot + e] = make_int4(static_cast<int>(cg), static_cast<int>(row0 + a), min(kMaxRun, hi - a), 0);
    }
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

// grouped gather-GEMM: one 128 x 128 output tile (items x d_local) per block;
// four waves in 2 x 2, each a 64 x 64 quadrant of 2 x 2 MFMA 32x32 tiles.
__global__ __launch_bounds__(256) void up_gemm(const uint16_t* __restrict__ gmat,
                                               const uint16_t* __restrict__ Wt,
                                               const uint16_t* __restrict__ h, UpGeom g,
                                               const int32_t* __restrict__ bin_off,
                                               const int32_t* __restrict__ bin_cnt,
                                               const int32_t* __restrict__ tile_off,
                                               const int4* __restrict__ items,
                                               uint16_t* __restrict__ out) {
  constexpr int kOLD = kBN + 4;  // fp32 row stride of the epilogue staging area
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kBM * kLDK];
  __shared__ int4 sItem[kBM];
  uint16_t* sA = smem;
  uint16_t* sB = smem + kBM * kLDK;
  float* sO = reinterpret_cast<float*>(smem);  // [64][kOLD] fp32, reused after the K loop
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
  // loader: thread moves rows lr + 32*q (q = 0..3), 16-byte column chunk lc;
  // the next K step's operands are in flight in named registers during the MFMAs
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const uint16_t* ar0 = gmat + static_cast<int64_t>(sItem[lr].x) * g.dg + lc;
  const uint16_t* ar1 = gmat + static_cast<int64_t>(sItem[lr + 32].x) * g.dg + lc;
  const uint16_t* ar2 = gmat + static_cast<int64_t>(sItem[lr + 64].x) * g.dg + lc;
  const uint16_t* ar3 = gmat + static_cast<int64_t>(sItem[lr + 96].x) * g.dg + lc;
  const uint16_t* wb = Wt + static_cast<int64_t>(b) * g.dl * g.dg + lc;
  const int nr0 = min(n0 + lr, g.dl - 1), nr1 = min(n0 + lr + 32, g.dl - 1);
  const int nr2 = min(n0 + lr + 64, g.dl - 1), nr3 = min(n0 + lr + 96, g.dl - 1);
  const uint16_t* br0 = wb + static_cast<int64_t>(nr0) * g.dg;
  const uint16_t* br1 = wb + static_cast<int64_t>(nr1) * g.dg;
  const uint16_t* br2 = wb + static_cast<int64_t>(nr2) * g.dg;
  const uint16_t* br3 = wb + static_cast<int64_t>(nr3) * g.dg;
  const bool a0 = lr < mcount, a1 = lr + 32 < mcount, a2 = lr + 64 < mcount, a3 = lr + 96 < mcount;
  const bool b0 = n0 + lr < g.dl, b1 = n0 + lr + 32 < g.dl, b2 = n0 + lr + 64 < g.dl, b3 = n0 + lr + 96 < g.dl;
  const uint4 z4 = make_uint4(0, 0, 0, 0);
  uint4 pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3;
  auto fetch = [&](int ko) {
    const bool kin = ko + lc < g.dg;
    pa0 = a0 && kin ? *reinterpret_cast<const uint4*>(ar0 + ko) : z4;
    pa1 = a1 && kin ? *reinterpret_cast<const uint4*>(ar1 + ko) : z4;
    pa2 = a2 && kin ? *reinterpret_cast<const uint4*>(ar2 + ko) : z4;
    pa3 = a3 && kin ? *reinterpret_cast<const uint4*>(ar3 + ko) : z4;
    pb0 = b0 && kin ? *reinterpret_cast<const uint4*>(br0 + ko) : z4;
    pb1 = b1 && kin ? *reinterpret_cast<const uint4*>(br1 + ko) : z4;
    pb2 = b2 && kin ? *reinterpret_cast<const uint4*>(br2 + ko) : z4;
    pb3 = b3 && kin ? *reinterpret_cast<const uint4*>(br3 + ko) : z4;
  };
  fetch(0);
  const int nk = (g.dg + kBK - 1) / kBK;
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    *reinterpret_cast<uint4*>(sA + lr * kLDK + lc) = pa0;
    *reinterpret_cast<uint4*>(sA + (lr + 32) * kLDK + lc) = pa1;
    *reinterpret_cast<uint4*>(sA + (lr + 64) * kLDK + lc) = pa2;
    *reinterpret_cast<uint4*>(sA + (lr + 96) * kLDK + lc) = pa3;
    *reinterpret_cast<uint4*>(sB + lr * kLDK + lc) = pb0;
    *reinterpret_cast<uint4*>(sB + (lr + 32) * kLDK + lc) = pb1;
    *reinterpret_cast<uint4*>(sB + (lr + 64) * kLDK + lc) = pb2;
    *reinterpret_cast<uint4*>(sB + (lr + 96) * kLDK + lc) = pb3;
    __syncthreads();
    if (kt + 1 < nk) fetch((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = *reinterpret_cast<const bf16x8*>(sA + (64 * wm + 32 * t + (lane & 31)) * kLDK + ks + 8 * (lane >> 5));
        bfr[t] = *reinterpret_cast<const bf16x8*>(sB + (64 * wn + 32 * t + (lane & 31)) * kLDK + ks + 8 * (lane >> 5));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[c], acc[a][c], 0, 0, 0);
    }
  }
  // epilogue, one pass per row half p (rows 64p..64p+63, written by the waves
  // with wm == p): stage the fp32 accumulators in LDS, then add h and write
  // every position of each item's run with 16-byte accesses.
  for (int p = 0; p < 2; ++p) {
    __syncthreads();
    if (wm == p) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sO[(32 * a + crow_of(r, lane)) * kOLD + 64 * wn + 32 * c + (lane & 31)] = acc[a][c][r];
    }
    __syncthreads();
    // one (item row, 8-column chunk) pair per thread and round: the pair's
    // 8 accumulator values are read once and its run (at most kMaxRun
    // positions) is written four positions at a time, all four h loads
    // issued before any is used
    const int nchunk = min(kBN, g.dl - n0) / 8;
    const int rows = min(64, max(0, mcount - 64 * p));
    for (int v = tid; v < rows * nchunk; v += 256) {
      const int r = v / nchunk, ch = v - r * nchunk;
      const int4 it = sItem[64 * p + r];
      float acc8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc8[e] = sO[r * kOLD + 8 * ch + e];
      const int64_t o0 = static_cast<int64_t>(it.y) * g.dl + n0 + 8 * ch;
      for (int q0 = 0; q0 < it.z; q0 += 4) {
        uint4 hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q = min(q0 + e, it.z - 1);  // past the run: reload its last position
          hv[e] = *reinterpret_cast<const uint4*>(h + o0 + static_cast<int64_t>(q) * g.dl);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (q0 + e >= it.z) break;
          const uint32_t wv[4] = {hv[e].x, hv[e].y, hv[e].z, hv[e].w};
          float sv[8];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            sv[2 * c] = acc8[2 * c] + bf16_to_f32(static_cast<uint16_t>(wv[c] & 0xFFFFu));
            sv[2 * c + 1] = acc8[2 * c + 1] + bf16_to_f32(static_cast<uint16_t>(wv[c] >> 16));
          }
          Vec<BLLM_BF16>::store(out, o0 + static_cast<int64_t>(q0 + e) * g.dl, sv);
        }
      }
    }
  }
}

struct UpWs {
  int32_t *counts, *base, *bin_off, *bin_cnt, *tile_off;
  int4* items;
  uint16_t* Wt;
};

// items per chunk <= min(L, B) + L / kMaxRun (one per present bin, one more
// per kMaxRun positions of its run), so per sequence <= T + T / kMaxRun
size_t up_max_items(const UpGeom& g) {
  return static_cast<size_t>(g.nseq) * (static_cast<size_t>(g.T) + g.T / kMaxRun + 1);
}

UpWs up_carve(void* ws, const UpGeom& g) {
  char* p = static_cast<char*>(ws);
  UpWs u;
  const size_t cb = align_up(static_cast<size_t>(g.nblk) * g.nbins * 4, 256);
  u.counts = reinterpret_cast<int32_t*>(p); p += cb;
  u.base = reinterpret_cast<int32_t*>(p); p += cb;
  u.bin_off = reinterpret_cast<int32_t*>(p); p += 256;
  u.bin_cnt = reinterpret_cast<int32_t*>(p); p += 256;
  u.tile_off = reinterpret_cast<int32_t*>(p); p += 512;
  u.items = reinterpret_cast<int4*>(p); p += align_up(up_max_items(g) * 16, 256);
  u.Wt = reinterpret_cast<uint16_t*>(p);
  return u;
}

size_t up_ws_bytes(const UpGeom& g) {
  const size_t cb = align_up(static_cast<size_t>(g.nblk) * g.nbins * 4, 256);
  return 2 * cb + 1024 + align_up(up_max_items(g) * 16, 256) +
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
  if (nbins > 64 || d_global % 8 != 0 || d_local % 8 != 0 || nseq * T >= (int64_t(1) << 31) ||
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
  hipLaunchKernelGGL(up_offsets, dim3(1), dim3(256), 0, st, u.counts, g, u.base, u.bin_off, u.bin_cnt,
                     u.tile_off);
  hipLaunchKernelGGL(up_items, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.base, u.items);
  const int64_t max_tiles = ceil_div(static_cast<int64_t>(up_max_items(g)), kBM) + nbins;
  hipLaunchKernelGGL(up_gemm, dim3(static_cast<unsigned>(max_tiles), static_cast<unsigned>(ceil_div(d_local, kBN))),
                     dim3(256), 0, st, static_cast<const uint16_t*>(gm), u.Wt,
                     static_cast<const uint16_t*>(h), g, u.bin_off, u.bin_cnt, u.tile_off, u.items,
                     static_cast<uint16_t*>(s_out));
  return launch_status();
}
