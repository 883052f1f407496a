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
// 128 * kMaxRun positions.  Items are bucketed by bin (counting sort with DPP
// wave scans; a deterministic order), then one grouped GEMM per bin on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16): A rows are gathered from g by chunk, B = W_b
// as stored (read down its columns with the transposing LDS read), and the
// epilogue adds h_t and writes every position of the item's run with 16-byte
// loads and stores.
#include <algorithm>

#include "common.h"

namespace bllm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChunksPerBlock = 256;
constexpr int kMaxRun = 32;  // positions per item at most (of 8..64, 32 is fastest on 32 x 8192, K 2048)
constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kPA = kBK + 8;   // LDS pitch (bf16) of the A tile [kBM][kBK]
constexpr int kPB = kBN + 16;  // LDS pitch (bf16) of the B tile [kBK][kBN]: rows 8 banks apart
#ifndef BLLM_UP_PAIRS
#define BLLM_UP_PAIRS 2
#endif
constexpr int kPairs = BLLM_UP_PAIRS;  // epilogue pairs per thread whose loads are issued together

// row of element r held by `lane` in a 32x32 MFMA accumulator
__device__ inline int crow_of(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

struct UpGeom {
  int nseq, T, K, dg, dl, nbins, nblk;
  int cap;  // item slots of the workspace
};

// first position offset of bin b in a chunk of length L: ceil(b L / B);
// BC is B when it is known at compile time (16), else 0
template <int BC>
__device__ inline int bin_lo(int b, int L, int B) {
  if constexpr (BC > 0) return (b * L + BC - 1) / BC;
  return (b * L + B - 1) / B;
}

// first position of chunk cg inside its sequence and its length.  With the
// positions ascending from 0 (as Top-K gives them) this is idx[cg] and
// idx[cg + 1] - idx[cg]; any other input is clamped into [0, T) and an empty
// or reversed chunk has length 0, so every position written lies inside its
// sequence.
__device__ inline int chunk_span(const int32_t* idx, const UpGeom& g, int64_t cg, int& start) {
  const int i = static_cast<int>(cg % g.K);
  start = min(max(idx[cg], 0), g.T);
  const int nxt = i + 1 < g.K ? min(max(idx[cg + 1], 0), g.T) : g.T;
  return max(nxt - start, 0);
}

// items of bin b of a chunk of length L: its run split into pieces of at most kMaxRun
template <int BC>
__device__ inline int bin_pieces(int b, int L, int B) {
  return (bin_lo<BC>(b + 1, L, B) - bin_lo<BC>(b, L, B) + kMaxRun - 1) / kMaxRun;
}

// Wave sums and exclusive wave scans of counts (DPP, no LDS round trip).
__device__ inline int wave_sum_i(int v) {
  int t;
  wave_incl_scan(v, t);
  return t;
}

__device__ inline int wave_excl_i(int v) {
  int t;
  return wave_incl_scan(v, t) - v;
}

// per-block, per-bin item counts
template <int BC>
__global__ __launch_bounds__(kChunksPerBlock) void up_count(const int32_t* __restrict__ idx, UpGeom g,
                                                            int32_t* __restrict__ counts) {
  __shared__ int wc[4][64];
  const int64_t cg = static_cast<int64_t>(blockIdx.x) * kChunksPerBlock + threadIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool valid = cg < static_cast<int64_t>(g.nseq) * g.K;
  int start = 0;
  const int L = valid ? chunk_span(idx, g, cg, start) : 0;
  for (int b = 0; b < g.nbins; ++b) {
    const int n = wave_sum_i(valid ? bin_pieces<BC>(b, L, g.nbins) : 0);
    if (lane == 0) wc[w][b] = n;
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < g.nbins)
    counts[static_cast<int64_t>(blockIdx.x) * g.nbins + threadIdx.x] =
        wc[0][threadIdx.x] + wc[1][threadIdx.x] + wc[2][threadIdx.x] + wc[3][threadIdx.x];
}

// Slot bases of the items: one workgroup turns the per-block counts into,
// for every (block, bin), the first item slot of that block's items of that
// bin (all items of earlier bins, then those of earlier blocks), in place,
// and writes the bins' item offsets, counts and GEMM tile offsets.  Wave w
// scans bins w, w + 16, ... over the blocks, 64 blocks per step: a first pass
// for the bin totals, a second for the bases.
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void up_scan(UpGeom g, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ bin_off,
                                                        int32_t* __restrict__ bin_cnt,
                                                        int32_t* __restrict__ tile_off) {
  // totals and offsets in 64 bits: with positions that are not ascending,
  // chunks overlap and their items can outgrow the workspace (g.cap slots);
  // the bins are then cut at g.cap and the items past it are not written
  __shared__ int64_t sTot[64], sOff[64];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  constexpr int nw = kScanThreads / 64;
  for (int b = w; b < g.nbins; b += nw) {
    int64_t tot = 0;
    for (int k0 = 0; k0 < g.nblk; k0 += 64) {
      const int k = k0 + lane;
      tot += k < g.nblk ? counts[static_cast<int64_t>(k) * g.nbins + b] : 0;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o, 64);
    if (lane == 0) sTot[b] = tot;
  }
  __syncthreads();
  if (w == 0) {
    const int64_t tb = lane < g.nbins ? sTot[lane] : 0;
    int64_t off = tb;  // inclusive scan over the bins, then exclusive
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(off, o, 64);
      if (lane >= o) off += y;
    }
    off -= tb;
    const int cnt = static_cast<int>(min(max(static_cast<int64_t>(g.cap) - off, int64_t(0)), tb));
    const int tc = (cnt + kBM - 1) / kBM;
    const int toff = wave_excl_i(tc);
    if (lane < g.nbins) {
      sOff[lane] = off;
      bin_off[lane] = static_cast<int>(min(off, static_cast<int64_t>(g.cap)));
      bin_cnt[lane] = cnt;
      tile_off[lane] = toff;
    }
    if (lane == g.nbins - 1) tile_off[g.nbins] = toff + tc;
  }
  __syncthreads();
  for (int b = w; b < g.nbins; b += nw) {
    int64_t run = sOff[b];
    for (int k0 = 0; k0 < g.nblk; k0 += 64) {
      const int k = k0 + lane;
      int32_t* cp = counts + static_cast<int64_t>(k < g.nblk ? k : 0) * g.nbins + b;
      const int v = k < g.nblk ? *cp : 0;
      int all;
      const int x = wave_incl_scan(v, all);  // at most 64 blocks of 256 chunks of 2^20 positions: fits
      if (k < g.nblk) *cp = static_cast<int>(min(run + x - v, static_cast<int64_t>(g.cap)));
      run += all;
    }
  }
}

// Items grouped by bin, in chunk order inside each bin: each block takes its
// slot base per bin from the scanned counts.
template <int BC>
__global__ __launch_bounds__(kChunksPerBlock) void up_items(const int32_t* __restrict__ idx, UpGeom g,
                                                            const int32_t* __restrict__ base,
                                                            int4* __restrict__ items) {
  __shared__ int wc[4][64];
  __shared__ int sBase[64];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  if (tid < g.nbins) sBase[tid] = base[static_cast<int64_t>(blockIdx.x) * g.nbins + tid];
  const int64_t cg = static_cast<int64_t>(blockIdx.x) * kChunksPerBlock + tid;
  const bool valid = cg < static_cast<int64_t>(g.nseq) * g.K;
  int start = 0;
  const int L = valid ? chunk_span(idx, g, cg, start) : 0;
  for (int b = 0; b < g.nbins; ++b) {
    const int n = wave_sum_i(valid ? bin_pieces<BC>(b, L, g.nbins) : 0);
    if (lane == 0) wc[w][b] = n;
  }
  __syncthreads();
  const int64_t row0 = valid ? (cg / g.K) * g.T + start : 0;
  for (int b = 0; b < g.nbins; ++b) {
    const int np = valid ? bin_pieces<BC>(b, L, g.nbins) : 0;
    int slot = sBase[b] + wave_excl_i(np);
    for (int q = 0; q < w; ++q) slot += wc[q][b];
    const int lo = bin_lo<BC>(b, L, g.nbins), hi = bin_lo<BC>(b + 1, L, g.nbins);
    for (int e = 0; e < np; ++e) {
      const int a = lo + e * kMaxRun;
      // only chunks that overlap (positions not ascending) can need more
      // slots than the workspace holds; their extra items are dropped
      if (slot + e < g.cap)
        items[slot + e] = make_int4(static_cast<int>(cg), static_cast<int>(row0 + a), min(kMaxRun, hi - a), 0);
    }
  }
}

// Two transposing LDS reads (ds_read_b64_tr_b16) give a lane the MFMA B
// operand of a [k][n] tile: 8 consecutive k of one column n.  Within each
// 16-lane group, lane j addresses row k + j/4 (and k + 4 + j/4), columns
// col + 4 (j % 4) .. +3, and lane i receives column i of those 4 rows; with
// row = 8 (lane / 32) + (lane % 16) / 4 and col = 16 ((lane / 16) % 2) +
// 4 (lane % 4) added to the tile origin, lane l gets column l % 32 and
// rows 8 (l / 32) .. +7.
typedef short shortx4 __attribute__((ext_vector_type(4)));

__device__ inline uint4 and4(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }

__device__ inline bf16x8 tr_frag(const uint16_t* s, int row, int col, int pitch) {
  typedef __attribute__((address_space(3))) shortx4 lds_s4;
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(s + row * pitch + col));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(s + (row + 4) * pitch + col));
  bf16x8 v;
  __builtin_memcpy(&v, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&v) + 8, &hi, 8);
  return v;
}

// grouped gather-GEMM: one 128 x 128 output tile (items x d_local) per block;
// four waves in 2 x 2, each a 64 x 64 quadrant of 2 x 2 MFMA 32x32 tiles.
// A rows are gathered from g by chunk; B is W_b in its stored [k][n] layout,
// staged row-major and read with the transposing LDS read.
// Block numbering: workgroup L runs on XCD L % 8, so the column tiles of one
// row tile are given ids 8 apart inside a group of 8 * ncol consecutive ids.
// They then run at about the same time on the same XCD and the gathered g
// rows of the row tile come from HBM into that XCD's L2 once.
template <bool FULLK>
__global__ __launch_bounds__(256, 3) void up_gemm(const uint16_t* gmat,
                                               const uint16_t* W,
                                               const uint16_t* __restrict__ h, UpGeom g,
                                               const int32_t* __restrict__ bin_off,
                                               const int32_t* __restrict__ bin_cnt,
                                               const int32_t* __restrict__ tile_off,
                                               const int4* __restrict__ items, int ncol,
                                               uint16_t* __restrict__ out) {
  constexpr int kOLD = kBN + 4;  // fp32 row stride of the epilogue staging area
  __shared__ __attribute__((aligned(16))) uint16_t smem[kBM * kPA + kBK * kPB];
  __shared__ int4 sItem[kBM];
  uint16_t* sA = smem;
  uint16_t* sB = smem + kBM * kPA;
  float* sO = reinterpret_cast<float*>(smem);  // [64][kOLD] fp32, reused after the K loop
  static_assert(64 * kOLD * 4 <= (kBM * kPA + kBK * kPB) * 2, "epilogue staging must fit");
  const int grp = blockIdx.x / (8 * ncol), rem = blockIdx.x % (8 * ncol);
  const int tau_f = 8 * grp + (rem & 7);
  if (tau_f >= tile_off[g.nbins]) return;
  const int tau = tile_off[g.nbins] - 1 - tau_f;  // last bins first: they hold the longest runs
  int b = 0;
  while (b + 1 < g.nbins && tile_off[b + 1] <= tau) ++b;
  const int64_t first = (static_cast<int64_t>(tau) - tile_off[b]) * kBM;
  const int mcount = static_cast<int>(
      min(static_cast<int64_t>(kBM), max(static_cast<int64_t>(bin_cnt[b]) - first, int64_t(0))));
  const int n0 = (rem >> 3) * kBN;
  const int tid = threadIdx.x;
  if (tid < kBM) {
    // a plan made by the plan kernels always passes these bounds; they keep a
    // workspace that holds no plan (bllm_upsample_apply alone) in bounds too
    int4 it = make_int4(0, 0, 0, 0);
    const int64_t slot = static_cast<int64_t>(bin_off[b]) + first + tid;
    if (tid < mcount && slot >= 0 && slot < g.cap) {
      it = items[slot];
      it.x = min(max(it.x, 0), g.nseq * g.K - 1);
      it.y = min(max(it.y, 0), g.nseq * g.T - 1);
      it.z = min(max(it.z, 0), min(kMaxRun, g.nseq * g.T - it.y));
    }
    sItem[tid] = it;
  }
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
  // A loader: thread moves rows lr + 32*q (q = 0..3), 16-byte column chunk lc;
  // B loader: K rows kr + 16*q of W_b, 16-byte column chunk nc (columns past
  // d_local read a valid column, their results are not written);
  // the next K step's operands are in flight in named registers during the MFMAs
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const int kr = tid >> 4, nc = (tid & 15) * 8;
  const uint16_t* ar0 = gmat + static_cast<int64_t>(sItem[lr].x) * g.dg + lc;
  const uint16_t* ar1 = gmat + static_cast<int64_t>(sItem[lr + 32].x) * g.dg + lc;
  const uint16_t* ar2 = gmat + static_cast<int64_t>(sItem[lr + 64].x) * g.dg + lc;
  const uint16_t* ar3 = gmat + static_cast<int64_t>(sItem[lr + 96].x) * g.dg + lc;
  const uint16_t* wb = W + static_cast<int64_t>(b) * g.dg * g.dl + min(n0 + nc, g.dl - 8);
  // A rows (gathered g rows) are prefetched two K steps ahead in two named
  // register sets used in turn (the loop takes steps in pairs, so every wait
  // count is static and leaves the later set's loads in flight); W_b rows,
  // which every row tile of the bin shares, one step ahead.
  uint4 pa0, pa1, pa2, pa3, qa0, qa1, qa2, qa3, pb0, pb1, pb2, pb3;
  // Every load is issued (rows past the items read chunk 0's g row, whose
  // results are not written; K past d_global, only in a last partial step,
  // reads column or row 0; steps past the last reload it).  The masks that
  // zero that K range are applied when the registers are stored to LDS: applied
  // here, they would make every load wait for its data at once and the
  // prefetch would not overlap the MFMAs.
  const int nk = (g.dg + kBK - 1) / kBK;
  auto fetch_a = [&](int kt, uint4& x0, uint4& x1, uint4& x2, uint4& x3) {
    const int ko = min(kt, nk - 1) * kBK;
    const int koa = FULLK || ko + lc < g.dg ? ko : 0;
    x0 = *reinterpret_cast<const uint4*>(ar0 + koa);
    x1 = *reinterpret_cast<const uint4*>(ar1 + koa);
    x2 = *reinterpret_cast<const uint4*>(ar2 + koa);
    x3 = *reinterpret_cast<const uint4*>(ar3 + koa);
  };
  auto fetch_b = [&](int kt) {
    const int ko = min(kt, nk - 1) * kBK;
    const int k0 = ko + kr, k1 = k0 + 16, k2 = k0 + 32, k3 = k0 + 48;
    pb0 = *reinterpret_cast<const uint4*>(wb + static_cast<int64_t>(FULLK || k0 < g.dg ? k0 : 0) * g.dl);
    pb1 = *reinterpret_cast<const uint4*>(wb + static_cast<int64_t>(FULLK || k1 < g.dg ? k1 : 0) * g.dl);
    pb2 = *reinterpret_cast<const uint4*>(wb + static_cast<int64_t>(FULLK || k2 < g.dg ? k2 : 0) * g.dl);
    pb3 = *reinterpret_cast<const uint4*>(wb + static_cast<int64_t>(FULLK || k3 < g.dg ? k3 : 0) * g.dl);
  };
  const int j16 = lane & 15;
  const int frow = 8 * (lane >> 5) + (j16 >> 2);
  const int fcol = 64 * wn + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
  // one K step: stage A (from the given set) and B, then issue the next B and
  // the A two steps ahead into the same set, then multiply
  auto step = [&](int kt, uint4& x0, uint4& x1, uint4& x2, uint4& x3) {
    const int ko = kt * kBK;
    // with d_global a multiple of the K step every staged value is in range
    const uint32_t ma = FULLK || ko + lc < g.dg ? 0xFFFFFFFFu : 0u;
    auto mb = [&](int k) { return FULLK || ko + k < g.dg ? 0xFFFFFFFFu : 0u; };
    __syncthreads();
    *reinterpret_cast<uint4*>(sA + lr * kPA + lc) = and4(x0, ma);
    *reinterpret_cast<uint4*>(sA + (lr + 32) * kPA + lc) = and4(x1, ma);
    *reinterpret_cast<uint4*>(sA + (lr + 64) * kPA + lc) = and4(x2, ma);
    *reinterpret_cast<uint4*>(sA + (lr + 96) * kPA + lc) = and4(x3, ma);
    *reinterpret_cast<uint4*>(sB + kr * kPB + nc) = and4(pb0, mb(kr));
    *reinterpret_cast<uint4*>(sB + (kr + 16) * kPB + nc) = and4(pb1, mb(kr + 16));
    *reinterpret_cast<uint4*>(sB + (kr + 32) * kPB + nc) = and4(pb2, mb(kr + 32));
    *reinterpret_cast<uint4*>(sB + (kr + 48) * kPB + nc) = and4(pb3, mb(kr + 48));
    __syncthreads();
    fetch_b(kt + 1);
    // keeps the next B rows ahead of the A rows in issue order, so that the
    // next step's wait for B leaves these A loads in flight
    __asm__ volatile("" ::: "memory");
    fetch_a(kt + 2, x0, x1, x2, x3);
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = *reinterpret_cast<const bf16x8*>(sA + (64 * wm + 32 * t + (lane & 31)) * kPA + ks + 8 * (lane >> 5));
        bfr[t] = tr_frag(sB, ks + frow, fcol + 32 * t, kPB);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[c], acc[a][c], 0, 0, 0);
    }
  };
  fetch_b(0);
  fetch_a(0, pa0, pa1, pa2, pa3);
  fetch_a(1, qa0, qa1, qa2, qa3);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, pa0, pa1, pa2, pa3);
    step(kt + 1, qa0, qa1, qa2, qa3);
  }
  if (kt < nk) step(kt, pa0, pa1, pa2, pa3);
  // epilogue, one pass per row half p (rows 64p..64p+63, written by the waves
  // with wm == p): stage the fp32 accumulators in LDS, then add h and write
  // every position of each item's run with 16-byte accesses.
  // The pass's work is cut into units of (4-position group of an item's run,
  // 8-column chunk), so that a few long runs do not leave most threads idle:
  // one wave numbers the groups of the pass's 64 items (an exclusive scan of
  // ceil(run / 4)) into a group -> (item, group) map in LDS while the waves
  // with wm == p stage their accumulators; then every thread takes units in
  // steps of 256, kPairs of them with all their loads in flight together.
  uint16_t* gmap = reinterpret_cast<uint16_t*>(sO + 64 * kOLD);  // [512]: item << 3 | group
  __shared__ int sGroups;
  static_assert(64 * kOLD * 4 + 512 * 2 <= (kBM * kPA + kBK * kPB) * 2, "epilogue staging and map must fit");
  static_assert(kMaxRun <= 32, "at most 8 groups of 4 positions per item");
  const int nchunk = min(kBN, g.dl - n0) / 8;
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
    } else if (wn == 0) {
      const int rows = min(64, max(0, mcount - 64 * p));
      const int ng = lane < rows ? (sItem[64 * p + lane].z + 3) >> 2 : 0;
      int total;
      const int g0 = wave_incl_scan(ng, total) - ng;
      for (int k = 0; k < ng; ++k) gmap[g0 + k] = static_cast<uint16_t>((lane << 3) | k);
      if (lane == 0) sGroups = total;
    }
    __syncthreads();
    const int nunits = sGroups * nchunk;
    for (int v0 = tid; v0 < nunits; v0 += kPairs * 256) {
      int np[kPairs], so[kPairs];
      int64_t o0[kPairs];
      uint4 hv[kPairs][4];
#pragma unroll
      for (int j = 0; j < kPairs; ++j) {
        const int v = v0 + j * 256;
        const int vv = v < nunits ? v : v0;
        const int gi = vv / nchunk, ch = vv - gi * nchunk;
        const int m = gmap[gi];
        const int r = m >> 3, grp4 = 4 * (m & 7);
        const int4 it = sItem[64 * p + r];
        np[j] = v < nunits ? min(4, it.z - grp4) : 0;
        so[j] = r * kOLD + 8 * ch;
        o0[j] = (static_cast<int64_t>(it.y) + grp4) * g.dl + n0 + 8 * ch;
        const int last = max(np[j], 1) - 1;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hv[j][e] = *reinterpret_cast<const uint4*>(h + o0[j] + static_cast<int64_t>(min(e, last)) * g.dl);
      }
#pragma unroll
      for (int j = 0; j < kPairs; ++j) {
        float acc8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc8[e] = sO[so[j] + e];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e >= np[j]) break;
          const uint32_t wv[4] = {hv[j][e].x, hv[j][e].y, hv[j][e].z, hv[j][e].w};
          float sv[8];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            sv[2 * c] = acc8[2 * c] + bf16_to_f32(static_cast<uint16_t>(wv[c] & 0xFFFFu));
            sv[2 * c + 1] = acc8[2 * c + 1] + bf16_to_f32(static_cast<uint16_t>(wv[c] >> 16));
          }
          Vec<BLLM_BF16>::store(out, o0[j] + static_cast<int64_t>(e) * g.dl, sv);
        }
      }
    }
  }
}

struct UpWs {
  int32_t *counts, *bin_off, *bin_cnt, *tile_off;
  int4* items;
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
  u.bin_off = reinterpret_cast<int32_t*>(p); p += 256;
  u.bin_cnt = reinterpret_cast<int32_t*>(p); p += 256;
  u.tile_off = reinterpret_cast<int32_t*>(p); p += 512;
  u.items = reinterpret_cast<int4*>(p);
  return u;
}

size_t up_ws_bytes(const UpGeom& g) {
  const size_t cb = align_up(static_cast<size_t>(g.nblk) * g.nbins * 4, 256);
  return cb + 1024 + align_up(up_max_items(g) * 16, 256) + 256;
}

}  // namespace
}  // namespace bllm

using namespace bllm;

extern "C" size_t bllm_upsample_workspace(int64_t nseq, int64_t T, int64_t K, int64_t d_global,
                                          int64_t d_local, int64_t nbins) {
  if (nseq < 1 || T < 1 || K < 1 || nbins < 1 || d_global < 1 || d_local < 1) return 0;
  UpGeom g{static_cast<int>(nseq), static_cast<int>(T), static_cast<int>(K), static_cast<int>(d_global),
           static_cast<int>(d_local), static_cast<int>(nbins),
           static_cast<int>(ceil_div(nseq * K, kChunksPerBlock)), 0};
  return up_ws_bytes(g);
}

// Shapes and the workspace of an upsample: BLLM_OK and the geometry, or the
// error the entry points return.
static int up_setup(int64_t nseq, int64_t T, int64_t K, int64_t nbins, const void* ws, size_t ws_bytes,
                    UpGeom* out) {
  if (nseq < 1 || T < 1 || K < 1 || K > T || nbins < 1) return BLLM_E_INVAL;
  if (nbins > 64 || nseq * T >= (int64_t(1) << 31) || T > (int64_t(1) << 20)) return BLLM_E_NOTSUP;
  UpGeom g{static_cast<int>(nseq), static_cast<int>(T), static_cast<int>(K), 0, 0, static_cast<int>(nbins),
           static_cast<int>(ceil_div(nseq * K, kChunksPerBlock)), 0};
  if (up_max_items(g) > static_cast<size_t>(INT32_MAX)) return BLLM_E_NOTSUP;
  g.cap = static_cast<int>(up_max_items(g));
  if (!ws || ws_bytes < up_ws_bytes(g) || !aligned16(ws)) return BLLM_E_WS;
  *out = g;
  return BLLM_OK;
}

static void up_plan_launch(const int32_t* idx, const UpGeom& g, const UpWs& u, hipStream_t st) {
  if (g.nbins == 16) {
    hipLaunchKernelGGL(up_count<16>, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.counts);
    hipLaunchKernelGGL(up_scan, dim3(1), dim3(kScanThreads), 0, st, g, u.counts, u.bin_off, u.bin_cnt, u.tile_off);
    hipLaunchKernelGGL(up_items<16>, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.counts, u.items);
  } else {
    hipLaunchKernelGGL(up_count<0>, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.counts);
    hipLaunchKernelGGL(up_scan, dim3(1), dim3(kScanThreads), 0, st, g, u.counts, u.bin_off, u.bin_cnt, u.tile_off);
    hipLaunchKernelGGL(up_items<0>, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.counts, u.items);
  }
}

static void up_apply_launch(const void* gm, const void* W, const void* h, const UpGeom& g, const UpWs& u,
                            void* s_out, hipStream_t st) {
  const int64_t max_tiles = ceil_div(static_cast<int64_t>(up_max_items(g)), kBM) + g.nbins;
  const int ncol = static_cast<int>(ceil_div(g.dl, kBN));
  const int64_t nblocks = ceil_div(max_tiles, 8) * 8 * ncol;
  if (g.dg % kBK == 0)
    hipLaunchKernelGGL(up_gemm<true>, dim3(static_cast<unsigned>(nblocks)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(gm), static_cast<const uint16_t*>(W),
                     static_cast<const uint16_t*>(h), g, u.bin_off,
                     u.bin_cnt, u.tile_off, u.items, ncol, static_cast<uint16_t*>(s_out));
  else
    hipLaunchKernelGGL(up_gemm<false>, dim3(static_cast<unsigned>(nblocks)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(gm), static_cast<const uint16_t*>(W),
                     static_cast<const uint16_t*>(h), g, u.bin_off,
                     u.bin_cnt, u.tile_off, u.items, ncol, static_cast<uint16_t*>(s_out));
}

// the apply's own arguments: every BLLM_E_INVAL condition of the call is
// checked before any BLLM_E_NOTSUP one
static int up_apply_args(const void* gm, const void* W, const void* h, int dtype, int64_t nseq, int64_t T,
                         int64_t K, int64_t d_global, int64_t d_local, int64_t nbins, void* s_out) {
  if (!gm || !W || !h || !s_out || d_global < 1 || d_local < 1 || nseq < 1 || T < 1 || K < 1 || K > T ||
      nbins < 1)
    return BLLM_E_INVAL;
  if (dtype != BLLM_BF16) return BLLM_E_NOTSUP;
  if (d_global % 8 != 0 || d_local % 8 != 0 || d_global >= (int64_t(1) << 20) || d_local >= (int64_t(1) << 20) ||
      !aligned16(gm) || !aligned16(W) || !aligned16(h) || !aligned16(s_out))
    return BLLM_E_NOTSUP;
  return BLLM_OK;
}

extern "C" int bllm_upsample_plan(const int32_t* idx, int64_t nseq, int64_t T, int64_t K, int64_t nbins,
                                  void* ws, size_t ws_bytes, void* stream) {
  if (!idx) return BLLM_E_INVAL;
  UpGeom g{};
  const int rc = up_setup(nseq, T, K, nbins, ws, ws_bytes, &g);
  if (rc != BLLM_OK) return rc;
  up_plan_launch(idx, g, up_carve(ws, g), static_cast<hipStream_t>(stream));
  return launch_status();
}

extern "C" int bllm_upsample_apply(const void* gm, const void* W, const void* h, int dtype, int64_t nseq,
                                   int64_t T, int64_t K, int64_t d_global, int64_t d_local, int64_t nbins,
                                   void* s_out, const void* ws, size_t ws_bytes, void* stream) {
  int rc = up_apply_args(gm, W, h, dtype, nseq, T, K, d_global, d_local, nbins, s_out);
  if (rc != BLLM_OK) return rc;
  UpGeom g{};
  rc = up_setup(nseq, T, K, nbins, ws, ws_bytes, &g);
  if (rc != BLLM_OK) return rc;
  g.dg = static_cast<int>(d_global);
  g.dl = static_cast<int>(d_local);
  up_apply_launch(gm, W, h, g, up_carve(const_cast<void*>(ws), g), s_out, static_cast<hipStream_t>(stream));
  return launch_status();
}

extern "C" int bllm_upsample_bins(const void* gm, const void* W, const int32_t* idx, const void* h,
                                  int dtype, int64_t nseq, int64_t T, int64_t K, int64_t d_global,
                                  int64_t d_local, int64_t nbins, void* s_out, void* ws,
                                  size_t ws_bytes, void* stream) {
  if (!idx) return BLLM_E_INVAL;
  int rc = up_apply_args(gm, W, h, dtype, nseq, T, K, d_global, d_local, nbins, s_out);
  if (rc != BLLM_OK) return rc;
  UpGeom g{};
  rc = up_setup(nseq, T, K, nbins, ws, ws_bytes, &g);
  if (rc != BLLM_OK) return rc;
  g.dg = static_cast<int>(d_global);
  g.dl = static_cast<int>(d_local);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const UpWs u = up_carve(ws, g);
  up_plan_launch(idx, g, u, st);
  up_apply_launch(gm, W, h, g, u, s_out, st);
  return launch_status();
}
