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
};

// first position offset of bin b in a chunk of length L: ceil(b L / B);
// BC is B when it is known at compile time (16), else 0
template <int BC>
__device__ inline int bin_lo(int b, int L, int B) {
  if constexpr (BC > 0) return (b * L + BC - 1) / BC;
  return (b * L + B - 1) / B;
}

__device__ inline int chunk_len(const int32_t* idx, const UpGeom& g, int64_t cg) {
  const int i = static_cast<int>(cg % g.K);
  const int nxt = i + 1 < g.K ? idx[cg + 1] : g.T;
  return nxt - idx[cg];
}

// items of bin b of a chunk of length L: its run split into pieces of at most kMaxRun
template <int BC>
__device__ inline int bin_pieces(int b, int L, int B) {
  return (bin_lo<BC>(b + 1, L, B) - bin_lo<BC>(b, L, B) + kMaxRun - 1) / kMaxRun;
}

// Wave sum and exclusive wave scan of small counts.  A lane holds at most one
// item per bin unless its run exceeds kMaxRun positions, so the common case
// is a ballot and a popcount (mbcnt); otherwise shuffles.
__device__ inline int wave_sum_i(int v) {
  if (__ballot(v > 1) == 0) return __popcll(__ballot(v == 1));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ inline int wave_excl_i(int v, int lane) {
  if (__ballot(v > 1) == 0) {
    const uint64_t m = __ballot(v == 1);
    return __popcll(m & ((uint64_t(1) << lane) - 1));
  }
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x - v;
}

// per-block, per-bin item counts
template <int BC>
__global__ __launch_bounds__(kChunksPerBlock) void up_count(const int32_t* __restrict__ idx, UpGeom g,
                                                            int32_t* __restrict__ counts) {
  __shared__ int wc[4][64];
  const int64_t cg = static_cast<int64_t>(blockIdx.x) * kChunksPerBlock + threadIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool valid = cg < static_cast<int64_t>(g.nseq) * g.K;
  const int L = valid ? chunk_len(idx, g, cg) : 0;
  for (int b = 0; b < g.nbins; ++b) {
    const int n = wave_sum_i(valid ? bin_pieces<BC>(b, L, g.nbins) : 0);
    if (lane == 0) wc[w][b] = n;
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < g.nbins)
    counts[static_cast<int64_t>(blockIdx.x) * g.nbins + threadIdx.x] =
        wc[0][threadIdx.x] + wc[1][threadIdx.x] + wc[2][threadIdx.x] + wc[3][threadIdx.x];
}

// Items grouped by bin, in chunk order inside each bin.  Each block first
// derives its own slot base per bin from all blocks' counts (the items of
// earlier blocks, after all items of earlier bins); block 0 also writes the
// bins' item offsets, counts and GEMM tile offsets.
template <int BC>
__global__ __launch_bounds__(kChunksPerBlock) void up_items(const int32_t* __restrict__ idx, UpGeom g,
                                                            const int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ bin_off,
                                                            int32_t* __restrict__ bin_cnt,
                                                            int32_t* __restrict__ tile_off,
                                                            int4* __restrict__ items) {
  __shared__ int wc[4][64];
  __shared__ int sBefore[4][64], sTot[4][64], sBase[64];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  {
    // lane = bin; wave w sums blocks [16 w, 16 w + 16) of every 64, sixteen
    // independent loads in flight at a time
    int before = 0, tot = 0;
    for (int k0 = 16 * w; k0 < g.nblk; k0 += 64) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int k = k0 + j;
        v[j] = lane < g.nbins && k < g.nblk ? counts[static_cast<int64_t>(k) * g.nbins + lane] : 0;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        tot += v[j];
        if (k0 + j < static_cast<int>(blockIdx.x)) before += v[j];
      }
    }
    sBefore[w][lane] = before;
    sTot[w][lane] = tot;
  }
  const int64_t cg = static_cast<int64_t>(blockIdx.x) * kChunksPerBlock + tid;
  const bool valid = cg < static_cast<int64_t>(g.nseq) * g.K;
  const int L = valid ? chunk_len(idx, g, cg) : 0;
  for (int b = 0; b < g.nbins; ++b) {
    const int n = wave_sum_i(valid ? bin_pieces<BC>(b, L, g.nbins) : 0);
    if (lane == 0) wc[w][b] = n;
  }
  __syncthreads();
  if (w == 0) {
    const int tb = sTot[0][lane] + sTot[1][lane] + sTot[2][lane] + sTot[3][lane];
    const int off = wave_excl_i(tb, lane);
    sBase[lane] = off + sBefore[0][lane] + sBefore[1][lane] + sBefore[2][lane] + sBefore[3][lane];
    if (blockIdx.x == 0) {
      const int tc = (tb + kBM - 1) / kBM;
      const int toff = wave_excl_i(tc, lane);
      if (lane < g.nbins) {
        bin_off[lane] = off;
        bin_cnt[lane] = tb;
        tile_off[lane] = toff;
      }
      if (lane == g.nbins - 1) tile_off[g.nbins] = toff + tc;
    }
  }
  __syncthreads();
  const int64_t row0 = valid ? (cg / g.K) * g.T + idx[cg] : 0;
  for (int b = 0; b < g.nbins; ++b) {
    const int np = valid ? bin_pieces<BC>(b, L, g.nbins) : 0;
    int slot = sBase[b] + wave_excl_i(np, lane);
    for (int q = 0; q < w; ++q) slot += wc[q][b];
    const int lo = bin_lo<BC>(b, L, g.nbins), hi = bin_lo<BC>(b + 1, L, g.nbins);
    for (int e = 0; e < np; ++e) {
      const int a = lo + e * kMaxRun;
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
__global__ __launch_bounds__(256) void up_gemm(const uint16_t* __restrict__ gmat,
                                               const uint16_t* __restrict__ W,
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
  while (tile_off[b + 1] <= tau) ++b;
  const int first = (tau - tile_off[b]) * kBM;
  const int mcount = min(kBM, bin_cnt[b] - first);
  const int n0 = (rem >> 3) * kBN;
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
  uint4 pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3;
  // Every load is issued (rows past the items read chunk 0's g row, whose
  // results are not written); K past d_global, only in a last partial step,
  // is masked to zero.
  auto fetch = [&](int ko) {
    const bool kin = ko + lc < g.dg;
    const uint32_t ma = kin ? 0xFFFFFFFFu : 0u;
    const int koa = kin ? ko : 0;
    pa0 = and4(*reinterpret_cast<const uint4*>(ar0 + koa), ma);
    pa1 = and4(*reinterpret_cast<const uint4*>(ar1 + koa), ma);
    pa2 = and4(*reinterpret_cast<const uint4*>(ar2 + koa), ma);
    pa3 = and4(*reinterpret_cast<const uint4*>(ar3 + koa), ma);
    const int k0 = ko + kr, k1 = k0 + 16, k2 = k0 + 32, k3 = k0 + 48;
    pb0 = and4(*reinterpret_cast<const uint4*>(wb + static_cast<int64_t>(k0 < g.dg ? k0 : 0) * g.dl),
               k0 < g.dg ? 0xFFFFFFFFu : 0u);
    pb1 = and4(*reinterpret_cast<const uint4*>(wb + static_cast<int64_t>(k1 < g.dg ? k1 : 0) * g.dl),
               k1 < g.dg ? 0xFFFFFFFFu : 0u);
    pb2 = and4(*reinterpret_cast<const uint4*>(wb + static_cast<int64_t>(k2 < g.dg ? k2 : 0) * g.dl),
               k2 < g.dg ? 0xFFFFFFFFu : 0u);
    pb3 = and4(*reinterpret_cast<const uint4*>(wb + static_cast<int64_t>(k3 < g.dg ? k3 : 0) * g.dl),
               k3 < g.dg ? 0xFFFFFFFFu : 0u);
  };
  const int j16 = lane & 15;
  const int frow = 8 * (lane >> 5) + (j16 >> 2);
  const int fcol = 64 * wn + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
  fetch(0);
  const int nk = (g.dg + kBK - 1) / kBK;
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    *reinterpret_cast<uint4*>(sA + lr * kPA + lc) = pa0;
    *reinterpret_cast<uint4*>(sA + (lr + 32) * kPA + lc) = pa1;
    *reinterpret_cast<uint4*>(sA + (lr + 64) * kPA + lc) = pa2;
    *reinterpret_cast<uint4*>(sA + (lr + 96) * kPA + lc) = pa3;
    *reinterpret_cast<uint4*>(sB + kr * kPB + nc) = pb0;
    *reinterpret_cast<uint4*>(sB + (kr + 16) * kPB + nc) = pb1;
    *reinterpret_cast<uint4*>(sB + (kr + 32) * kPB + nc) = pb2;
    *reinterpret_cast<uint4*>(sB + (kr + 48) * kPB + nc) = pb3;
    __syncthreads();
    if (kt + 1 < nk) fetch((kt + 1) * kBK);
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
    // (item row, 8-column chunk) pairs, kPairs per thread and round: the
    // first four positions of every pair's run are loaded before any is
    // written (most runs are that short); longer runs continue four
    // positions at a time
    const int nchunk = min(kBN, g.dl - n0) / 8;
    const int rows = min(64, max(0, mcount - 64 * p));
    const int npairs = rows * nchunk;
    for (int v0 = tid; v0 < npairs; v0 += kPairs * 256) {
      int4 it[kPairs];
      int so[kPairs];
      int64_t o0[kPairs];
      uint4 hv[kPairs][4];
#pragma unroll
      for (int j = 0; j < kPairs; ++j) {
        const int v = v0 + j * 256;
        const int vv = v < npairs ? v : v0;
        const int r = vv / nchunk, ch = vv - r * nchunk;
        it[j] = sItem[64 * p + r];
        if (v >= npairs) it[j].z = 0;
        so[j] = r * kOLD + 8 * ch;
        o0[j] = static_cast<int64_t>(it[j].y) * g.dl + n0 + 8 * ch;
        const int last = max(it[j].z, 1) - 1;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hv[j][e] = *reinterpret_cast<const uint4*>(h + o0[j] + static_cast<int64_t>(min(e, last)) * g.dl);
      }
#pragma unroll
      for (int j = 0; j < kPairs; ++j) {
        float acc8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc8[e] = sO[so[j] + e];
        for (int q0 = 0; q0 < it[j].z; q0 += 4) {
          if (q0 > 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int q = min(q0 + e, it[j].z - 1);  // past the run: reload its last position
              hv[j][e] = *reinterpret_cast<const uint4*>(h + o0[j] + static_cast<int64_t>(q) * g.dl);
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (q0 + e >= it[j].z) break;
            const uint32_t wv[4] = {hv[j][e].x, hv[j][e].y, hv[j][e].z, hv[j][e].w};
            float sv[8];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              sv[2 * c] = acc8[2 * c] + bf16_to_f32(static_cast<uint16_t>(wv[c] & 0xFFFFu));
              sv[2 * c + 1] = acc8[2 * c + 1] + bf16_to_f32(static_cast<uint16_t>(wv[c] >> 16));
            }
            Vec<BLLM_BF16>::store(out, o0[j] + static_cast<int64_t>(q0 + e) * g.dl, sv);
          }
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
  if (nbins == 16) {
    hipLaunchKernelGGL(up_count<16>, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.counts);
    hipLaunchKernelGGL(up_items<16>, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.counts,
                       u.bin_off, u.bin_cnt, u.tile_off, u.items);
  } else {
    hipLaunchKernelGGL(up_count<0>, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.counts);
    hipLaunchKernelGGL(up_items<0>, dim3(g.nblk), dim3(kChunksPerBlock), 0, st, idx, g, u.counts,
                       u.bin_off, u.bin_cnt, u.tile_off, u.items);
  }
  const int64_t max_tiles = ceil_div(static_cast<int64_t>(up_max_items(g)), kBM) + nbins;
  const int ncol = static_cast<int>(ceil_div(d_local, kBN));
  const int64_t nblocks = ceil_div(max_tiles, 8) * 8 * ncol;
  hipLaunchKernelGGL(up_gemm, dim3(static_cast<unsigned>(nblocks)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(gm), static_cast<const uint16_t*>(W),
                     static_cast<const uint16_t*>(h), g, u.bin_off,
                     u.bin_cnt, u.tile_off, u.items, ncol, static_cast<uint16_t*>(s_out));
  return launch_status();
}
