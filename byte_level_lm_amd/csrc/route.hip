// H-Net boundary scoring and the per-stage score quantile.
//
// ByteGen report, section 2.3 (H-Net dynamic chunking): the boundary
// probability of a byte comes from the cosine similarity between its own
// representation and its predecessor's.  Here p_t = (1 - cos(q_t, k_{t-1}))/2,
// p = 1 at a sequence start, b_t = [p_t >= tau].  For a hierarchy stage whose
// kept fraction is fixed (1/4 per stage in the report), tau is an order
// statistic of the stage's scores, found by a radix select on the fp32 bits.
//
// Memory layout: q, k packed rows [total x d]; p fp32 [total]; b uint8 [total].
// HBM-bound: 2*d*e bytes read and 5 bytes written per position.
#include <algorithm>
#include <cmath>

#include "common.h"

namespace bllm {
namespace {

// ------------------------------------------------------------- radix select
// Select the key of 0-based rank r (ascending) among the fp32 bit patterns of
// p.  Every score is >= +0 or the canonical NaN 0x7FC00000, so bit 31 is 0 and
// the unsigned bit order is the value order with NaN last.  Three digits:
// bits [20, 31), [10, 20), [0, 10), most significant first.
//
// One launch of G <= kSelMaxBlocks workgroups runs all three digits and the
// threshold.  A workgroup holds one tile of 4096 scores in
// registers (with more tiles than workgroups, each digit re-reads them), adds
// its LDS histogram of the digit to a global one with device atomics, and
// after a grid barrier every workgroup reads the whole histogram and narrows
// the prefix itself, so all of them reach the same digit without a further
// exchange.  Same-address device atomics serialize, so the flush grows with
// G (measured optimum near 64 workgroups at 2^18 scores).  Last, each
// workgroup writes b = [p >= tau] for its own scores.  The scoring kernel's
// first workgroup zeroes the histograms and barrier counters beforehand.

constexpr int kSelBins = 2048;
constexpr int kSelThreads = 256;
constexpr int kSelPerThread = 16;
constexpr int kSelTile = kSelThreads * kSelPerThread;
constexpr int kSelMaxBlocks = 64;
constexpr int kSelDigits = 3;
// The grid barriers need all G workgroups resident at once.  A workgroup
// takes 256 threads, 64 VGPRs and 8 KB of LDS, so eight CUs already hold 64
// of them, and the launch follows the scoring kernel on the same stream.
// The spin bound (each round sleeps ~100 clocks, ~1 s in all) is never
// reached in that case; if it were, tau comes out NaN, b is 0 everywhere,
// BLLM_S_INCOMPLETE is ORed into the caller's status word and the kernel ends.
#ifndef BLLM_SELECT_SPIN_LIMIT
#define BLLM_SELECT_SPIN_LIMIT (1u << 22)
#endif
constexpr uint32_t kSelSpinLimit = BLLM_SELECT_SPIN_LIMIT;
constexpr uint32_t kNoKey = 0xFFFFFFFFu;  // past the end: bit 31 set, never selected

struct SelectState {
  uint32_t arrive[kSelDigits];  // grid-barrier arrivals, one counter per digit
  uint32_t pad[8 - kSelDigits];
  uint32_t hist[kSelDigits][kSelBins];
};

// called by every thread of the scoring kernel's first workgroup
__device__ inline void select_init(SelectState* st) {
  uint32_t* w = reinterpret_cast<uint32_t*>(st);
  constexpr int nw = static_cast<int>(sizeof(SelectState) / 4);
  for (int i = threadIdx.x; i < nw; i += blockDim.x) w[i] = 0;
}

// Every workgroup of the grid arrives once at `arrive`; false if not all
// nblocks arrived within the spin limit.  What the workgroups publish before
// it (the histogram) is written with device-scope atomics only, so the
// release needs no L2 write-back: each wave waits until its atomics are
// acknowledged (vmcnt 0) before the arrival is counted.
__device__ bool grid_barrier(uint32_t* arrive, uint32_t nblocks) {
  __shared__ int all_in;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(arrive, 1u);
    int done = 0;
    for (uint32_t spin = 0; spin < kSelSpinLimit; ++spin) {
      if (__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= nblocks) {
        done = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    all_in = done;
  }
  __syncthreads();
  return all_in != 0;
}

__device__ inline void sel_load(const float* __restrict__ p, int64_t n, int64_t tile,
                                uint32_t (&key)[kSelPerThread]) {
  const int64_t base = tile * kSelTile + threadIdx.x;
#pragma unroll
  for (int e = 0; e < kSelPerThread; ++e) {
    const int64_t i = base + static_cast<int64_t>(e) * kSelThreads;
    key[e] = i < n ? __float_as_uint(p[i]) : kNoKey;
  }
}

// Add the keys under (prefix, mask) to the LDS histogram of the digit at
// `shift`.  Scores often crowd into one or two bins of a digit and
// same-address LDS atomics of one wave serialize, so each wave first peels
// off up to two bins with one aggregated add each (ballot + popcount).
__device__ inline void sel_count(const uint32_t (&key)[kSelPerThread], uint32_t prefix,
                                 uint32_t mask, int shift, uint32_t nb, uint32_t* lh) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < kSelPerThread; ++e) {
    uint32_t bin = (key[e] & mask) == prefix && key[e] != kNoKey ? (key[e] >> shift) & (nb - 1) : kNoKey;
    uint64_t active = __ballot(bin != kNoKey);
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      if (active == 0) break;
      const int leader = __builtin_ctzll(active);
      const uint32_t lb = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), leader));
      const uint64_t same = __ballot(bin == lb);
      if (lane == leader) atomicAdd(&lh[lb], static_cast<uint32_t>(__popcll(same)));
      if (bin == lb) bin = kNoKey;
      active &= ~same;
    }
    if (bin != kNoKey) atomicAdd(&lh[bin], 1u);
  }
}

__device__ inline void sel_mark(const uint32_t (&key)[kSelPerThread], int64_t n, int64_t tile,
                                float tau, uint8_t* __restrict__ b) {
  const int64_t base = tile * kSelTile + threadIdx.x;
#pragma unroll
  for (int e = 0; e < kSelPerThread; ++e) {
    const int64_t i = base + static_cast<int64_t>(e) * kSelThreads;
    if (i < n) b[i] = static_cast<uint8_t>(__uint_as_float(key[e]) >= tau);
  }
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ p, int64_t n,
                                                             uint32_t rank, SelectState* st,
                                                             float* __restrict__ tau_out,
                                                             uint8_t* __restrict__ b,
                                                             int32_t* __restrict__ status) {
  __shared__ uint32_t lh[kSelBins];
  __shared__ uint32_t wtot[kSelThreads / kWave];
  __shared__ uint32_t found[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const uint32_t G = gridDim.x;
  const int64_t ntiles = (n + kSelTile - 1) / kSelTile;
  const bool resident = ntiles <= static_cast<int64_t>(G);  // then G == ntiles
  uint32_t key[kSelPerThread];
  if (resident) sel_load(p, n, blockIdx.x, key);
  uint32_t prefix = 0, mask = 0;
  bool ok = true;
  for (int dg = 0; dg < kSelDigits; ++dg) {
    const int shift = dg == 0 ? 20 : (dg == 1 ? 10 : 0);
    const uint32_t nb = dg == 0 ? 2048u : 1024u;
    for (int i = tid; i < static_cast<int>(nb); i += kSelThreads) lh[i] = 0;
    __syncthreads();
    if (resident) {
      sel_count(key, prefix, mask, shift, nb, lh);
    } else {
      for (int64_t t = blockIdx.x; t < ntiles; t += G) {
        uint32_t kk[kSelPerThread];
        sel_load(p, n, t, kk);
        sel_count(kk, prefix, mask, shift, nb, lh);
      }
    }
    __syncthreads();
    uint32_t* gh = st->hist[dg];
    for (int i = tid; i < static_cast<int>(nb); i += kSelThreads)
      if (lh[i]) atomicAdd(&gh[i], lh[i]);
    ok = grid_barrier(&st->arrive[dg], G) && ok;
    // every workgroup: thread j owns bins [j*per, (j+1)*per); find the bin
    // in which the remaining rank falls
    const int per = static_cast<int>(nb) / kSelThreads;
    uint32_t cnt[kSelBins / kSelThreads];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < kSelBins / kSelThreads; ++q) {
      cnt[q] = q < per ? __hip_atomic_load(&gh[tid * per + q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
      mine += cnt[q];
    }
    int wall;  // at most 2^31 scores: the int scan is exact
    uint32_t incl = static_cast<uint32_t>(wave_incl_scan(static_cast<int>(mine), wall));
    if (lane == kWave - 1) wtot[wv] = incl;
    __syncthreads();
    for (int w = 0; w < wv; ++w) incl += wtot[w];
    const uint32_t cum = incl - mine;
    if (cum <= rank && rank < incl) {
      uint32_t c = cum;
#pragma unroll
      for (int q = 0; q < kSelBins / kSelThreads; ++q) {
        if (q < per && rank >= c && rank < c + cnt[q]) {
          found[0] = rank - c;
          found[1] = static_cast<uint32_t>(tid * per + q);
        }
        c += cnt[q];
      }
    }
    __syncthreads();
    rank = found[0];
    prefix |= found[1] << shift;
    mask |= (nb - 1) << shift;
    __syncthreads();  // found, wtot and lh are rewritten by the next digit
  }
  const float tau = ok ? __uint_as_float(prefix) : __builtin_nanf("");
  if (blockIdx.x == 0 && tid == 0 && tau_out != nullptr) *tau_out = tau;
  if (!ok && tid == 0 && status != nullptr) atomicOr(status, BLLM_S_INCOMPLETE);
  if (resident) {
    sel_mark(key, n, blockIdx.x, tau, b);
  } else {
    for (int64_t t = blockIdx.x; t < ntiles; t += G) {
      uint32_t kk[kSelPerThread];
      sel_load(p, n, t, kk);
      sel_mark(kk, n, t, tau, b);
    }
  }
}

// ------------------------------------------------------------- scoring
// One group of G lanes per row (G a power of two, at most 8; each lane
// covers `iters` of the row's 16-byte vectors).  A group scores kRows
// consecutive rows at a time with every q/k load of those rows issued before
// the reductions, and a block walks `passes` (at most kPasses) such row sets,
// as few as keep the grid at kRouteBlocks workgroups or more.  The sequence
// starts inside a block's row range are marked in LDS once per block, from a
// block-uniform (scalar) search of the offsets.  With a select state the
// first block initialises it for the select passes that follow.
constexpr int kRows = 2;
constexpr int kPasses = 8;
#ifndef BLLM_ROUTE_BLOCKS
#define BLLM_ROUTE_BLOCKS 1024
#endif
constexpr int kRouteBlocks = BLLM_ROUTE_BLOCKS;
constexpr int kRouteMaxRows = 256 * kRows * kPasses;

// first s in [0, n) with a[s] >= x (n if none)
__device__ inline int lower_seq(const int64_t* a, int n, int64_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <int DT, int GS>
__global__ __launch_bounds__(256) void route_kernel(const void* __restrict__ q,
                                                    const void* __restrict__ k, int d,
                                                    const int64_t* __restrict__ offsets, int nseq,
                                                    int64_t total, int iters, int passes,
                                                    float threshold,
                                                    float* __restrict__ p_out,
                                                    uint8_t* __restrict__ b_out,
                                                    float* __restrict__ tau_out,
                                                    SelectState* sel) {
  using V = Vec<DT>;
  __shared__ uint8_t sstart[kRouteMaxRows];
  constexpr int G = 1 << GS;
  constexpr int ngroups = 256 >> GS;
  const int rows_per_block = ngroups * kRows * passes;
  const int tid = threadIdx.x;
  const int g = tid & (G - 1);
  const int grp = tid >> GS;
  const int64_t rb = static_cast<int64_t>(blockIdx.x) * rows_per_block;
  const int64_t re = rb + rows_per_block < total ? rb + rows_per_block : total;
  const bool write_mask = sel == nullptr;
  if (write_mask && tau_out != nullptr && blockIdx.x == 0 && tid == 0) *tau_out = threshold;
  if (!write_mask && blockIdx.x == 0) select_init(sel);
  for (int i = tid; i < rows_per_block; i += 256) sstart[i] = 0;
  __syncthreads();
  {
    const int slo = lower_seq(offsets, nseq, rb);
    const int shi = lower_seq(offsets, nseq, re);
    for (int s = slo + tid; s < shi; s += 256) sstart[offsets[s] - rb] = 1;
  }
  __syncthreads();
  const int nvec = d / V::N;
  for (int ps = 0; ps < passes; ++ps) {
    const int64_t t0 = rb + static_cast<int64_t>(ps * ngroups + grp) * kRows;
    if (t0 >= re) break;
    // rows past the end are clamped to the last row and not written; a
    // sequence start reads its own k row (its score is replaced by 1)
    int64_t tq[kRows], tk[kRows];
    bool st[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t t = t0 + r < re ? t0 + r : re - 1;
      st[r] = sstart[t - rb] != 0;
      tq[r] = t * d;
      tk[r] = (st[r] || t == 0 ? t : t - 1) * d;
    }
    float dot[kRows], nq[kRows], nk[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) dot[r] = nq[r] = nk[r] = 0.f;
    for (int it = 0; it < iters; ++it) {
      const int v = g + it * G;
      const int64_t e0 = static_cast<int64_t>(v < nvec ? v : nvec - 1) * V::N;
      const float m = v < nvec ? 1.f : 0.f;
      float a[kRows][V::N], b[kRows][V::N];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        V::load(q, tq[r] + e0, a[r]);
        V::load(k, tk[r] + e0, b[r]);
      }
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        float pd = 0.f, pq = 0.f, pk = 0.f;
#pragma unroll
        for (int e = 0; e < V::N; ++e) {
          pd = fmaf(a[r][e], b[r][e], pd);
          pq = fmaf(a[r][e], a[r][e], pq);
          pk = fmaf(b[r][e], b[r][e], pk);
        }
        dot[r] = fmaf(m, pd, dot[r]);
        nq[r] = fmaf(m, pq, nq[r]);
        nk[r] = fmaf(m, pk, nk[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      dot[r] = group_sum<G>(dot[r]);
      nq[r] = group_sum<G>(nq[r]);
      nk[r] = group_sum<G>(nk[r]);
    }
    // lane r of the group writes row r (lane 0 writes all rows when G < kRows)
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t t = t0 + r;
      const bool mine = G >= kRows ? g == r : g == 0;
      if (mine && t < re) {
        float p;
        if (st[r]) {
          p = 1.0f;
        } else {
          const float den = fmaxf(sqrtf(nq[r]) * sqrtf(nk[r]), 1e-12f);
          const float cs = dot[r] / den;
          p = 0.5f * (1.0f - cs);
          if (p != p) p = __int_as_float(0x7FC00000);  // canonical NaN
          else p = fminf(fmaxf(p, 0.0f), 1.0f);
          if (p == 0.0f) p = 0.0f;  // +0.0
        }
        p_out[t] = p;
        if (write_mask) b_out[t] = static_cast<uint8_t>(p >= threshold);
      }
    }
  }
}

template <int DT>
void launch_route(int gshift, dim3 grid, hipStream_t st, const void* q, const void* k, int d,
                  const int64_t* offsets, int nseq, int64_t total, int iters, int passes,
                  float threshold,
                  float* p_out, uint8_t* b_out, float* tau_out, SelectState* sel) {
#define BLLM_ROUTE_CASE(GS)                                                                      \
  case GS:                                                                                       \
    hipLaunchKernelGGL((route_kernel<DT, GS>), grid, dim3(256), 0, st, q, k, d, offsets, nseq,  \
                       total, iters, passes, threshold, p_out, b_out, tau_out, sel);             \
    break;
  switch (gshift) {
    BLLM_ROUTE_CASE(0) BLLM_ROUTE_CASE(1) BLLM_ROUTE_CASE(2) BLLM_ROUTE_CASE(3) BLLM_ROUTE_CASE(4)
  }
#undef BLLM_ROUTE_CASE
}

// ------------------------------------------------------------- fused projection + scoring
// The routing projections q = h Wq, k = h Wk (row-vector convention) and the
// score in one kernel, so q and k never reach memory.  A workgroup owns 128
// rows t0 .. t0+127.  Its h tile is staged with one extra row above
// (t0 - 1), and the k half of the GEMM reads the staged rows shifted by one:
// row t of the tile holds q_t and k_{t-1} side by side, so the cosine needs
// only per-row sums: dot = sum_j q_t[j] k_{t-1}[j], |q_t|^2, |k_{t-1}|^2.
// Columns are taken in blocks of 128 (of q and of k); four waves in 2 x 2
// each compute a 64 x 64 quadrant of both (bf16 MFMA 32x32x16, W read down
// its columns with the transposing LDS read), reduce its per-row sums over
// its 64 columns with DPP, and add them to an LDS slot of its own, so the
// sums are formed in a fixed order.  The next K step's operands are in
// flight in registers while the MFMAs consume the one in LDS.
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

constexpr int kFR = 128;        // rows per tile
constexpr int kFC = 128;        // q and k columns per block
constexpr int kFK = 64;         // K step
constexpr int kFPA = kFK + 8;   // LDS pitch (bf16) of the staged h rows
constexpr int kFPB = kFC + 16;  // LDS pitch (bf16) of the staged W rows: rows 8 banks apart

// row of element r held by `lane` in a 32x32 MFMA accumulator
__device__ inline int frow_of(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// two transposing LDS reads (ds_read_b64_tr_b16) give a lane the B operand
// of a [k][n] tile: with row = 8 (lane / 32) + (lane % 16) / 4 and col =
// 16 ((lane / 16) % 2) + 4 (lane % 4) added to the origin, lane l receives
// column l % 32, rows 8 (l / 32) .. +7
__device__ inline bf16x8 tr_b_frag(const uint16_t* s, int row, int col, int pitch) {
  typedef __attribute__((address_space(3))) shortx4 lds_s4;
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(s + row * pitch + col));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(s + (row + 4) * pitch + col));
  bf16x8 v;
  __builtin_memcpy(&v, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&v) + 8, &hi, 8);
  return v;
}

__global__ __launch_bounds__(256, 2) void route_fused_kernel(const uint16_t* __restrict__ h,
                                                             const uint16_t* __restrict__ Wq,
                                                             const uint16_t* __restrict__ Wk, int d,
                                                             const int64_t* __restrict__ offsets, int nseq,
                                                             int64_t total, float threshold,
                                                             float* __restrict__ p_out,
                                                             uint8_t* __restrict__ b_out,
                                                             float* __restrict__ tau_out, SelectState* sel) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[(kFR + 1) * kFPA];
  __shared__ __attribute__((aligned(16))) uint16_t sBq[kFK * kFPB];
  __shared__ __attribute__((aligned(16))) uint16_t sBk[kFK * kFPB];
  __shared__ float sSum[2][kFR][3];  // [column half][row][dot, |q|^2, |k|^2]
  __shared__ uint8_t sstart[kFR];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kFR;
  const int64_t te = t0 + kFR < total ? t0 + kFR : total;
  const bool write_mask = sel == nullptr;
  if (write_mask && tau_out != nullptr && blockIdx.x == 0 && tid == 0) *tau_out = threshold;
  if (!write_mask && blockIdx.x == 0) select_init(sel);
  for (int e = tid; e < 2 * kFR * 3; e += 256) (&sSum[0][0][0])[e] = 0.f;
  if (tid < kFR) sstart[tid] = 0;
  __syncthreads();
  {
    const int slo = lower_seq(offsets, nseq, t0);
    const int shi = lower_seq(offsets, nseq, te);
    for (int s = slo + tid; s < shi; s += 256) sstart[offsets[s] - t0] = 1;
  }
  // loaders.  h: staged row i is h row t0 - 1 + i (clamped into [0, total));
  // thread: rows 1 + ra + 32 q (q = 0..3), 16-byte chunk la; threads 0..7 also
  // row 0.  W: K rows kb + 16 q of the block's 128 columns, chunk nb.
  const int ra = tid >> 3, la = (tid & 7) * 8;
  const int kb = tid >> 4, nb = (tid & 15) * 8;
  auto hrow = [&](int64_t r) { return (r < 0 ? 0 : (r < total ? r : total - 1)) * static_cast<int64_t>(d); };
  const int64_t ho0 = hrow(t0 + ra) + la, ho1 = hrow(t0 + ra + 32) + la;
  const int64_t ho2 = hrow(t0 + ra + 64) + la, ho3 = hrow(t0 + ra + 96) + la;
  const int64_t hoh = hrow(t0 - 1) + (tid & 7) * 8;
  uint4 pa0, pa1, pa2, pa3, ph, pq0, pq1, pq2, pq3, pk0, pk1, pk2, pk3;
  auto fetch = [&](int jb, int kt) {
    const int ko = kt * kFK;
    pa0 = *reinterpret_cast<const uint4*>(h + ho0 + ko);
    pa1 = *reinterpret_cast<const uint4*>(h + ho1 + ko);
    pa2 = *reinterpret_cast<const uint4*>(h + ho2 + ko);
    pa3 = *reinterpret_cast<const uint4*>(h + ho3 + ko);
    ph = *reinterpret_cast<const uint4*>(h + hoh + ko);
    const int64_t wo = static_cast<int64_t>(ko + kb) * d + jb * kFC + nb;
    const int64_t w16 = static_cast<int64_t>(16) * d;
    pq0 = *reinterpret_cast<const uint4*>(Wq + wo);
    pq1 = *reinterpret_cast<const uint4*>(Wq + wo + w16);
    pq2 = *reinterpret_cast<const uint4*>(Wq + wo + 2 * w16);
    pq3 = *reinterpret_cast<const uint4*>(Wq + wo + 3 * w16);
    pk0 = *reinterpret_cast<const uint4*>(Wk + wo);
    pk1 = *reinterpret_cast<const uint4*>(Wk + wo + w16);
    pk2 = *reinterpret_cast<const uint4*>(Wk + wo + 2 * w16);
    pk3 = *reinterpret_cast<const uint4*>(Wk + wo + 3 * w16);
  };
  auto stash = [&]() {
    *reinterpret_cast<uint4*>(sA + (1 + ra) * kFPA + la) = pa0;
    *reinterpret_cast<uint4*>(sA + (33 + ra) * kFPA + la) = pa1;
    *reinterpret_cast<uint4*>(sA + (65 + ra) * kFPA + la) = pa2;
    *reinterpret_cast<uint4*>(sA + (97 + ra) * kFPA + la) = pa3;
    if (tid < 8) *reinterpret_cast<uint4*>(sA + (tid & 7) * 8) = ph;
    *reinterpret_cast<uint4*>(sBq + kb * kFPB + nb) = pq0;
    *reinterpret_cast<uint4*>(sBq + (kb + 16) * kFPB + nb) = pq1;
    *reinterpret_cast<uint4*>(sBq + (kb + 32) * kFPB + nb) = pq2;
    *reinterpret_cast<uint4*>(sBq + (kb + 48) * kFPB + nb) = pq3;
    *reinterpret_cast<uint4*>(sBk + kb * kFPB + nb) = pk0;
    *reinterpret_cast<uint4*>(sBk + (kb + 16) * kFPB + nb) = pk1;
    *reinterpret_cast<uint4*>(sBk + (kb + 32) * kFPB + nb) = pk2;
    *reinterpret_cast<uint4*>(sBk + (kb + 48) * kFPB + nb) = pk3;
  };
  const int j16 = lane & 15;
  const int brow = 8 * (lane >> 5) + (j16 >> 2);
  const int bcol = 64 * wn + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
  const int nkt = d / kFK, njb = d / kFC;
  fetch(0, 0);
  for (int jb = 0; jb < njb; ++jb) {
    floatx16 aq[2][2], ak[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) aq[a][c][r] = ak[a][c][r] = 0.f;
    for (int kt = 0; kt < nkt; ++kt) {
      __syncthreads();
      stash();
      __syncthreads();
      if (kt + 1 < nkt) fetch(jb, kt + 1);
      else if (jb + 1 < njb) fetch(jb + 1, 0);
#pragma unroll
      for (int ks = 0; ks < kFK; ks += 16) {
        bf16x8 fq[2], fk[2], bq[2], bk[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int r0 = 64 * wm + 32 * a + (lane & 31);
          fq[a] = *reinterpret_cast<const bf16x8*>(sA + (r0 + 1) * kFPA + ks + 8 * (lane >> 5));
          fk[a] = *reinterpret_cast<const bf16x8*>(sA + r0 * kFPA + ks + 8 * (lane >> 5));
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          bq[c] = tr_b_frag(sBq, ks + brow, bcol + 32 * c, kFPB);
          bk[c] = tr_b_frag(sBk, ks + brow, bcol + 32 * c, kFPB);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            aq[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[a], bq[c], aq[a][c], 0, 0, 0);
            ak[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[a], bk[c], ak[a][c], 0, 0, 0);
          }
      }
    }
    // per-row sums over this wave's 64 columns of the block
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float dq = 0.f, nq = 0.f, nk = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          dq = fmaf(aq[a][c][r], ak[a][c][r], dq);
          nq = fmaf(aq[a][c][r], aq[a][c][r], nq);
          nk = fmaf(ak[a][c][r], ak[a][c][r], nk);
        }
        dq = group_sum<32>(dq);
        nq = group_sum<32>(nq);
        nk = group_sum<32>(nk);
        if ((lane & 31) == 0) {
          float* sp = sSum[wn][64 * wm + 32 * a + frow_of(r, lane)];
          sp[0] += dq;
          sp[1] += nq;
          sp[2] += nk;
        }
      }
    }
  }
  __syncthreads();
  if (tid < kFR) {
    const int64_t t = t0 + tid;
    if (t < total) {
      float p;
      if (sstart[tid]) {
        p = 1.0f;
      } else {
        const float dot = sSum[0][tid][0] + sSum[1][tid][0];
        const float nq = sSum[0][tid][1] + sSum[1][tid][1];
        const float nk = sSum[0][tid][2] + sSum[1][tid][2];
        const float den = fmaxf(sqrtf(nq) * sqrtf(nk), 1e-12f);
        p = 0.5f * (1.0f - dot / den);
        if (p != p) p = __int_as_float(0x7FC00000);  // canonical NaN
        else p = fminf(fmaxf(p, 0.0f), 1.0f);
        if (p == 0.0f) p = 0.0f;  // +0.0
      }
      p_out[t] = p;
      if (write_mask) b_out[t] = static_cast<uint8_t>(p >= threshold);
    }
  }
}

}  // namespace
}  // namespace bllm

using namespace bllm;

extern "C" size_t bllm_route_workspace(int64_t total) {
  (void)total;
  return sizeof(SelectState);
}

extern "C" int bllm_route(const void* q, const void* k, int dtype, int64_t d,
                          const int64_t* offsets, int64_t nseq, int64_t total, float threshold,
                          double quantile, float* p_out, uint8_t* b_out, float* tau_out,
                          int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  if (!offsets || d < 1 || nseq < 1 || total < 0 || quantile > 1.0) return BLLM_E_INVAL;
  if (total > 0 && (!q || !k || !p_out || !b_out)) return BLLM_E_INVAL;  // may be NULL for an empty batch
  if (!valid_dtype(dtype)) return BLLM_E_NOTSUP;
  if ((d * elem_size(dtype)) % 16 != 0 || !aligned16(q) || !aligned16(k)) return BLLM_E_NOTSUP;
  if (total >= (int64_t(1) << 31) || nseq >= (int64_t(1) << 30)) return BLLM_E_NOTSUP;
  const bool use_q = quantile >= 0.0;
  if (use_q && (!ws || ws_bytes < sizeof(SelectState))) return BLLM_E_WS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (total == 0) {
    if (tau_out) hipLaunchKernelGGL(fill_f32, dim3(1), dim3(64), 0, st, tau_out, 1,
                                    use_q ? __builtin_nanf("") : threshold);
    return launch_status();
  }
  const int vn = dtype == BLLM_F32 ? 4 : 8;
  const int nvec = static_cast<int>(d / vn);
  // 8 lanes per row (fewer for rows of under 8 vectors): 128-byte segments
  // per load instruction and three DPP steps per reduction; 16 lanes for rows
  // of 96 vectors or more (1.5 KB: stage-2 rows of 768 bf16), 4 DPP steps
  int gshift = 0;
  const int gmax = nvec >= 96 ? 4 : 3;
  while ((1 << gshift) < nvec && gshift < gmax) ++gshift;
  const int iters = static_cast<int>(ceil_div(nvec, 1 << gshift));
  const int64_t rows_per_pass = (256 >> gshift) * kRows;
  const int passes = static_cast<int>(
      std::min<int64_t>(kPasses, std::max<int64_t>(1, total / (rows_per_pass * kRouteBlocks))));
  const int64_t rows_per_block = rows_per_pass * passes;
  const dim3 grid(static_cast<unsigned>(ceil_div(total, rows_per_block)));
  SelectState* sst = use_q ? static_cast<SelectState*>(ws) : nullptr;
  if (dtype == BLLM_F32)
    launch_route<BLLM_F32>(gshift, grid, st, q, k, static_cast<int>(d), offsets,
                           static_cast<int>(nseq), total, iters, passes, threshold, p_out, b_out, tau_out,
                           sst);
  else
    launch_route<BLLM_BF16>(gshift, grid, st, q, k, static_cast<int>(d), offsets,
                            static_cast<int>(nseq), total, iters, passes, threshold, p_out, b_out, tau_out,
                            sst);
  if (!use_q) return launch_status();
  if (launch_status() != BLLM_OK) return BLLM_E_HIP;
  const uint32_t rank = static_cast<uint32_t>(std::floor(quantile * static_cast<double>(total - 1)));
  const unsigned nblk = static_cast<unsigned>(std::min<int64_t>(kSelMaxBlocks, ceil_div(total, kSelTile)));
  hipLaunchKernelGGL(select_kernel, dim3(nblk), dim3(kSelThreads), 0, st, p_out, total, rank, sst,
                     tau_out, b_out, status);
  return launch_status();
}

extern "C" int bllm_route_fused(const void* h, const void* Wq, const void* Wk, int dtype, int64_t d,
                                const int64_t* offsets, int64_t nseq, int64_t total, float threshold,
                                double quantile, float* p_out, uint8_t* b_out, float* tau_out,
                                int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  if (!Wq || !Wk || !offsets || d < 1 || nseq < 1 || total < 0 || quantile > 1.0) return BLLM_E_INVAL;
  if (total > 0 && (!h || !p_out || !b_out)) return BLLM_E_INVAL;  // may be NULL for an empty batch
  if (dtype != BLLM_BF16) return BLLM_E_NOTSUP;
  if (d % kFC != 0 || d > 4096 || !aligned16(h) || !aligned16(Wq) || !aligned16(Wk)) return BLLM_E_NOTSUP;
  if (total >= (int64_t(1) << 31) || nseq >= (int64_t(1) << 30)) return BLLM_E_NOTSUP;
  const bool use_q = quantile >= 0.0;
  if (use_q && (!ws || ws_bytes < sizeof(SelectState))) return BLLM_E_WS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (total == 0) {
    if (tau_out) hipLaunchKernelGGL(fill_f32, dim3(1), dim3(64), 0, st, tau_out, 1,
                                    use_q ? __builtin_nanf("") : threshold);
    return launch_status();
  }
  SelectState* sst = use_q ? static_cast<SelectState*>(ws) : nullptr;
  hipLaunchKernelGGL(route_fused_kernel, dim3(static_cast<unsigned>(ceil_div(total, kFR))), dim3(256), 0, st,
                     static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(Wq),
                     static_cast<const uint16_t*>(Wk), static_cast<int>(d), offsets, static_cast<int>(nseq),
                     total, threshold, p_out, b_out, tau_out, sst);
  if (!use_q) return launch_status();
  if (launch_status() != BLLM_OK) return BLLM_E_HIP;
  const uint32_t rank = static_cast<uint32_t>(std::floor(quantile * static_cast<double>(total - 1)));
  const unsigned nblk = static_cast<unsigned>(std::min<int64_t>(kSelMaxBlocks, ceil_div(total, kSelTile)));
  hipLaunchKernelGGL(select_kernel, dim3(nblk), dim3(kSelThreads), 0, st, p_out, total, rank, sst,
                     tau_out, b_out, status);
  return launch_status();
}
