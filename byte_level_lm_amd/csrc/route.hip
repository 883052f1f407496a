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
#include <cmath>

#include "common.h"

namespace bllm {
namespace {

// ------------------------------------------------------------- radix select
// Select the key of 0-based rank r (ascending) among the fp32 bit patterns of
// p.  Every score is >= +0 or the canonical NaN 0x7FC00000, so bit 31 is 0 and
// the unsigned bit order is the value order with NaN last.  Three digits:
// bits [20, 31), [10, 20), [0, 10), most significant first, one pass over p
// each.  A pass runs one workgroup per 4096 scores: every workgroup adds to
// one global histogram and takes a completion ticket, and these same-address
// device atomics serialize, so the pass time grows with the workgroup count
// (measured optimum near 64 workgroups at 2^18 scores).  The last workgroup
// of each pass turns the histogram into the next digit and clears it for the
// following pass.  The scoring kernel's first workgroup initialises the state.

constexpr int kSelBins = 2048;
constexpr int kSelThreads = 256;
constexpr int kSelPerThread = 16;
struct SelectState {
  uint32_t prefix;
  uint32_t mask;
  uint32_t rank;
  uint32_t ticket;
  float tau;
  uint32_t pad[3];
  uint32_t hist[kSelBins];
};

// called by every thread of the scoring kernel's first workgroup
__device__ inline void select_init(SelectState* st, uint32_t rank) {
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) st->hist[i] = 0;
  if (threadIdx.x == 0) {
    st->prefix = 0;
    st->mask = 0;
    st->rank = rank;
    st->ticket = 0;
  }
}

// Add this workgroup's LDS histogram `lh` (nb bins, nb in {1024, 2048}) to the
// global one; the last workgroup of the grid then picks the digit holding the
// remaining rank, narrows prefix/mask/rank (and at shift 0 stores tau), and
// clears the histogram and ticket.  All kSelThreads threads call this; the
// digit search runs on the first 256.
__device__ void select_flush_and_digit(SelectState* st, const uint32_t* lh, uint32_t nb,
                                       int shift, float* tau_out, uint32_t* scan) {
  __shared__ int is_last;
  const int tid = threadIdx.x;
  for (int i = tid; i < static_cast<int>(nb); i += kSelThreads)
    if (lh[i]) atomicAdd(&st->hist[i], lh[i]);
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = (atomicAdd(&st->ticket, 1u) == gridDim.x - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  // thread j < 256 owns bins [j*per, (j+1)*per)
  const int per = static_cast<int>(nb) / 256;
  uint32_t cnt[8];
  uint32_t mine = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    cnt[b] = 0;
    if (tid < 256 && b < per)
      cnt[b] = __hip_atomic_load(&st->hist[tid * per + b], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    mine += cnt[b];
  }
  if (tid < 256) scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t v = tid < 256 && tid >= off ? scan[tid - off] : 0u;
    __syncthreads();
    if (tid < 256) scan[tid] += v;
    __syncthreads();
  }
  const uint32_t rank = st->rank, prefix = st->prefix, mask = st->mask;
  const uint32_t incl = tid < 256 ? scan[tid] : 0u;
  uint32_t cum = incl - mine;
  __syncthreads();  // every thread has read rank/prefix/mask before one rewrites them
  if (tid < 256 && cum <= rank && rank < incl) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (b < per && rank >= cum && rank < cum + cnt[b]) {
        const uint32_t bin = tid * per + b;
        st->rank = rank - cum;
        st->prefix = prefix | (bin << shift);
        st->mask = mask | ((nb - 1) << shift);
        if (shift == 0) {
          st->tau = __uint_as_float(prefix | bin);
          if (tau_out) *tau_out = st->tau;
        }
      }
      cum += b < per ? cnt[b] : 0u;
    }
  }
  __syncthreads();
  for (int i = tid; i < static_cast<int>(nb); i += kSelThreads) st->hist[i] = 0;
  if (tid == 0) st->ticket = 0;
}

__global__ __launch_bounds__(kSelThreads) void select_pass(const float* __restrict__ p, int64_t n,
                                                           SelectState* st, int shift, int bits,
                                                           float* tau_out) {
  __shared__ uint32_t lh[kSelBins];
  __shared__ uint32_t scan[256];
  const uint32_t nb = 1u << bits;
  for (int i = threadIdx.x; i < static_cast<int>(nb); i += kSelThreads) lh[i] = 0;
  __syncthreads();
  const uint32_t prefix = st->prefix, mask = st->mask;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSelThreads * kSelPerThread;
  uint32_t key[kSelPerThread];
#pragma unroll
  for (int e = 0; e < kSelPerThread; ++e) {
    const int64_t i = base + static_cast<int64_t>(e) * kSelThreads + threadIdx.x;
    key[e] = i < n ? __float_as_uint(p[i]) : 0xFFFFFFFFu;  // never matches: bit 31 set
  }
  // Scores often crowd into one or two bins of a digit; same-address LDS
  // atomics of one wave serialize, so each wave first peels off up to two
  // bins with one aggregated add each (ballot + popcount).
  constexpr uint32_t kNone = 0xFFFFFFFFu;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < kSelPerThread; ++e) {
    uint32_t bin = (key[e] & mask) == prefix && key[e] != kNone ? (key[e] >> shift) & (nb - 1) : kNone;
    uint64_t active = __ballot(bin != kNone);
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      if (active == 0) break;
      const int leader = __builtin_ctzll(active);
      const uint32_t lb = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), leader));
      const uint64_t same = __ballot(bin == lb);
      if (lane == leader) atomicAdd(&lh[lb], static_cast<uint32_t>(__popcll(same)));
      if (bin == lb) bin = kNone;
      active &= ~same;
    }
    if (bin != kNone) atomicAdd(&lh[bin], 1u);
  }
  __syncthreads();
  select_flush_and_digit(st, lh, nb, shift, tau_out, scan);
}

__global__ __launch_bounds__(256) void threshold_kernel(const float* __restrict__ p, int64_t n,
                                                        const SelectState* st,
                                                        uint8_t* __restrict__ b) {
  const float tau = st->tau;
  const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (i0 + e < n) b[i0 + e] = static_cast<uint8_t>(p[i0 + e] >= tau);
}

// ------------------------------------------------------------- scoring
// One group of G lanes per row (G a power of two, at most 8; each lane
// covers `iters` of the row's 16-byte vectors).  A group scores kRows
// consecutive rows at a time with every q/k load of those rows issued before
// the reductions, and a block walks kPasses such row sets.  The sequence
// starts inside a block's row range are marked in LDS once per block, from a
// block-uniform (scalar) search of the offsets.  With a select state the
// first block initialises it for the select passes that follow.
constexpr int kRows = 2;
constexpr int kPasses = 8;
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
                                                    int64_t total, int iters, float threshold,
                                                    float* __restrict__ p_out,
                                                    uint8_t* __restrict__ b_out,
                                                    float* __restrict__ tau_out,
                                                    SelectState* sel, uint32_t rank) {
  using V = Vec<DT>;
  __shared__ uint8_t sstart[kRouteMaxRows];
  constexpr int G = 1 << GS;
  constexpr int ngroups = 256 >> GS;
  const int rows_per_block = ngroups * kRows * kPasses;
  const int tid = threadIdx.x;
  const int g = tid & (G - 1);
  const int grp = tid >> GS;
  const int64_t rb = static_cast<int64_t>(blockIdx.x) * rows_per_block;
  const int64_t re = rb + rows_per_block < total ? rb + rows_per_block : total;
  const bool write_mask = sel == nullptr;
  if (write_mask && tau_out != nullptr && blockIdx.x == 0 && tid == 0) *tau_out = threshold;
  if (!write_mask && blockIdx.x == 0) select_init(sel, rank);
  for (int i = tid; i < rows_per_block; i += 256) sstart[i] = 0;
  __syncthreads();
  {
    const int slo = lower_seq(offsets, nseq, rb);
    const int shi = lower_seq(offsets, nseq, re);
    for (int s = slo + tid; s < shi; s += 256) sstart[offsets[s] - rb] = 1;
  }
  __syncthreads();
  const int nvec = d / V::N;
  for (int ps = 0; ps < kPasses; ++ps) {
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
                  const int64_t* offsets, int nseq, int64_t total, int iters, float threshold,
                  float* p_out, uint8_t* b_out, float* tau_out, SelectState* sel,
                  uint32_t rank) {
#define BLLM_ROUTE_CASE(GS)                                                                      \
  case GS:                                                                                       \
    hipLaunchKernelGGL((route_kernel<DT, GS>), grid, dim3(256), 0, st, q, k, d, offsets, nseq,  \
                       total, iters, threshold, p_out, b_out, tau_out, sel, rank);               \
    break;
  switch (gshift) {
    BLLM_ROUTE_CASE(0) BLLM_ROUTE_CASE(1) BLLM_ROUTE_CASE(2) BLLM_ROUTE_CASE(3)
  }
#undef BLLM_ROUTE_CASE
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
                          double quantile, float* p_out, uint8_t* b_out, float* tau_out, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!q || !k || !offsets || !p_out || !b_out || d < 1 || nseq < 1 || total < 0 || quantile > 1.0)
    return BLLM_E_INVAL;
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
  // per load instruction and three DPP steps per reduction
  int gshift = 0;
  while ((1 << gshift) < nvec && gshift < 3) ++gshift;
  const int iters = static_cast<int>(ceil_div(nvec, 1 << gshift));
  const int rows_per_block = (256 >> gshift) * kRows * kPasses;
  const dim3 grid(static_cast<unsigned>(ceil_div(total, rows_per_block)));
  SelectState* sst = use_q ? static_cast<SelectState*>(ws) : nullptr;
  const uint32_t rank =
      use_q ? static_cast<uint32_t>(std::floor(quantile * static_cast<double>(total - 1))) : 0u;
  if (dtype == BLLM_F32)
    launch_route<BLLM_F32>(gshift, grid, st, q, k, static_cast<int>(d), offsets,
                           static_cast<int>(nseq), total, iters, threshold, p_out, b_out, tau_out,
                           sst, rank);
  else
    launch_route<BLLM_BF16>(gshift, grid, st, q, k, static_cast<int>(d), offsets,
                            static_cast<int>(nseq), total, iters, threshold, p_out, b_out, tau_out,
                            sst, rank);
  if (!use_q) return launch_status();
  const unsigned nblk = static_cast<unsigned>(ceil_div(total, kSelThreads * kSelPerThread));
  const dim3 sb(kSelThreads);
  hipLaunchKernelGGL(select_pass, dim3(nblk), sb, 0, st, p_out, total, sst, 20, 11, tau_out);
  hipLaunchKernelGGL(select_pass, dim3(nblk), sb, 0, st, p_out, total, sst, 10, 10, tau_out);
  hipLaunchKernelGGL(select_pass, dim3(nblk), sb, 0, st, p_out, total, sst, 0, 10, tau_out);
  hipLaunchKernelGGL(threshold_kernel, dim3(static_cast<unsigned>(ceil_div(total, 1024))),
                     dim3(256), 0, st, p_out, total, sst, b_out);
  return launch_status();
}
