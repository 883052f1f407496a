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

// One group of G lanes per row (G = power of two covering the row's 16-byte
// vectors, at most 64); a 256-thread block handles 4*64/G rows.
template <int DT>
__global__ __launch_bounds__(256) void route_kernel(const void* __restrict__ q,
                                                    const void* __restrict__ k, int d,
                                                    const int64_t* __restrict__ offsets, int nseq,
                                                    int64_t total, int gshift, float threshold,
                                                    int write_mask, float* __restrict__ p_out,
                                                    uint8_t* __restrict__ b_out,
                                                    float* __restrict__ tau_out) {
  using V = Vec<DT>;
  const int G = 1 << gshift;
  const int lane = threadIdx.x & 63;
  const int g = lane & (G - 1);
  const int rows_per_block = blockDim.x >> gshift;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * rows_per_block + (threadIdx.x >> gshift);
  if (write_mask && tau_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *tau_out = threshold;
  if (t >= total) return;
  const int s = upper_seq(offsets, nseq, t);
  const bool start = offsets[s] == t;
  const int nvec = d / V::N;
  float dot = 0.f, nq = 0.f, nk = 0.f;
  if (!start) {
    const int64_t qb = t * d, kb = (t - 1) * d;
    for (int v = g; v < nvec; v += G) {
      float a[V::N], b[V::N];
      V::load(q, qb + v * V::N, a);
      V::load(k, kb + v * V::N, b);
#pragma unroll
      for (int i = 0; i < V::N; ++i) {
        dot = fmaf(a[i], b[i], dot);
        nq = fmaf(a[i], a[i], nq);
        nk = fmaf(b[i], b[i], nk);
      }
    }
    dot = group_sum(dot, G);
    nq = group_sum(nq, G);
    nk = group_sum(nk, G);
  }
  if (g == 0) {
    float p;
    if (start) {
      p = 1.0f;
    } else {
      const float den = fmaxf(sqrtf(nq) * sqrtf(nk), 1e-12f);
      const float cs = dot / den;
      p = 0.5f * (1.0f - cs);
      if (p != p) p = __int_as_float(0x7FC00000);  // canonical NaN
      else p = fminf(fmaxf(p, 0.0f), 1.0f);
      if (p == 0.0f) p = 0.0f;  // +0.0
    }
    p_out[t] = p;
    if (write_mask) b_out[t] = static_cast<uint8_t>(p >= threshold);
  }
}

// ------------------------------------------------------------- radix select
// Select the key of 0-based rank r (ascending) among the fp32 bit patterns of
// p (all >= +0 or canonical NaN, so the unsigned bit order is the value order
// with NaN last).  Three passes of 11, 11 and 10 bits, most significant first.
// The last block of each pass (atomic ticket) turns the global histogram into
// the next digit and clears the histogram for the following pass.

constexpr int kSelBins = 2048;
struct SelectState {
  uint32_t prefix;
  uint32_t mask;
  uint32_t rank;
  uint32_t ticket;
  float tau;
  uint32_t pad[3];
  uint32_t hist[kSelBins];
};

__global__ void select_init(SelectState* st, uint32_t rank) {
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) st->hist[i] = 0;
  if (threadIdx.x == 0) {
    st->prefix = 0;
    st->mask = 0;
    st->rank = rank;
    st->ticket = 0;
  }
}

constexpr int kSelPerThread = 16;

__global__ __launch_bounds__(256) void select_pass(const float* __restrict__ p, int64_t n,
                                                   SelectState* st, int shift, int bits,
                                                   float* tau_out) {
  __shared__ uint32_t lh[kSelBins];
  __shared__ uint32_t scan[256];
  __shared__ int is_last;
  const uint32_t nb = 1u << bits;
  for (int i = threadIdx.x; i < static_cast<int>(nb); i += blockDim.x) lh[i] = 0;
  __syncthreads();
  const uint32_t prefix = st->prefix, mask = st->mask;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x * kSelPerThread;
  for (int e = 0; e < kSelPerThread; ++e) {
    const int64_t i = base + static_cast<int64_t>(e) * blockDim.x + threadIdx.x;
    if (i < n) {
      const uint32_t key = __float_as_uint(p[i]);
      if ((key & mask) == prefix) atomicAdd(&lh[(key >> shift) & (nb - 1)], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < static_cast<int>(nb); i += blockDim.x)
    if (lh[i]) atomicAdd(&st->hist[i], lh[i]);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = (atomicAdd(&st->ticket, 1u) == gridDim.x - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  // digit search: thread j owns bins [j*per, (j+1)*per)
  const int per = static_cast<int>(nb) / 256;
  uint32_t mine = 0;
  for (int b = 0; b < per; ++b)
    mine += __hip_atomic_load(&st->hist[threadIdx.x * per + b], __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
  scan[threadIdx.x] = mine;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t v = threadIdx.x >= static_cast<unsigned>(off) ? scan[threadIdx.x - off] : 0u;
    __syncthreads();
    scan[threadIdx.x] += v;
    __syncthreads();
  }
  const uint32_t rank = st->rank;
  const uint32_t incl = scan[threadIdx.x];
  const uint32_t excl = incl - mine;
  if (excl <= rank && rank < incl) {
    uint32_t cum = excl;
    for (int b = 0; b < per; ++b) {
      const uint32_t bin = threadIdx.x * per + b;
      const uint32_t c = __hip_atomic_load(&st->hist[bin], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      if (rank < cum + c) {
        st->rank = rank - cum;
        st->prefix = prefix | (bin << shift);
        st->mask = mask | ((nb - 1) << shift);
        if (shift == 0) {
          st->tau = __uint_as_float(prefix | bin);
          if (tau_out) *tau_out = st->tau;
        }
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) st->hist[i] = 0;
  if (threadIdx.x == 0) st->ticket = 0;
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
  int gshift = 0;
  while ((1 << gshift) < nvec && gshift < 6) ++gshift;
  const int rows_per_block = 256 >> gshift;
  const dim3 grid(static_cast<unsigned>(ceil_div(total, rows_per_block)));
  if (dtype == BLLM_F32)
    hipLaunchKernelGGL(route_kernel<BLLM_F32>, grid, dim3(256), 0, st, q, k, static_cast<int>(d),
                       offsets, static_cast<int>(nseq), total, gshift, threshold, use_q ? 0 : 1,
                       p_out, b_out, tau_out);
  else
    hipLaunchKernelGGL(route_kernel<BLLM_BF16>, grid, dim3(256), 0, st, q, k, static_cast<int>(d),
                       offsets, static_cast<int>(nseq), total, gshift, threshold, use_q ? 0 : 1,
                       p_out, b_out, tau_out);
  if (!use_q) return launch_status();
  SelectState* sst = static_cast<SelectState*>(ws);
  const uint32_t rank = static_cast<uint32_t>(std::floor(quantile * static_cast<double>(total - 1)));
  hipLaunchKernelGGL(select_init, dim3(1), dim3(256), 0, st, sst, rank);
  const unsigned nblk = static_cast<unsigned>(ceil_div(total, 256 * kSelPerThread));
  hipLaunchKernelGGL(select_pass, dim3(nblk), dim3(256), 0, st, p_out, total, sst, 21, 11, tau_out);
  hipLaunchKernelGGL(select_pass, dim3(nblk), dim3(256), 0, st, p_out, total, sst, 10, 11, tau_out);
  hipLaunchKernelGGL(select_pass, dim3(nblk), dim3(256), 0, st, p_out, total, sst, 0, 10, tau_out);
  hipLaunchKernelGGL(threshold_kernel, dim3(static_cast<unsigned>(ceil_div(total, 1024))),
                     dim3(256), 0, st, p_out, total, sst, b_out);
  return launch_status();
}
