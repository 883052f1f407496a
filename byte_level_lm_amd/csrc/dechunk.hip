// EMA dechunk: smooth the chunk sequence and expand it back to byte length.
//
// ByteGen report, section 2.3: an exponential moving average over the chunk
// sequence makes the discrete boundaries differentiable.  Per sequence,
//   zbar_c = P_c z_c + (1 - P_c) zbar_{c-1}   (zbar before the first chunk = 0)
//   out_t  = zbar_{c(t)}                       (c(t): last chunk starting <= t)
//
// The recurrence x_c = a_c x_{c-1} + u_c (a_c = 1 - P_c, or 0 at the first
// chunk of a sequence; u_c = P_c z_c) is a linear recurrence, scanned in three
// passes over a fixed grid of kNT tiles of consecutive chunks (flat over the
// packed batch; the a = 0 resets keep sequences independent):
//   1. per tile: its affine aggregate (A = prod a, U = scan end from 0)
//   2. per 4-feature slice: scan of the kNT aggregates -> carry into each tile
//   3. per tile: rescan from the carry and write every byte row of each chunk
// HBM-bound: z is read twice, the [total x d] output is written once
// (nontemporal); the tile aggregates add 2 * kNT * d * 4 bytes.
#include "common.h"

namespace bllm {
namespace {

constexpr int kNT = 4096;

struct Tile {
  int64_t c0, c1;
};

__device__ inline Tile tile_range(int64_t M, int64_t i) {
  const int64_t L = (M + kNT - 1) / kNT;
  const int64_t c0 = i * L;
  return {c0, c0 + L < M ? c0 + L : M};
}

template <int DT>
__global__ __launch_bounds__(256) void ema_tile_aggregate(const void* __restrict__ z,
                                                          const float* __restrict__ P, int d,
                                                          const int64_t* __restrict__ chunk_offsets,
                                                          int nseq, float* __restrict__ Aagg,
                                                          float* __restrict__ Uagg) {
  using V = Vec<DT>;
  const int lane = threadIdx.x & 63;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int v = blockIdx.y * 64 + lane;
  const bool active = v < d / V::N;
  const int64_t M = chunk_offsets[nseq];
  const Tile tr = tile_range(M, i);
  float x[V::N];
#pragma unroll
  for (int e = 0; e < V::N; ++e) x[e] = 0.f;
  float A = 1.f;
  if (tr.c0 < tr.c1) {
    int s = upper_seq(chunk_offsets, nseq, tr.c0);
    for (int64_t c = tr.c0; c < tr.c1; ++c) {
      while (chunk_offsets[s + 1] <= c) ++s;
      const float Pc = P[c];
      const float a = c == chunk_offsets[s] ? 0.f : 1.f - Pc;
      if (active) {
        float zz[V::N];
        V::load(z, c * d + v * V::N, zz);
#pragma unroll
        for (int e = 0; e < V::N; ++e) x[e] = fmaf(a, x[e], Pc * zz[e]);
      }
      A *= a;
    }
  }
  if (active) {
    float* u = Uagg + i * d + v * V::N;
#pragma unroll
    for (int e = 0; e < V::N; e += 4) *reinterpret_cast<float4*>(u + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
  }
  if (blockIdx.y == 0 && lane == 0) Aagg[i] = A;
}

// one block per 4 features; thread j owns tiles [16j, 16j+16)
__global__ __launch_bounds__(256) void ema_tile_carry(const float* __restrict__ Aagg,
                                                      const float* __restrict__ Uagg, int d,
                                                      float* __restrict__ carry) {
  __shared__ float shA[256];
  __shared__ float4 shU[256];
  constexpr int per = kNT / 256;
  const int f0 = blockIdx.x * 4;
  const int j = threadIdx.x;
  // this thread's tiles, all loads in flight at once
  float ta[per];
  float4 tu[per];
#pragma unroll
  for (int q = 0; q < per; ++q) {
    const int64_t i = static_cast<int64_t>(j) * per + q;
    ta[q] = Aagg[i];
    tu[q] = *reinterpret_cast<const float4*>(Uagg + i * d + f0);
  }
  float A = 1.f;
  float4 U = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int q = 0; q < per; ++q) {
    const float a = ta[q];
    const float4 u = tu[q];
    U = make_float4(fmaf(a, U.x, u.x), fmaf(a, U.y, u.y), fmaf(a, U.z, u.z), fmaf(a, U.w, u.w));
    A *= a;
  }
  shA[j] = A;
  shU[j] = U;
  __syncthreads();
  // inclusive Hillis-Steele scan with the (ordered) affine composition
  for (int off = 1; off < 256; off <<= 1) {
    float pa = 1.f;
    float4 pu = make_float4(0.f, 0.f, 0.f, 0.f);
    const bool has = j >= off;
    if (has) { pa = shA[j - off]; pu = shU[j - off]; }
    __syncthreads();
    if (has) {
      const float a = shA[j];
      const float4 u = shU[j];
      shA[j] = a * pa;
      shU[j] = make_float4(fmaf(a, pu.x, u.x), fmaf(a, pu.y, u.y), fmaf(a, pu.z, u.z), fmaf(a, pu.w, u.w));
    }
    __syncthreads();
  }
  float4 cv = j > 0 ? shU[j - 1] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int q = 0; q < per; ++q) {
    const int64_t i = static_cast<int64_t>(j) * per + q;
    *reinterpret_cast<float4*>(carry + i * d + f0) = cv;
    const float a = ta[q];
    const float4 u = tu[q];
    cv = make_float4(fmaf(a, cv.x, u.x), fmaf(a, cv.y, u.y), fmaf(a, cv.z, u.z), fmaf(a, cv.w, u.w));
  }
}

template <int DT>
__global__ __launch_bounds__(256) void ema_tile_expand(const void* __restrict__ z,
                                                       const float* __restrict__ P, int d,
                                                       const int32_t* __restrict__ idx,
                                                       const int64_t* __restrict__ chunk_offsets,
                                                       const int64_t* __restrict__ offsets, int nseq,
                                                       const float* __restrict__ carry,
                                                       void* __restrict__ out) {
  using V = Vec<DT>;
  const int lane = threadIdx.x & 63;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int v = blockIdx.y * 64 + lane;
  const bool active = v < d / V::N;
  const int64_t M = chunk_offsets[nseq];
  const Tile tr = tile_range(M, i);
  if (tr.c0 >= tr.c1) return;
  float x[V::N];
  if (active) {
    const float* cp = carry + i * d + v * V::N;
#pragma unroll
    for (int e = 0; e < V::N; e += 4) {
      const float4 t = *reinterpret_cast<const float4*>(cp + e);
      x[e] = t.x; x[e + 1] = t.y; x[e + 2] = t.z; x[e + 3] = t.w;
    }
  }
  int s = upper_seq(chunk_offsets, nseq, tr.c0);
  for (int64_t c = tr.c0; c < tr.c1; ++c) {
    while (chunk_offsets[s + 1] <= c) ++s;
    const float Pc = P[c];
    const float a = c == chunk_offsets[s] ? 0.f : 1.f - Pc;
    const int64_t t0 = idx[c];
    const int64_t t1 = c + 1 < chunk_offsets[s + 1] ? static_cast<int64_t>(idx[c + 1]) : offsets[s + 1];
    if (active) {
      float zz[V::N];
      V::load(z, c * d + v * V::N, zz);
#pragma unroll
      for (int e = 0; e < V::N; ++e) x[e] = fmaf(a, x[e], Pc * zz[e]);
      for (int64_t t = t0; t < t1; ++t) V::store_nt(out, t * d + v * V::N, x);
    }
  }
}

// rows of a sequence before its first chunk (or all rows if it has none) are 0
template <int DT>
__global__ __launch_bounds__(256) void ema_zero_prefix(const int32_t* __restrict__ idx,
                                                       const int64_t* __restrict__ chunk_offsets,
                                                       const int64_t* __restrict__ offsets, int d,
                                                       void* __restrict__ out) {
  using V = Vec<DT>;
  const int s = blockIdx.x;
  const int64_t cf = chunk_offsets[s];
  const int64_t first = cf < chunk_offsets[s + 1] ? static_cast<int64_t>(idx[cf]) : offsets[s + 1];
  const int64_t t0 = offsets[s];
  const int nvec = d / V::N;
  const int64_t n = (first - t0) * nvec;
  float zero[V::N];
#pragma unroll
  for (int e = 0; e < V::N; ++e) zero[e] = 0.f;
  for (int64_t w = threadIdx.x; w < n; w += blockDim.x) {
    const int64_t t = t0 + w / nvec;
    const int v = static_cast<int>(w % nvec);
    V::store(out, t * d + v * V::N, zero);
  }
}

template <int DT>
void launch_dechunk(const void* z, const float* P, int d, const int32_t* idx,
                    const int64_t* chunk_offsets, const int64_t* offsets, int nseq, void* out,
                    float* ws, hipStream_t st) {
  constexpr int N = Vec<DT>::N;
  float* Aagg = ws;
  float* Uagg = ws + kNT;
  float* carry = Uagg + static_cast<int64_t>(kNT) * d;
  const int nslices = (d / N + 63) / 64;
  const dim3 grid(kNT / 4, nslices);
  hipLaunchKernelGGL(ema_zero_prefix<DT>, dim3(nseq), dim3(256), 0, st, idx, chunk_offsets, offsets, d, out);
  hipLaunchKernelGGL(ema_tile_aggregate<DT>, grid, dim3(256), 0, st, z, P, d, chunk_offsets, nseq, Aagg, Uagg);
  hipLaunchKernelGGL(ema_tile_carry, dim3(d / 4), dim3(256), 0, st, Aagg, Uagg, d, carry);
  hipLaunchKernelGGL(ema_tile_expand<DT>, grid, dim3(256), 0, st, z, P, d, idx, chunk_offsets,
                     offsets, nseq, carry, out);
}

}  // namespace
}  // namespace bllm

using namespace bllm;

extern "C" size_t bllm_dechunk_workspace(int64_t d) {
  return (static_cast<size_t>(kNT) + 2 * static_cast<size_t>(kNT) * static_cast<size_t>(d)) * 4 + 256;
}

extern "C" int bllm_dechunk_ema(const void* z, const float* P, int dtype, int64_t d,
                                const int32_t* idx, const int64_t* chunk_offsets,
                                const int64_t* offsets, int64_t nseq, int64_t total,
                                int64_t max_chunks, void* out, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!z || !P || !idx || !chunk_offsets || !offsets || !out || d < 1 || nseq < 1 || total < 0 ||
      max_chunks < 0)
    return BLLM_E_INVAL;
  if (!valid_dtype(dtype)) return BLLM_E_NOTSUP;
  if ((d * elem_size(dtype)) % 16 != 0 || !aligned16(z) || !aligned16(out)) return BLLM_E_NOTSUP;
  if (total >= (int64_t(1) << 31) || nseq >= (int64_t(1) << 30) || d > (1 << 16)) return BLLM_E_NOTSUP;
  if (!ws || ws_bytes < bllm_dechunk_workspace(d) || !aligned16(ws)) return BLLM_E_WS;
  if (total == 0) return BLLM_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == BLLM_F32)
    launch_dechunk<BLLM_F32>(z, P, static_cast<int>(d), idx, chunk_offsets, offsets,
                             static_cast<int>(nseq), out, static_cast<float*>(ws), st);
  else
    launch_dechunk<BLLM_BF16>(z, P, static_cast<int>(d), idx, chunk_offsets, offsets,
                              static_cast<int>(nseq), out, static_cast<float*>(ws), st);
  return launch_status();
}
