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
//   1. per tile: its affine aggregate (A = prod a, U = scan end from 0); the
//      same launch zeroes the rows of each sequence before its first chunk
//   2. per 32-feature column block: scan of the kNT aggregates -> carry into
//      each tile
//   3. per tile: rescan from the carry and write every byte row of each chunk
// A wave owns one (tile, feature slice).  It first reads the metadata of up
// to 64 chunks at once, one chunk per lane (P, first row, last row, whether
// the chunk starts its sequence), so that the serial loop over the chunks only
// waits on the z rows, which it loads kUnroll chunks at a time.
// HBM-bound: z is read twice, the [total x d] output is written once
// (nontemporal); the tile aggregates and carries add 3 * kNT * d * 4 bytes.
#include <algorithm>

#include "common.h"

namespace bllm {
namespace {

constexpr int kNT = 2048;      // tiles of consecutive chunks
constexpr int kLaneBytes = 8;  // bytes of a row per lane
constexpr int kUnroll = 4;     // z rows in flight per wave
constexpr int kRowBatch = 8;   // output-gradient rows in flight per wave (backward)
constexpr int kCarryCols = 8;                   // float4 columns per carry block
constexpr int kCarryThreads = 1024;
constexpr int kCarryGroups = kCarryThreads / kCarryCols;
constexpr int kCarryPer = kNT / kCarryGroups;   // tiles per carry thread
static_assert(kNT % kCarryGroups == 0, "tile count must split over the carry groups");

// kLaneBytes of one row per lane (2, 4 or 8 elements), unpacked to fp32
template <int DT> struct Lane {
  static constexpr int E = DT == BLLM_F32 ? 4 : 2;
  static constexpr int N = kLaneBytes / E;
  static constexpr int W = kLaneBytes / 4;  // 32-bit words
  __device__ static inline void load(const void* base, int64_t elem, float* x) {
    const char* p = static_cast<const char*>(base) + elem * E;
    uint32_t w[W];
    if constexpr (W == 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (W == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x; w[1] = v.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if constexpr (DT == BLLM_F32) {
        x[i] = __uint_as_float(w[i]);
      } else {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
  __device__ static inline void store(void* base, int64_t elem, const float* x) {
    uint32_t* p = reinterpret_cast<uint32_t*>(static_cast<char*>(base) + elem * E);
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if constexpr (DT == BLLM_F32)
        p[i] = __float_as_uint(x[i]);
      else
        p[i] = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
    }
  }
  __device__ static inline void store_nt(void* base, int64_t elem, const float* x) {
    uint32_t* p = reinterpret_cast<uint32_t*>(static_cast<char*>(base) + elem * E);
#pragma unroll
    for (int i = 0; i < W; ++i) {
      uint32_t w;
      if constexpr (DT == BLLM_F32)
        w = __float_as_uint(x[i]);
      else
        w = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) |
            (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
      __builtin_nontemporal_store(w, p + i);
    }
  }
};

struct Tile {
  int64_t c0, c1;
};

// Chunk offsets as the kernels see them: every entry clamped to the number of
// chunk rows the caller provides (max_chunks).  When a compaction overflowed
// its capacity, chunk_offsets hold the true counts while only `capacity` rows
// of z, P and idx exist; the chunks past the bound are then treated as absent
// (a sequence cut short keeps its last available chunk to its end, a sequence
// left without chunks gets zero rows), so no kernel reads or writes past them.
struct ChunkOffs {
  const int64_t* p;
  int64_t cap;
  __device__ int64_t operator[](int64_t s) const {
    const int64_t v = p[s];
    return v < cap ? v : cap;
  }
};

// last s in [0, n) with co[s] <= x (co non-decreasing, co[0] <= x)
__device__ inline int upper_seq(const ChunkOffs& co, int n, int64_t x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (co[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ inline Tile tile_range(int64_t M, int64_t i) {
  const int64_t L = (M + kNT - 1) / kNT;
  const int64_t c0 = i * L < M ? i * L : M;
  return {c0, c0 + L < M ? c0 + L : M};
}

// Metadata of chunk c = cb + lane (cb .. ce-1, ce - cb <= 64), one per lane:
// the multiplier a_c, P_c, whether the chunk starts its sequence (1 or 0),
// the first and one-past-last row of the chunk.
// The sequences overlapping the range are walked with wave-uniform loads.
struct ChunkMeta {
  float a, P, start;
  int64_t t0, t1;
};

__device__ inline ChunkMeta chunk_meta(const float* __restrict__ P, const int32_t* __restrict__ idx,
                                       ChunkOffs chunk_offsets,
                                       const int64_t* __restrict__ offsets, int nseq, int64_t M,
                                       int64_t cb, int64_t ce, int lane) {
  const int64_t c = cb + lane < ce ? cb + lane : ce - 1;
  ChunkMeta m;
  m.P = P[c];
  m.t0 = idx[c];
  const int64_t cn = c + 1 < M ? c + 1 : c;
  int64_t t1 = idx[cn];
  bool start = false;
  int s = upper_seq(chunk_offsets, nseq, cb);  // the sequence holding chunk cb
  for (;;) {
    const int64_t cs = chunk_offsets[s], ce_s = chunk_offsets[s + 1];
    if (cs < ce_s) {  // empty sequences own no chunk
      if (c == cs) start = true;
      if (c == ce_s - 1) t1 = offsets[s + 1];
    }
    if (ce_s >= ce || s + 1 >= nseq) break;
    ++s;
  }
  m.a = start ? 0.f : 1.f - m.P;
  m.start = start ? 1.f : 0.f;
  m.t1 = t1;
  return m;
}

__device__ inline float lane_f(float v, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}
__device__ inline int64_t lane_i64(int64_t v, int j) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u & 0xFFFFFFFFu), j));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), j));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Pass 1.  Grid: (kNT/4 + nzero, nslices) blocks of 4 waves; blocks past the
// tiles zero the rows before each sequence's first chunk (slice 0 only).
template <int DT>
__global__ __launch_bounds__(256) void ema_tile_aggregate(const void* __restrict__ z,
                                                          const float* __restrict__ P, int d,
                                                          const int32_t* __restrict__ idx,
                                                          ChunkOffs chunk_offsets,
                                                          const int64_t* __restrict__ offsets,
                                                          int nseq, float* __restrict__ Aagg,
                                                          float* __restrict__ Uagg,
                                                          void* __restrict__ out) {
  using V = Lane<DT>;
  const int lane = threadIdx.x & 63;
  const int nvec = d / V::N;
  if (blockIdx.x >= kNT / 4) {
    if (blockIdx.y != 0) return;
    float zero[V::N];
#pragma unroll
    for (int e = 0; e < V::N; ++e) zero[e] = 0.f;
    const int nzb = gridDim.x - kNT / 4;
    for (int s = blockIdx.x - kNT / 4; s < nseq; s += nzb) {
      const int64_t cf = chunk_offsets[s];
      const int64_t first = cf < chunk_offsets[s + 1] ? static_cast<int64_t>(idx[cf]) : offsets[s + 1];
      const int64_t t0 = offsets[s];
      const int64_t n = (first - t0) * nvec;
      for (int64_t w = threadIdx.x; w < n; w += blockDim.x) {
        const int64_t t = t0 + w / nvec;
        const int v = static_cast<int>(w % nvec);
        V::store_nt(out, t * d + static_cast<int64_t>(v) * V::N, zero);
      }
    }
    return;
  }
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int v = blockIdx.y * 64 + lane;
  const int vc = v < nvec ? v : nvec - 1;  // clamped: every lane loads, the tail lanes do not store
  const int64_t M = chunk_offsets[nseq];
  const Tile tr = tile_range(M, i);
  float x[V::N];
#pragma unroll
  for (int e = 0; e < V::N; ++e) x[e] = 0.f;
  float A = 1.f;
  for (int64_t cb = tr.c0; cb < tr.c1; cb += 64) {
    const int64_t ce = cb + 64 < tr.c1 ? cb + 64 : tr.c1;
    const ChunkMeta m = chunk_meta(P, idx, chunk_offsets, offsets, nseq, M, cb, ce, lane);
    const int n = static_cast<int>(ce - cb);
    for (int j = 0; j < n; j += kUnroll) {
      float zz[kUnroll][V::N];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = cb + (j + u < n ? j + u : n - 1);
        V::load(z, c * d + static_cast<int64_t>(vc) * V::N, zz[u]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (j + u < n) {
          const float a = lane_f(m.a, j + u);
          const float Pc = lane_f(m.P, j + u);
#pragma unroll
          for (int e = 0; e < V::N; ++e) x[e] = fmaf(a, x[e], Pc * zz[u][e]);
          A *= a;
        }
      }
    }
  }
  if (v < nvec) {
    float* u = Uagg + i * d + static_cast<int64_t>(v) * V::N;
#pragma unroll
    for (int e = 0; e < V::N; ++e) u[e] = x[e];
  }
  if (blockIdx.y == 0 && lane == 0) Aagg[i] = A;
}

// affine maps x -> A x + U composed in order: first (a1, u1), then (a2, u2)
__device__ inline void compose(float a1, float4 u1, float a2, float4 u2, float& a, float4& u) {
  a = a2 * a1;
  u = make_float4(fmaf(a2, u1.x, u2.x), fmaf(a2, u1.y, u2.y), fmaf(a2, u1.z, u2.z), fmaf(a2, u1.w, u2.w));
}

__device__ inline float4 shfl_up4(float4 v, int off) {
  return make_float4(__shfl_up(v.x, off, kWave), __shfl_up(v.y, off, kWave), __shfl_up(v.z, off, kWave),
                     __shfl_up(v.w, off, kWave));
}

// Pass 2.  One block per 32 features (whole 128-byte lines of the aggregate
// rows, so no two blocks share a line); thread (group g, column col) owns
// tiles [g*kCarryPer, (g+1)*kCarryPer) of its float4 column.  Group scans:
// within the wave by shuffles (8 groups per wave), across the 16 waves
// through LDS.  Writes the carry into every tile (the scan value before it).
// The tile values are read in batches of at most 16 (twice: for the group
// fold and for the carries) to stay within 128 VGPRs at 1024 threads.
// blockIdx.y = 1 scans a second set of aggregates (the backward's reverse
// scan in the same launch as its forward one)
__global__ __launch_bounds__(kCarryThreads) void ema_tile_carry(const float* __restrict__ Aagg,
                                                                const float* __restrict__ Uagg, int d,
                                                                float* __restrict__ carry,
                                                                const float* __restrict__ Aagg2,
                                                                const float* __restrict__ Uagg2,
                                                                float* __restrict__ carry2) {
  if (blockIdx.y == 1) {
    Aagg = Aagg2;
    Uagg = Uagg2;
    carry = carry2;
  }
  __shared__ float shA[kCarryThreads / kWave][kCarryCols];
  __shared__ float4 shU[kCarryThreads / kWave][kCarryCols];
  const int tid = threadIdx.x;
  const int col = tid & (kCarryCols - 1);
  const int g = tid / kCarryCols;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int f = blockIdx.x * (kCarryCols * 4) + col * 4;
  const bool active = f < d;
  const int fc = active ? f : d - 4;
  constexpr int kBatch = kCarryPer < 16 ? kCarryPer : 16;
  float A = 1.f;
  float4 U = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 1
  for (int q0 = 0; q0 < kCarryPer; q0 += kBatch) {
    float ta[kBatch];
    float4 tu[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int64_t i = static_cast<int64_t>(g) * kCarryPer + q0 + q;
      ta[q] = Aagg[i];
      tu[q] = *reinterpret_cast<const float4*>(Uagg + i * d + fc);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) compose(A, U, ta[q], tu[q], A, U);
  }
  // inclusive scan over the 8 groups of this wave (lanes 8 apart)
#pragma unroll
  for (int off = kCarryCols; off < kWave; off <<= 1) {
    const float pa = __shfl_up(A, off, kWave);
    const float4 pu = shfl_up4(U, off);
    if (lane >= off) compose(pa, pu, A, U, A, U);
  }
  if (lane >= kWave - kCarryCols) {
    shA[wv][col] = A;
    shU[wv][col] = U;
  }
  // exclusive value of this group: previous group of the wave, after the
  // totals of the earlier waves
  float ea = __shfl_up(A, kCarryCols, kWave);
  float4 eu = shfl_up4(U, kCarryCols);
  if (lane < kCarryCols) {
    ea = 1.f;
    eu = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  float pa = 1.f;
  float4 pu = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int w = 0; w < wv; ++w) compose(pa, pu, shA[w][col], shU[w][col], pa, pu);
  float cva;
  float4 cv;
  compose(pa, pu, ea, eu, cva, cv);
  if (!active) return;
#pragma unroll 1
  for (int q0 = 0; q0 < kCarryPer; q0 += kBatch) {
    float ta[kBatch];
    float4 tu[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int64_t i = static_cast<int64_t>(g) * kCarryPer + q0 + q;
      ta[q] = Aagg[i];
      tu[q] = *reinterpret_cast<const float4*>(Uagg + i * d + fc);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int64_t i = static_cast<int64_t>(g) * kCarryPer + q0 + q;
      *reinterpret_cast<float4*>(carry + i * d + f) = cv;
      compose(cva, cv, ta[q], tu[q], cva, cv);
    }
  }
}

// Pass 3.  Same grid as pass 1 without the zeroing blocks.
template <int DT>
__global__ __launch_bounds__(256) void ema_tile_expand(const void* __restrict__ z,
                                                       const float* __restrict__ P, int d,
                                                       const int32_t* __restrict__ idx,
                                                       ChunkOffs chunk_offsets,
                                                       const int64_t* __restrict__ offsets, int nseq,
                                                       const float* __restrict__ carry,
                                                       void* __restrict__ out) {
  using V = Lane<DT>;
  const int lane = threadIdx.x & 63;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int nvec = d / V::N;
  const int v = blockIdx.y * 64 + lane;
  const bool active = v < nvec;
  const int vc = active ? v : nvec - 1;
  const int64_t M = chunk_offsets[nseq];
  const Tile tr = tile_range(M, i);
  if (tr.c0 >= tr.c1) return;
  float x[V::N];
  {
    const float* cp = carry + i * d + static_cast<int64_t>(vc) * V::N;
#pragma unroll
    for (int e = 0; e < V::N; ++e) x[e] = cp[e];
  }
  for (int64_t cb = tr.c0; cb < tr.c1; cb += 64) {
    const int64_t ce = cb + 64 < tr.c1 ? cb + 64 : tr.c1;
    const ChunkMeta m = chunk_meta(P, idx, chunk_offsets, offsets, nseq, M, cb, ce, lane);
    const int n = static_cast<int>(ce - cb);
    for (int j = 0; j < n; j += kUnroll) {
      float zz[kUnroll][V::N];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = cb + (j + u < n ? j + u : n - 1);
        V::load(z, c * d + static_cast<int64_t>(vc) * V::N, zz[u]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (j + u < n) {
          const float a = lane_f(m.a, j + u);
          const float Pc = lane_f(m.P, j + u);
          const int64_t t0 = lane_i64(m.t0, j + u);
          const int64_t t1 = lane_i64(m.t1, j + u);
#pragma unroll
          for (int e = 0; e < V::N; ++e) x[e] = fmaf(a, x[e], Pc * zz[u][e]);
          if (active)
            for (int64_t t = t0; t < t1; ++t) V::store_nt(out, t * d + static_cast<int64_t>(v) * V::N, x);
        }
      }
    }
  }
}

template <int DT>
void launch_dechunk(const void* z, const float* P, int d, const int32_t* idx,
                    const int64_t* chunk_offsets_in, int64_t max_chunks, const int64_t* offsets, int nseq,
                    void* out, float* ws, hipStream_t st) {
  constexpr int N = Lane<DT>::N;
  const ChunkOffs chunk_offsets{chunk_offsets_in, max_chunks};
  float* Aagg = ws;
  float* Uagg = ws + kNT;
  float* carry = Uagg + static_cast<int64_t>(kNT) * d;
  const int nslices = (d / N + 63) / 64;
  const int nzero = nseq < 256 ? nseq : 256;
  hipLaunchKernelGGL(ema_tile_aggregate<DT>, dim3(kNT / 4 + nzero, nslices), dim3(256), 0, st, z, P, d,
                     idx, chunk_offsets, offsets, nseq, Aagg, Uagg, out);
  hipLaunchKernelGGL(ema_tile_carry, dim3((d + kCarryCols * 4 - 1) / (kCarryCols * 4)),
                     dim3(kCarryThreads), 0, st, Aagg, Uagg, d, carry, nullptr, nullptr, nullptr);
  hipLaunchKernelGGL(ema_tile_expand<DT>, dim3(kNT / 4, nslices), dim3(256), 0, st, z, P, d, idx,
                     chunk_offsets, offsets, nseq, carry, out);
}

// ------------------------------------------------------------------ backward
// Gradients of L = sum(dout * out) for the EMA dechunk (ByteGen report,
// section 2.3: the EMA keeps the chunking differentiable end to end).  Per
// chunk c: gbar_c = sum of dout over the chunk's rows; the adjoint
// lam_c = dL/dzbar_c runs backwards, lam_c = gbar_c + a_{c+1} lam_{c+1}
// (a_{c+1} = 0 when c + 1 starts a sequence or c is the last chunk);
// dz_c = P_c lam_c; dP_c = lam_c . (z_c - zbar_{c-1}) with zbar_{c-1} = 0 at a
// sequence's first chunk.  Same tiles and slices as the forward:
//   1. per tile: the forward aggregate (A, U_f) over z, the chunk sums gbar_c
//      (stored in the activations' type) and the reverse aggregate U_r = a_{c0} sum_c pi_c gbar_c
//      with pi_c = prod_{c0 < j <= c} a_j, accumulated in ascending order; the
//      reverse aggregates are stored in reversed tile order
//   2. the forward carry scan, and the same scan over the reversed tiles,
//      which gives mu_i = a_{c1} lam_{c1}, what flows into tile i from the right
//   3. per tile, descending: lam_c from mu_i, written over gbar_c
//   4. per tile, ascending: zbar from the forward carry; dz_c = P_c lam_c and
//      one partial dot product per feature slice
//   5. dP_c = the slice partials summed in slice order
// (the two scans of 2 run in one launch, and 3 and 4 in one launch, each wave
// rescanning its tile from the right and then from the left)
// HBM: dout read once; z read twice; gbar/lam (M x d, the activations' type;
// every sum and scan runs in fp32) written twice and read twice (the second
// read mostly from the cache); dz written once.

template <int DT>
__global__ __launch_bounds__(256) void emab_aggregate(const void* __restrict__ z,
                                                      const float* __restrict__ P,
                                                      const void* __restrict__ dout, int d,
                                                      const int32_t* __restrict__ idx,
                                                      ChunkOffs chunk_offsets,
                                                      const int64_t* __restrict__ offsets, int nseq,
                                                      float* __restrict__ Aagg, float* __restrict__ Uf,
                                                      float* __restrict__ Arev, float* __restrict__ Urev,
                                                      void* __restrict__ gbar) {
  using V = Lane<DT>;
  const int lane = threadIdx.x & 63;
  const int nvec = d / V::N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int v = blockIdx.y * 64 + lane;
  const bool active = v < nvec;
  const int vc = active ? v : nvec - 1;
  const int64_t col = static_cast<int64_t>(vc) * V::N;
  const int64_t M = chunk_offsets[nseq];
  const Tile tr = tile_range(M, i);
  float xf[V::N], ur[V::N], gs[V::N];
#pragma unroll
  for (int e = 0; e < V::N; ++e) xf[e] = ur[e] = gs[e] = 0.f;
  float A = 1.f, pi = 1.f, a0 = 1.f;
  for (int64_t cb = tr.c0; cb < tr.c1; cb += 64) {
    const int64_t ce = cb + 64 < tr.c1 ? cb + 64 : tr.c1;
    const ChunkMeta m = chunk_meta(P, idx, chunk_offsets, offsets, nseq, M, cb, ce, lane);
    const int n = static_cast<int>(ce - cb);
    if (cb > tr.c0) pi *= lane_f(m.a, 0);  // the group's first chunk continues the product
    // forward aggregate over z, kUnroll chunks in flight
    for (int j = 0; j < n; j += kUnroll) {
      float zz[kUnroll][V::N];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) V::load(z, (cb + (j + u < n ? j + u : n - 1)) * d + col, zz[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (j + u < n) {
          const float a = lane_f(m.a, j + u);
          const float Pc = lane_f(m.P, j + u);
#pragma unroll
          for (int e = 0; e < V::N; ++e) xf[e] = fmaf(a, xf[e], Pc * zz[u][e]);
          A *= a;
        }
      }
    }
    // chunk sums of dout over the group's rows, kRowBatch rows in flight; a
    // chunk is closed when the rows pass its end: gbar stored, reverse
    // aggregate ur += pi_c gbar_c, then pi picks up the next chunk's a.  Rows
    // between a sequence's end and the next chunk (a sequence that does not
    // start with a boundary) belong to no chunk and are skipped.
    const int64_t r0 = lane_i64(m.t0, 0), r1 = lane_i64(m.t1, n - 1);
    int j = 0;
    int64_t tbeg = r0, tend = lane_i64(m.t1, 0);
    for (int64_t t = r0; t < r1; t += kRowBatch) {
      float g8[kRowBatch][V::N];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) V::load(dout, (t + u < r1 ? t + u : r1 - 1) * d + col, g8[u]);
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        if (t + u < r1) {
          if (t + u >= tend) {  // row t + u opens chunk j + 1
            const int64_t c = cb + j;
            if (active) V::store(gbar, c * d + col, gs);
            if (c == tr.c0) a0 = lane_f(m.a, j);
#pragma unroll
            for (int e = 0; e < V::N; ++e) {
              ur[e] = fmaf(pi, gs[e], ur[e]);
              gs[e] = 0.f;
            }
            ++j;
            pi *= lane_f(m.a, j);
            tbeg = lane_i64(m.t0, j);
            tend = lane_i64(m.t1, j);
          }
          if (t + u >= tbeg) {
#pragma unroll
            for (int e = 0; e < V::N; ++e) gs[e] += g8[u][e];
          }
        }
      }
    }
    {  // close the group's last chunk
      const int64_t c = cb + j;
      if (active) V::store(gbar, c * d + col, gs);
      if (c == tr.c0) a0 = lane_f(m.a, j);
#pragma unroll
      for (int e = 0; e < V::N; ++e) {
        ur[e] = fmaf(pi, gs[e], ur[e]);
        gs[e] = 0.f;
      }
    }
  }
  const int64_t ir = kNT - 1 - i;
  if (active) {
    float* uf = Uf + i * d + col;
    float* urp = Urev + ir * d + col;
#pragma unroll
    for (int e = 0; e < V::N; ++e) {
      uf[e] = xf[e];
      urp[e] = a0 * ur[e];
    }
  }
  if (blockIdx.y == 0 && lane == 0) {
    Aagg[i] = A;
    Arev[ir] = A;
  }
}

// 3. lam_c over the tile, last chunk first, written over gbar_c
template <int DT>
__device__ inline void emab_reverse(const float* __restrict__ P, int d,
                                                    const int32_t* __restrict__ idx,
                                                    ChunkOffs chunk_offsets,
                                                    const int64_t* __restrict__ offsets, int nseq,
                                                    const float* __restrict__ carry_rev,
                                                    void* __restrict__ lam) {
  using V = Lane<DT>;
  const int lane = threadIdx.x & 63;
  const int nvec = d / V::N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int v = blockIdx.y * 64 + lane;
  const bool active = v < nvec;
  const int vc = active ? v : nvec - 1;
  const int64_t col = static_cast<int64_t>(vc) * V::N;
  const int64_t M = chunk_offsets[nseq];
  const Tile tr = tile_range(M, i);
  if (tr.c0 >= tr.c1) return;
  // mu_i: what flows into the tile's last chunk from the right
  float mu[V::N];
  {
    const float* cp = carry_rev + (kNT - 1 - i) * d + col;
#pragma unroll
    for (int e = 0; e < V::N; ++e) mu[e] = cp[e];
  }
  const int64_t ngrp = (tr.c1 - tr.c0 + 63) / 64;
  for (int64_t gi = ngrp - 1; gi >= 0; --gi) {
    const int64_t cb = tr.c0 + gi * 64;
    const int64_t ce = cb + 64 < tr.c1 ? cb + 64 : tr.c1;
    const ChunkMeta m = chunk_meta(P, idx, chunk_offsets, offsets, nseq, M, cb, ce, lane);
    const int n = static_cast<int>(ce - cb);
    for (int j = n - 1; j >= 0; j -= 4) {
      float gv[4][V::N];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jj = j - u >= 0 ? j - u : 0;
        V::load(lam, (cb + jj) * d + col, gv[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j - u >= 0) {
#pragma unroll
          for (int e = 0; e < V::N; ++e) mu[e] += gv[u][e];  // mu now holds lam_c
          if (active) V::store(lam, (cb + j - u) * d + col, mu);
          const float a = lane_f(m.a, j - u);  // a_c: carries lam_c to chunk c - 1
#pragma unroll
          for (int e = 0; e < V::N; ++e) mu[e] *= a;
        }
      }
    }
  }
}

// 4. zbar from the forward carry, dz_c = P_c lam_c, and the slice's partial dP_c
template <int DT>
__device__ inline void emab_forward(const void* __restrict__ z,
                                                    const float* __restrict__ P, int d,
                                                    const int32_t* __restrict__ idx,
                                                    ChunkOffs chunk_offsets,
                                                    const int64_t* __restrict__ offsets, int nseq,
                                                    const float* __restrict__ carry,
                                                    const void* __restrict__ lam,
                                                    void* __restrict__ dz, float* __restrict__ dPpart,
                                                    int64_t mcap) {
  using V = Lane<DT>;
  const int lane = threadIdx.x & 63;
  const int nvec = d / V::N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int v = blockIdx.y * 64 + lane;
  const bool active = v < nvec;
  const int vc = active ? v : nvec - 1;
  const int64_t col = static_cast<int64_t>(vc) * V::N;
  const int64_t M = chunk_offsets[nseq];
  const Tile tr = tile_range(M, i);
  if (tr.c0 >= tr.c1) return;
  float x[V::N];
  {
    const float* cp = carry + i * d + col;
#pragma unroll
    for (int e = 0; e < V::N; ++e) x[e] = cp[e];
  }
  float* dpp = dPpart + static_cast<int64_t>(blockIdx.y) * mcap;
  for (int64_t cb = tr.c0; cb < tr.c1; cb += 64) {
    const int64_t ce = cb + 64 < tr.c1 ? cb + 64 : tr.c1;
    const ChunkMeta m = chunk_meta(P, idx, chunk_offsets, offsets, nseq, M, cb, ce, lane);
    const int n = static_cast<int>(ce - cb);
    for (int j = 0; j < n; j += kUnroll) {
      float zz[kUnroll][V::N], lv[kUnroll][V::N];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = cb + (j + u < n ? j + u : n - 1);
        V::load(z, c * d + col, zz[u]);
        V::load(lam, c * d + col, lv[u]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (j + u < n) {
          const int64_t c = cb + j + u;
          const float a = lane_f(m.a, j + u);
          const float Pc = lane_f(m.P, j + u);
          // zbar_{c-1} counts as 0 at a sequence's first chunk
          const float keep = 1.f - lane_f(m.start, j + u);
          float part = 0.f, g[V::N];
#pragma unroll
          for (int e = 0; e < V::N; ++e) {
            part = fmaf(lv[u][e], zz[u][e] - keep * x[e], part);
            g[e] = Pc * lv[u][e];
            x[e] = fmaf(a, x[e], Pc * zz[u][e]);
          }
          if (active) V::store_nt(dz, c * d + col, g);
          part = group_sum<64>(active ? part : 0.f);
          if (lane == 0) dpp[c] = part;
        }
      }
    }
  }
}

// 3 and 4 in one launch: each wave rescans its (tile, feature slice) from the
// right and then from the left, so the lam_c it has just written are read
// back from the cache instead of memory
template <int DT>
__global__ __launch_bounds__(256) void emab_rescan(const void* __restrict__ z, const float* __restrict__ P, int d,
                                                   const int32_t* __restrict__ idx, ChunkOffs chunk_offsets,
                                                   const int64_t* __restrict__ offsets, int nseq,
                                                   const float* __restrict__ carry,
                                                   const float* __restrict__ carry_rev, void* __restrict__ lam,
                                                   void* __restrict__ dz, float* __restrict__ dPpart, int64_t mcap) {
  emab_reverse<DT>(P, d, idx, chunk_offsets, offsets, nseq, carry_rev, lam);
  // this wave's lam stores complete before its loads of the same words
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  emab_forward<DT>(z, P, d, idx, chunk_offsets, offsets, nseq, carry, lam, dz, dPpart, mcap);
}

__global__ __launch_bounds__(256) void emab_dp_reduce(const float* __restrict__ dPpart,
                                                      ChunkOffs chunk_offsets, int nseq,
                                                      int nslices, int64_t mcap, float* __restrict__ dP) {
  const int64_t M = chunk_offsets[nseq];
  for (int64_t c = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; c < M;
       c += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float s = 0.f;
    for (int k = 0; k < nslices; ++k) s += dPpart[k * mcap + c];
    dP[c] = s;
  }
}

struct BwdWs {
  float *Aagg, *Uf, *Arev, *Urev, *carry, *carry_rev, *lam, *dPpart;
};

__host__ inline size_t bwd_ws_bytes(int64_t d, int nslices, int64_t mcap) {
  return (2 * static_cast<size_t>(kNT) + 4 * static_cast<size_t>(kNT) * d +
          static_cast<size_t>(mcap) * d + static_cast<size_t>(nslices) * mcap) * 4 + 512;
}

__host__ inline BwdWs bwd_ws(void* ws, int64_t d, int64_t mcap) {
  float* p = static_cast<float*>(ws);
  BwdWs b;
  b.Aagg = p; p += kNT;
  b.Arev = p; p += kNT;
  b.Uf = p; p += static_cast<size_t>(kNT) * d;
  b.Urev = p; p += static_cast<size_t>(kNT) * d;
  b.carry = p; p += static_cast<size_t>(kNT) * d;
  b.carry_rev = p; p += static_cast<size_t>(kNT) * d;
  b.lam = p; p += static_cast<size_t>(mcap) * d;
  b.dPpart = p;
  return b;
}

template <int DT>
void launch_dechunk_bwd(const void* z, const float* P, const void* dout, int d, const int32_t* idx,
                        const int64_t* chunk_offsets_in, const int64_t* offsets, int nseq, int64_t mcap,
                        void* dz, float* dP, void* ws, hipStream_t st) {
  constexpr int N = Lane<DT>::N;
  const ChunkOffs chunk_offsets{chunk_offsets_in, mcap};
  const int nslices = (d / N + 63) / 64;
  const BwdWs w = bwd_ws(ws, d, mcap);
  const dim3 grid(kNT / 4, nslices);
  const dim3 cgrid((d + kCarryCols * 4 - 1) / (kCarryCols * 4));
  hipLaunchKernelGGL(emab_aggregate<DT>, grid, dim3(256), 0, st, z, P, dout, d, idx, chunk_offsets, offsets,
                     nseq, w.Aagg, w.Uf, w.Arev, w.Urev, w.lam);
  hipLaunchKernelGGL(ema_tile_carry, dim3(cgrid.x, 2), dim3(kCarryThreads), 0, st, w.Aagg, w.Uf, d, w.carry,
                     w.Arev, w.Urev, w.carry_rev);
  hipLaunchKernelGGL(emab_rescan<DT>, grid, dim3(256), 0, st, z, P, d, idx, chunk_offsets, offsets, nseq,
                     w.carry, w.carry_rev, w.lam, dz, w.dPpart, mcap);
  const unsigned rblocks = static_cast<unsigned>(std::min<int64_t>(ceil_div(mcap, 256), 1024));
  hipLaunchKernelGGL(emab_dp_reduce, dim3(rblocks > 0 ? rblocks : 1), dim3(256), 0, st, w.dPpart, chunk_offsets,
                     nseq, nslices, mcap, dP);
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
  if (!chunk_offsets || !offsets || d < 1 || nseq < 1 || total < 0 || max_chunks < 0) return BLLM_E_INVAL;
  if (total > 0 && !out) return BLLM_E_INVAL;  // may be NULL for an empty batch
  if (total > 0 && max_chunks > 0 && (!z || !P || !idx)) return BLLM_E_INVAL;  // never read without chunks
  if (!valid_dtype(dtype)) return BLLM_E_NOTSUP;
  if ((d * elem_size(dtype)) % 16 != 0 || !aligned16(z) || !aligned16(out)) return BLLM_E_NOTSUP;
  if (total >= (int64_t(1) << 31) || nseq >= (int64_t(1) << 30) || d > (1 << 16)) return BLLM_E_NOTSUP;
  if (!ws || ws_bytes < bllm_dechunk_workspace(d) || !aligned16(ws)) return BLLM_E_WS;
  if (total == 0) return BLLM_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == BLLM_F32)
    launch_dechunk<BLLM_F32>(z, P, static_cast<int>(d), idx, chunk_offsets, max_chunks, offsets,
                             static_cast<int>(nseq), out, static_cast<float*>(ws), st);
  else
    launch_dechunk<BLLM_BF16>(z, P, static_cast<int>(d), idx, chunk_offsets, max_chunks, offsets,
                              static_cast<int>(nseq), out, static_cast<float*>(ws), st);
  return launch_status();
}

extern "C" size_t bllm_dechunk_ema_backward_workspace(int64_t d, int64_t max_chunks) {
  if (d < 1 || max_chunks < 0) return 0;
  // the larger of the two dtypes' slice counts (fp32 lanes hold fewer features)
  const int nslices = static_cast<int>((d * 4 / kLaneBytes + kWave - 1) / kWave);
  return bwd_ws_bytes(d, nslices, max_chunks);
}

extern "C" int bllm_dechunk_ema_backward(const void* z, const float* P, const void* dout, int dtype,
                                         int64_t d, const int32_t* idx, const int64_t* chunk_offsets,
                                         const int64_t* offsets, int64_t nseq, int64_t total,
                                         int64_t max_chunks, void* dz_out, float* dP_out, void* ws,
                                         size_t ws_bytes, void* stream) {
  if (!chunk_offsets || !offsets || d < 1 || nseq < 1 || total < 0 || max_chunks < 0) return BLLM_E_INVAL;
  if (total > 0 && (!z || !P || !dout || !idx || !dz_out || !dP_out)) return BLLM_E_INVAL;  // NULL when empty
  if (!valid_dtype(dtype)) return BLLM_E_NOTSUP;
  if ((d * elem_size(dtype)) % 16 != 0 || !aligned16(z) || !aligned16(dout) || !aligned16(dz_out))
    return BLLM_E_NOTSUP;
  if (total >= (int64_t(1) << 31) || nseq >= (int64_t(1) << 30) || d > (1 << 16)) return BLLM_E_NOTSUP;
  if (!ws || ws_bytes < bllm_dechunk_ema_backward_workspace(d, max_chunks) || !aligned16(ws)) return BLLM_E_WS;
  if (total == 0 || max_chunks == 0) return BLLM_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == BLLM_F32)
    launch_dechunk_bwd<BLLM_F32>(z, P, dout, static_cast<int>(d), idx, chunk_offsets, offsets,
                                 static_cast<int>(nseq), max_chunks, dz_out, dP_out, ws, st);
  else
    launch_dechunk_bwd<BLLM_BF16>(z, P, dout, static_cast<int>(d), idx, chunk_offsets, offsets,
                                  static_cast<int>(nseq), max_chunks, dz_out, dP_out, ws, st);
  return launch_status();
}
