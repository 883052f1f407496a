// Shared device/host helpers for the chunk-layer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bllm.h"

#define BLLM_VERSION_NUMBER 100

namespace bllm {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 <-> f32

__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = static_cast<uint32_t>(b) << 16;
  return v.f;
}

// round to nearest even; NaN stays NaN (quiet bit set)
__host__ __device__ inline uint16_t f32_to_bf16(float f) {
  union { uint32_t u; float f; } v;
  v.f = f;
  uint32_t u = v.u;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 16-byte vector of row elements: 8 bf16 or 4 fp32, unpacked to fp32.
template <int DT> struct Vec;
template <> struct Vec<BLLM_F32> {
  static constexpr int N = 4;
  __device__ static inline void load(const void* base, int64_t elem, float* x) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  __device__ static inline void store(void* base, int64_t elem, const float* x) {
    float4 v = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(static_cast<float*>(base) + elem) = v;
  }
  __device__ static inline void store_nt(void* base, int64_t elem, const float* x) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + elem);
    __builtin_nontemporal_store(x[0], &p->x);
    __builtin_nontemporal_store(x[1], &p->y);
    __builtin_nontemporal_store(x[2], &p->z);
    __builtin_nontemporal_store(x[3], &p->w);
  }
};
template <> struct Vec<BLLM_BF16> {
  static constexpr int N = 8;
  __device__ static inline void load(const void* base, int64_t elem, float* x) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
      x[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
    }
  }
  __device__ static inline uint4 pack(const float* x) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ static inline void store(void* base, int64_t elem, const float* x) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + elem) = pack(x);
  }
  __device__ static inline void store_nt(void* base, int64_t elem, const float* x) {
    const uint4 v = pack(x);
    uint32_t* p = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(base) + elem);
    __builtin_nontemporal_store(v.x, p + 0);
    __builtin_nontemporal_store(v.y, p + 1);
    __builtin_nontemporal_store(v.z, p + 2);
    __builtin_nontemporal_store(v.w, p + 3);
  }
};

__device__ inline float load_elem(const void* base, int64_t i, int dtype) {
  return dtype == BLLM_F32 ? static_cast<const float*>(base)[i]
                           : bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
}

// ---------------------------------------------------------------- wave helpers

// Inclusive integer scan over the 64 lanes of a wave: an inclusive scan
// inside each row of 16 lanes by four DPP row shifts (lanes with no source
// lane read 0), then the three lower rows' totals added by readlane.  No LDS
// round trip (a shuffle scan waits on six LDS permutes).  Every lane of the
// wave must be active; `total` is the wave's sum, in every lane.
template <int N>
__device__ inline int dpp_row_shr(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x110 + N, 0xF, 0xF, true);
}
__device__ inline int wave_incl_scan(int v, int& total) {
  v += dpp_row_shr<1>(v);
  v += dpp_row_shr<2>(v);
  v += dpp_row_shr<4>(v);
  v += dpp_row_shr<8>(v);
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31);
  const int t2 = __builtin_amdgcn_readlane(v, 47), t3 = __builtin_amdgcn_readlane(v, 63);
  const int r = (threadIdx.x & 63) >> 4;
  total = t0 + t1 + t2 + t3;
  return v + (r > 0 ? t0 : 0) + (r > 1 ? t1 : 0) + (r > 2 ? t2 : 0);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// sum over aligned groups of G lanes, every lane of a group gets the sum:
// DPP quad permutes and row mirrors inside a row of 16 lanes, then swizzle
// and permute across rows
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int G>
__device__ inline float group_sum(float v) {
  if (G >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  if (G >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  if (G >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if (G >= 16) v += dpp_f<0x140>(v); // row_mirror
  if (G >= 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // xor 16
  if (G >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

__device__ inline int lane_id() { return __lane_id(); }

// Workgroup barrier that orders LDS only: unlike __syncthreads it does not
// wait for this wave's outstanding global loads, so prefetches stay in flight
// across it.  Global stores are not made visible by it.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// number of set bits of `mask` in lanes below this one
__device__ inline int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// last s in [0, n) with a[s] <= x (a non-decreasing, a[0] <= x); int64 array
__device__ inline int upper_seq(const int64_t* a, int n, int64_t x) {
  int lo = 0, hi = n;  // invariant: a[lo] <= x, answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? BLLM_OK : BLLM_E_HIP;
}

inline int elem_size(int dtype) { return dtype == BLLM_F32 ? 4 : 2; }
inline bool valid_dtype(int dtype) { return dtype == BLLM_F32 || dtype == BLLM_BF16; }

}  // namespace bllm

namespace bllm {
// tiny fills used instead of hipMemsetAsync (safe under stream capture)
[[maybe_unused]] static __global__ void fill_f32(float* p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) p[i] = v;
}
[[maybe_unused]] static __global__ void fill_i64(int64_t* p, int64_t n, int64_t v) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) p[i] = v;
}
}  // namespace bllm
