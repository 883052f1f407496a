// ByteFlow marginal coding rate Delta R_t on fp32 MFMA.
//
// ByteFlow paper page: "lossy coding rate" prerequisite, R(H) = 1/2 logdet(I +
// (d/eps^2) H H^T); method step details, stage 2, Delta R_t = R(h_1..t) -
// R(h_1..t-1).  Delta R_t is the log of the t-th Cholesky pivot of
// I_T + alpha H H^T.  Rows are cut into blocks of c; for block j with rows B_j
// (scaled by sqrt(alpha)) and prefix matrix A_j = I_d + alpha sum_{i<j} H_i^T H_i,
// the pivots of the block's rows are those of S_j = I_c + B_j A_j^{-1} B_j^T
// (Woodbury; the incremental route the page's weakness analysis points to).
// Every block is independent once A_j is known, so each gets one workgroup
// that factors the (d'+c) x (d'+c) quasi-definite matrix
//     [ A_j   B_j^T ]            = L diag(+1 (d'), -1 (c)) L^T
//     [ B_j   -I_c  ]
// with a left-looking blocked signed Cholesky (32-wide panels): columns of the
// A part subtract earlier panels as usual; columns of the S part add the A-part
// panels and subtract the S-part panels.  The diagonal of the S part of L are
// the pivots; Delta R = log(pivot).
//
// Kernels: cr_gram_prefix (A_j for every block, one 32x32 tile per workgroup,
// 4 waves split the rows), cr_factor (one workgroup per block matrix).
// Workspace: nseq * nblk * ldm^2 fp32 (ldm = d' + c), the A part written by
// the first kernel, the rest of L written by the second.
#include <cmath>

#include "common.h"

namespace bllm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ inline floatx16 mfma32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// C/D layout of v_mfma_f32_32x32x2f32: lane l, register r holds element
// (row 8*(r/4) + 4*(l/32) + r%4, column l%32).
__device__ inline int crow(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

struct CRGeom {
  int T, d, dp, c, nblk, ldm;
};

template <int DT>
__global__ __launch_bounds__(256) void cr_gram_prefix(const void* __restrict__ h, float* __restrict__ ws,
                                                      CRGeom g, float alpha) {
  __shared__ float red[4][16][64];
  const int s = blockIdx.y;
  int t = blockIdx.x, I = 0;
  while (t > I) { t -= I + 1; ++I; }
  const int J = t;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int colA = 32 * I + (lane & 31), colB = 32 * J + (lane & 31);
  const bool okA = colA < g.d, okB = colB < g.d;
  const int64_t mstride = static_cast<int64_t>(g.ldm) * g.ldm;
  const int64_t hbase = static_cast<int64_t>(s) * g.T * g.d;
  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int j = 0; j < g.nblk; ++j) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[w][r][lane] = acc[r];
    __syncthreads();
    float* Mj = ws + (static_cast<int64_t>(s) * g.nblk + j) * mstride;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * w + q;
      const float v = red[0][r][lane] + red[1][r][lane] + red[2][r][lane] + red[3][r][lane];
      const int row = 32 * I + crow(r, lane), col = 32 * J + (lane & 31);
      Mj[static_cast<int64_t>(row) * g.ldm + col] = (row == col ? 1.f : 0.f) + alpha * v;
    }
    __syncthreads();
    if (j == g.nblk - 1) break;
    const int rbeg = j * g.c, rend = min(rbeg + g.c, g.T);
    for (int r = rbeg + 2 * w; r < rend; r += 8) {
      const int row = r + (lane >> 5);
      float a = 0.f, b = 0.f;
      if (row < rend) {
        if (okA) a = load_elem(h, hbase + static_cast<int64_t>(row) * g.d + colA, DT);
        if (okB) b = load_elem(h, hbase + static_cast<int64_t>(row) * g.d + colB, DT);
      }
      acc = mfma32(a, b, acc);
    }
  }
}

template <int DT>
__device__ inline float orig_elem(const void* h, const float* Mx, const CRGeom& g, int s, int r0,
                                  int cj, float salpha, int row, int col) {
  if (col >= g.dp) return row == col ? 1.f : 0.f;
  if (row < g.dp) return Mx[static_cast<int64_t>(row) * g.ldm + col];
  const int rr = row - g.dp;
  if (rr >= cj || col >= g.d) return 0.f;
  return salpha * load_elem(h, (static_cast<int64_t>(s) * g.T + r0 + rr) * g.d + col, DT);
}

// acc = orig(tile i, panel k) -/+ sum over earlier panels kk of L[i,kk] L[k,kk]^T
template <int DT>
__device__ inline floatx16 panel_update(const void* h, const float* Mx, const CRGeom& g, int s,
                                        int r0, int cj, float salpha, int i, int k, int ntA,
                                        int lane) {
  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    acc[r] = orig_elem<DT>(h, Mx, g, s, r0, cj, salpha, 32 * i + crow(r, lane), 32 * k + (lane & 31));
  const bool panelS = k >= ntA;
  const float* ra = Mx + static_cast<int64_t>(32 * i + (lane & 31)) * g.ldm + 16 * (lane >> 5);
  const float* rb = Mx + static_cast<int64_t>(32 * k + (lane & 31)) * g.ldm + 16 * (lane >> 5);
  for (int kk = 0; kk < k; ++kk) {
    const float sg = (panelS && kk < ntA) ? 1.f : -1.f;
    float a[16], b[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 x = *reinterpret_cast<const float4*>(ra + 32 * kk + 4 * v);
      const float4 y = *reinterpret_cast<const float4*>(rb + 32 * kk + 4 * v);
      a[4 * v] = sg * x.x; a[4 * v + 1] = sg * x.y; a[4 * v + 2] = sg * x.z; a[4 * v + 3] = sg * x.w;
      b[4 * v] = y.x; b[4 * v + 1] = y.y; b[4 * v + 2] = y.z; b[4 * v + 3] = y.w;
    }
#pragma unroll
    for (int st = 0; st < 16; ++st) acc = mfma32(a[st], b[st], acc);
  }
  return acc;
}

template <int DT>
__global__ __launch_bounds__(256) void cr_factor(const void* __restrict__ h, float* __restrict__ ws,
                                                 float* __restrict__ dR, int32_t* __restrict__ status,
                                                 CRGeom g, float salpha) {
  __shared__ float sdiag[32][33];
  __shared__ float slinv[32][33];
  __shared__ float sstage[4][32][33];
  __shared__ int sbad;
  const int j = blockIdx.x, s = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = j * g.c;
  const int cj = min(g.c, g.T - r0);
  const int n = g.dp + ((cj + 31) & ~31);
  const int nt = n >> 5, ntA = g.dp >> 5;
  float* Mx = ws + (static_cast<int64_t>(s) * g.nblk + j) * static_cast<int64_t>(g.ldm) * g.ldm;
  if (threadIdx.x == 0) sbad = 0;
  for (int k = 0; k < nt; ++k) {
    // phase A: wave w updates tile k + w (wave 0 holds the diagonal tile)
    floatx16 acc0;
    const int i0 = k + w;
    if (i0 < nt) acc0 = panel_update<DT>(h, Mx, g, s, r0, cj, salpha, i0, k, ntA, lane);
    if (w == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sdiag[crow(r, lane)][lane & 31] = acc0[r];
    }
    __syncthreads();
    if (w == 0) {
      // unblocked Cholesky of the 32x32 diagonal tile; lane i < 32 owns row i
      float a[32];
      const int me = lane & 31;
#pragma unroll
      for (int m = 0; m < 32; ++m) a[m] = m <= me ? sdiag[me][m] : 0.f;
      bool bad = false;
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) {
        const float pv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[jj]), jj));
        bad |= !(pv > 0.f);
        const float l = sqrtf(pv);
        const float inv = 1.f / l;
        if (me == jj) a[jj] = l;
        else if (me > jj) a[jj] *= inv;
#pragma unroll
        for (int kk = jj + 1; kk < 32; ++kk) {
          const float lk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[jj]), kk));
          if (me >= kk) a[kk] = fmaf(-a[jj], lk, a[kk]);
        }
      }
      if (lane < 32) {
#pragma unroll
        for (int m = 0; m < 32; ++m) sdiag[me][m] = m <= me ? a[m] : 0.f;
        if (k >= ntA) {
          const int rr = 32 * k + me - g.dp;
          if (rr < cj) dR[static_cast<int64_t>(s) * g.T + r0 + rr] = logf(a[me]);
        }
      }
      if (bad && lane == 0) sbad = 1;
    }
    __syncthreads();
    if (w == 0 && lane < 32) {
      // column `lane` of the inverse of the diagonal tile's factor
      const int m = lane;
      float x[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        float acc = (i == m) ? 1.f : 0.f;
#pragma unroll
        for (int p = 0; p < i; ++p) acc = fmaf(-sdiag[i][p], x[p], acc);
        x[i] = acc / sdiag[i][i];
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) slinv[i][m] = x[i];
    }
    __syncthreads();
    // phase B: X = acc * Linv^T for every tile below the diagonal
#pragma unroll 1
    for (int q = 0;; ++q) {
      const int i = k + w + 4 * q;
      if (i >= nt) break;
      if (i == k) continue;
      floatx16 acc = q == 0 ? acc0 : panel_update<DT>(h, Mx, g, s, r0, cj, salpha, i, k, ntA, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) sstage[w][crow(r, lane)][lane & 31] = acc[r];
      float a[16], b[16];
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        a[st] = sstage[w][lane & 31][16 * (lane >> 5) + st];
        b[st] = slinv[lane & 31][16 * (lane >> 5) + st];
      }
      floatx16 x;
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = 0.f;
#pragma unroll
      for (int st = 0; st < 16; ++st) x = mfma32(a[st], b[st], x);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        Mx[static_cast<int64_t>(32 * i + crow(r, lane)) * g.ldm + 32 * k + (lane & 31)] = x[r];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0 && sbad && status) atomicOr(status, BLLM_S_NONFINITE);
}

CRGeom cr_geometry(int64_t T, int64_t d) {
  CRGeom g;
  g.T = static_cast<int>(T);
  g.d = static_cast<int>(d);
  g.dp = static_cast<int>((d + 31) / 32 * 32);
  int c = (g.dp / 2 + 31) / 32 * 32;
  c = c < 32 ? 32 : (c > 128 ? 128 : c);
  g.c = c;
  g.nblk = static_cast<int>((T + c - 1) / c);
  g.ldm = g.dp + c;
  return g;
}

}  // namespace
}  // namespace bllm

using namespace bllm;

extern "C" size_t bllm_coding_rate_workspace(int64_t nseq, int64_t T, int64_t d) {
  if (nseq < 1 || T < 1 || d < 1) return 0;
  const CRGeom g = cr_geometry(T, d);
  return static_cast<size_t>(nseq) * g.nblk * static_cast<size_t>(g.ldm) * g.ldm * 4 + 256;
}

extern "C" int bllm_coding_rate(const void* h, int dtype, int64_t nseq, int64_t T, int64_t d,
                                double eps2, float* dR_out, int32_t* status, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!h || !dR_out || nseq < 1 || T < 1 || d < 1 || !(eps2 > 0.0)) return BLLM_E_INVAL;
  if (!valid_dtype(dtype)) return BLLM_E_NOTSUP;
  if (d > 640 || nseq > 65535 || T > (int64_t(1) << 24)) return BLLM_E_NOTSUP;
  if (!ws || ws_bytes < bllm_coding_rate_workspace(nseq, T, d) || !aligned16(ws)) return BLLM_E_WS;
  const CRGeom g = cr_geometry(T, d);
  const double alpha = static_cast<double>(d) / eps2;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int nt = g.dp / 32;
  const dim3 ggrid(static_cast<unsigned>(nt * (nt + 1) / 2), static_cast<unsigned>(nseq));
  const dim3 fgrid(static_cast<unsigned>(g.nblk), static_cast<unsigned>(nseq));
  float* w = static_cast<float*>(ws);
  if (dtype == BLLM_F32) {
    hipLaunchKernelGGL(cr_gram_prefix<BLLM_F32>, ggrid, dim3(256), 0, st, h, w, g, static_cast<float>(alpha));
    hipLaunchKernelGGL(cr_factor<BLLM_F32>, fgrid, dim3(256), 0, st, h, w, dR_out, status, g,
                       static_cast<float>(std::sqrt(alpha)));
  } else {
    hipLaunchKernelGGL(cr_gram_prefix<BLLM_BF16>, ggrid, dim3(256), 0, st, h, w, g, static_cast<float>(alpha));
    hipLaunchKernelGGL(cr_factor<BLLM_BF16>, fgrid, dim3(256), 0, st, h, w, dR_out, status, g,
                       static_cast<float>(std::sqrt(alpha)));
  }
  return launch_status();
}
