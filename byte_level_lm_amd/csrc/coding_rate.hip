// ByteFlow marginal coding rate Delta R_t on MFMA.
//
// ByteFlow paper page: "lossy coding rate" prerequisite, R(H) = 1/2 logdet(I +
// (d/eps^2) H H^T); method step details, stage 2, Delta R_t = R(h_1..t) -
// R(h_1..t-1).  Delta R_t is the log of the t-th Cholesky pivot of
// I_T + alpha H H^T.  Rows are cut into blocks of c; for block j with rows B_j
// (scaled by sqrt(alpha)) and prefix matrix A_j = I_d + alpha sum_{i<j} H_i^T H_i,
// the pivots of the block's rows are those of S_j = I_c + B_j A_j^{-1} B_j^T
// (Woodbury; the incremental route the page's weakness analysis points to).
// Every block is independent once A_j is known; each block matrix
//     [ A_j   B_j^T ]            = L diag(+1 (d'), -1 (c)) L^T
//     [ B_j   -I_c  ]
// is factored by a blocked signed Cholesky with 64-wide panels: columns of
// the A part subtract earlier panels as usual; columns of the S part add the
// A-part panels and subtract the S-part panels.  The diagonal of the S part
// of L are the pivots; Delta R = log(pivot).
//
// Launch sequence for a batch (all block matrices of all sequences at once):
//   cr_gram_prefix  A_j for every block j (64x64 output tile per workgroup,
//                   bf16 or fp32 MFMA over rows staged transposed in LDS)
//   for each panel k:
//     cr_diag       one wave per matrix factors the 64x64 diagonal tile (k, k),
//                   writes the S-part pivots' logs and the inverse of the factor
//     cr_panel      every tile below the diagonal of panel k, two tiles per
//                   workgroup (left-looking update over the earlier panels on
//                   bf16 MFMA with three-part splits, then X = acc L_kk^-T on
//                   fp32 MFMA); the first workgroup also builds the next
//                   diagonal tile
// Workspace: nmat = nseq * nblk matrices of ldm^2 fp32 (ldm = d' + c), plus a
// 64x64 inverse slot per matrix.
//
// A batch of at least kSplitMatrices block matrices runs as two halves (whole
// sequences each): one on the caller's stream, one on a stream the library
// owns, forked and joined with events.  The halves' launch sequences then
// overlap, so one half's latency-bound diagonal launches and the partly
// filled last rounds of its panel launches share the chip with the other
// half's work (-5% at 32 x 8192 x 512 against one sequence of launches).
#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.h"

namespace bllm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NB = 64;  // panel width

__device__ inline floatx16 mfma32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// C/D layout of the 32x32 MFMAs: lane l, register r holds element
// (row 8*(r/4) + 4*(l/32) + r%4, column l%32).
__device__ inline int crow(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ inline floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

struct CRGeom {
  int T, d, dp, c, nblk, ldm, nmat, nseq;
};

// Gram tiles: 1-D grid of ceil(nseq/8)*8 * ntp blocks.  Block b runs on XCD
// b % 8; every tile of one sequence lands on the same XCD so the rows of h
// they all stream are fetched into that XCD's L2 once.
__device__ inline bool gram_tile_of_block(const CRGeom& g, int& s, int& t) {
  const int ntile = g.dp / 64, ntp = ntile * (ntile + 1) / 2;
  const int b = blockIdx.x, xcd = b & 7, q = b >> 3;
  s = (q / ntp) * 8 + xcd;
  t = q % ntp;
  return s < g.nseq;
}

__device__ inline int block_rows(const CRGeom& g, int j) { return min(g.c, g.T - j * g.c); }
__device__ inline int block_n(const CRGeom& g, int j) {
  return g.dp + ((block_rows(g, j) + NB - 1) / NB) * NB;
}

// ------------------------------------------------------------------ Gram prefix

template <int DT> struct GramLds;
template <> struct GramLds<BLLM_BF16> { typedef uint16_t T; static constexpr int LD = 40; };
template <> struct GramLds<BLLM_F32> { typedef float T; static constexpr int LD = 36; };

// rows [r0, r0+32) (those < rend) of feature strip [f0, f0+64) -> s[feature][row]
template <int DT>
__device__ inline void stage_strip(const void* h, int64_t hrow0, int d, int r0, int rend, int f0,
                                   typename GramLds<DT>::T* s) {
  constexpr int LD = GramLds<DT>::LD;
  const int t = threadIdx.x;
  if (DT == BLLM_BF16) {
    const int row = t >> 3, fc = (t & 7) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + row < rend && f0 + fc < d)
      v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(h) + (hrow0 + r0 + row) * d + f0 + fc);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint16_t* sb = reinterpret_cast<uint16_t*>(s);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sb[(fc + 2 * e) * LD + row] = static_cast<uint16_t>(w[e] & 0xFFFFu);
      sb[(fc + 2 * e + 1) * LD + row] = static_cast<uint16_t>(w[e] >> 16);
    }
  } else {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = (t >> 4) + 16 * hh, fc = (t & 15) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r0 + row < rend && f0 + fc < d)
        v = *reinterpret_cast<const float4*>(static_cast<const float*>(h) + (hrow0 + r0 + row) * d + f0 + fc);
      float* sf = reinterpret_cast<float*>(s);
      sf[(fc + 0) * LD + row] = v.x;
      sf[(fc + 1) * LD + row] = v.y;
      sf[(fc + 2) * LD + row] = v.z;
      sf[(fc + 3) * LD + row] = v.w;
    }
  }
}

template <int DT>
__device__ inline floatx16 gram_chunk(const typename GramLds<DT>::T* sI, const typename GramLds<DT>::T* sJ,
                                      int wm, int wn, int lane, floatx16 acc) {
  constexpr int LD = GramLds<DT>::LD;
  if (DT == BLLM_BF16) {
#pragma unroll
    for (int k0 = 0; k0 < 32; k0 += 16) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(sI) +
                                                        (32 * wm + (lane & 31)) * LD + k0 + 8 * (lane >> 5));
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(sJ) +
                                                        (32 * wn + (lane & 31)) * LD + k0 + 8 * (lane >> 5));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
  } else {
    const float* pa = reinterpret_cast<const float*>(sI) + (32 * wm + (lane & 31)) * LD + 16 * (lane >> 5);
    const float* pb = reinterpret_cast<const float*>(sJ) + (32 * wn + (lane & 31)) * LD + 16 * (lane >> 5);
#pragma unroll
    for (int st = 0; st < 16; ++st) acc = mfma32(pa[st], pb[st], acc);
  }
  return acc;
}

// The carried prefix matrix S of a stream (fp32 [d x d] per sequence, row
// major) enters as the accumulator's start, (S - I) / alpha, so that
// I + alpha acc is S before the window's first row (zero where there is no
// carry and past d): the entries (r0 + crow(r), c0 + lane % 32) of one
// wave's 32x32 quadrant.
__device__ inline floatx16 carried_acc(const float* sin, const CRGeom& g, int s, int r0, int c0, int lane,
                                       float alpha) {
  floatx16 a = zero16();
  if (!sin) return a;
  const int col = c0 + (lane & 31);
  const float inv = 1.f / alpha;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = r0 + crow(r, lane);
    if (row < g.d && col < g.d)
      a[r] = (sin[(static_cast<int64_t>(s) * g.d + row) * g.d + col] - (row == col ? 1.f : 0.f)) * inv;
  }
  return a;
}

// The next window's carry, I + alpha acc after the window's last row,
// written to the quadrant and to its mirror image above the diagonal.
__device__ inline void write_carry(float* sout, const CRGeom& g, int s, int r0, int c0, int lane,
                                   const floatx16& acc, float alpha) {
  if (!sout) return;
  const int col = c0 + (lane & 31);
  float* o = sout + static_cast<int64_t>(s) * g.d * g.d;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = r0 + crow(r, lane);
    if (row >= g.d || col >= g.d) continue;
    const float v = (row == col ? 1.f : 0.f) + alpha * acc[r];
    o[static_cast<int64_t>(row) * g.d + col] = v;
    if (row / 64 != col / 64) o[static_cast<int64_t>(col) * g.d + row] = v;
  }
}

// One 64x64 tile (I >= J) of A_j for all blocks j of one sequence; wave
// (wm, wn) owns the 32x32 quadrant and keeps its running sum in registers.
template <int DT>
__global__ __launch_bounds__(256) void cr_gram_prefix(const void* __restrict__ h, float* __restrict__ ws,
                                                      CRGeom g, float alpha, const float* sin, float* sout) {
  typedef typename GramLds<DT>::T E;
  constexpr int LD = GramLds<DT>::LD;
  __shared__ __attribute__((aligned(16))) E sI[64 * LD];
  __shared__ __attribute__((aligned(16))) E sJ[64 * LD];
  int s, t;
  if (!gram_tile_of_block(g, s, t)) return;
  int I = 0;
  while (t > I) { t -= I + 1; ++I; }
  const int J = t;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = w >> 1, wn = w & 1;
  const int64_t mstride = static_cast<int64_t>(g.ldm) * g.ldm;
  const int64_t hrow0 = static_cast<int64_t>(s) * g.T;
  floatx16 acc = carried_acc(sin, g, s, 64 * I + 32 * wm, 64 * J + 32 * wn, lane, alpha);
  for (int j = 0; j <= g.nblk; ++j) {
    if (j == g.nblk) {
      write_carry(sout, g, s, 64 * I + 32 * wm, 64 * J + 32 * wn, lane, acc, alpha);
      break;
    }
    float* Mj = ws + (static_cast<int64_t>(s) * g.nblk + j) * mstride;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 64 * I + 32 * wm + crow(r, lane), col = 64 * J + 32 * wn + (lane & 31);
      Mj[static_cast<int64_t>(row) * g.ldm + col] = (row == col ? 1.f : 0.f) + alpha * acc[r];
    }
    if (j == g.nblk - 1 && !sout) break;
    const int rbeg = j * g.c, rend = min(rbeg + g.c, g.T);
    for (int r0 = rbeg; r0 < rend; r0 += 32) {
      __syncthreads();
      stage_strip<DT>(h, hrow0, g.d, r0, rend, 64 * I, sI);
      if (I != J) stage_strip<DT>(h, hrow0, g.d, r0, rend, 64 * J, sJ);
      __syncthreads();
      acc = gram_chunk<DT>(sI, I != J ? sJ : sI, wm, wn, lane, acc);
    }
  }
}

// bf16 input: the same 64x64 prefix tiles, rows taken in sub-chunks of R = 128
// rows (64 when c is not a multiple of 128), so a block holds c / R of them.
// Rows are staged row-major in LDS with plain 16-byte stores; the MFMA
// operands (8 consecutive rows of one feature per lane) are read with the
// gfx950 transposing LDS read ds_read_b64_tr_b16: within each 16-lane group,
// lane j points at row j/4 and features 4 (j % 4) .. +3, and lane i receives
// feature i of those 4 rows.  Registers hold the next sub-chunk's rows; the
// barriers around the single LDS stage order LDS only, so those loads stay in
// flight across them.
typedef short shortx4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 tr_frag(const uint16_t* s, int row, int col, int pitch) {
  typedef __attribute__((address_space(3))) shortx4 lds_s4;
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(s + row * pitch + col));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(s + (row + 4) * pitch + col));
  bf16x8 v;
  __builtin_memcpy(&v, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&v) + 8, &hi, 8);
  return v;
}

__global__ __launch_bounds__(256) void cr_gram_prefix_bf16(const uint16_t* __restrict__ h,
                                                           float* __restrict__ ws, CRGeom g, float alpha,
                                                           const float* sin, float* sout) {
  constexpr int GP = 72;  // LDS pitch (bf16) of a staged row: 64 features + 8 pad
  __shared__ __attribute__((aligned(16))) uint16_t sI[128 * GP];
  __shared__ __attribute__((aligned(16))) uint16_t sJ[128 * GP];
  int s, tt;
  if (!gram_tile_of_block(g, s, tt)) return;
  int I = 0;
  while (tt > I) { tt -= I + 1; ++I; }
  const int J = tt;
  const bool same = I == J;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  const int64_t mstride = static_cast<int64_t>(g.ldm) * g.ldm;
  const int R = g.c % 128 == 0 ? 128 : 64;
  const int spb = g.c / R;                // sub-chunks per block
  const int nq = (g.nblk - (sout ? 0 : 1)) * spb;  // sub-chunks that feed some prefix or the carry
  const int lr = tid >> 3, lc = (tid & 7) * 8;  // rows lr + 32 q, features lc .. lc + 7
  const bool fiok = 64 * I + lc < g.d, fjok = 64 * J + lc < g.d;
  const uint16_t* hI = h + static_cast<int64_t>(s) * g.T * g.d + 64 * I + lc;
  const uint16_t* hJ = h + static_cast<int64_t>(s) * g.T * g.d + 64 * J + lc;
  // one sub-chunk: rows q R + lr + 32 e; rows past the sequence or features
  // past d read row 0 / feature 0 and are masked to zero (unconditional loads)
  auto ld = [&](const uint16_t* base, bool fok, int q, int e) {
    const int r = q * R + lr + 32 * e;
    const bool ok = fok && r < g.T && lr + 32 * e < R;
    uint4 v = *reinterpret_cast<const uint4*>(base - (fok ? 0 : lc) + static_cast<int64_t>(ok ? r : 0) * g.d);
    const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
    v.x &= m; v.y &= m; v.z &= m; v.w &= m;
    return v;
  };
  uint4 ai0, ai1, ai2, ai3, aj0, aj1, aj2, aj3;
  auto fetch_a = [&](int q) {
    ai0 = ld(hI, fiok, q, 0); ai1 = ld(hI, fiok, q, 1); ai2 = ld(hI, fiok, q, 2); ai3 = ld(hI, fiok, q, 3);
    if (!same) { aj0 = ld(hJ, fjok, q, 0); aj1 = ld(hJ, fjok, q, 1); aj2 = ld(hJ, fjok, q, 2); aj3 = ld(hJ, fjok, q, 3); }
  };
  auto stash = [&](const uint4& x0, const uint4& x1, const uint4& x2, const uint4& x3, const uint4& y0,
                   const uint4& y1, const uint4& y2, const uint4& y3) {
    *reinterpret_cast<uint4*>(sI + lr * GP + lc) = x0;
    *reinterpret_cast<uint4*>(sI + (lr + 32) * GP + lc) = x1;
    *reinterpret_cast<uint4*>(sI + (lr + 64) * GP + lc) = x2;
    *reinterpret_cast<uint4*>(sI + (lr + 96) * GP + lc) = x3;
    if (!same) {
      *reinterpret_cast<uint4*>(sJ + lr * GP + lc) = y0;
      *reinterpret_cast<uint4*>(sJ + (lr + 32) * GP + lc) = y1;
      *reinterpret_cast<uint4*>(sJ + (lr + 64) * GP + lc) = y2;
      *reinterpret_cast<uint4*>(sJ + (lr + 96) * GP + lc) = y3;
    }
  };
  floatx16 acc = carried_acc(sin, g, s, 64 * I + 32 * wm, 64 * J + 32 * wn, lane, alpha);
  const uint16_t* sJr = same ? sI : sJ;
  const int j16 = lane & 15;
  const int frow = 8 * (lane >> 5) + (j16 >> 2);                  // + k0
  const int fcolA = 32 * wm + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
  const int fcolB = 32 * wn + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
  auto compute = [&]() {
    for (int k0 = 0; k0 < R; k0 += 16) {
      const bf16x8 a = tr_frag(sI, k0 + frow, fcolA, GP);
      const bf16x8 b = tr_frag(sJr, k0 + frow, fcolB, GP);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
  };
  if (nq > 0) fetch_a(0);
  int q = 0;
  for (int j = 0; j <= g.nblk; ++j) {
    if (j == g.nblk) {
      write_carry(sout, g, s, 64 * I + 32 * wm, 64 * J + 32 * wn, lane, acc, alpha);
      break;
    }
    float* Mj = ws + (static_cast<int64_t>(s) * g.nblk + j) * mstride;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 64 * I + 32 * wm + crow(r, lane), col = 64 * J + 32 * wn + (lane & 31);
      // streaming stores: the 600 MB of prefix tiles would otherwise push the
      // rows of h that the other tiles of the sequence still read out of L2
      __builtin_nontemporal_store((row == col ? 1.f : 0.f) + alpha * acc[r],
                                  Mj + static_cast<int64_t>(row) * g.ldm + col);
    }
    if (j == g.nblk - 1 && !sout) break;
    for (int sq = 0; sq < spb; ++sq, ++q) {
      lds_barrier();
      stash(ai0, ai1, ai2, ai3, aj0, aj1, aj2, aj3);
      lds_barrier();
      fetch_a(q + 1);
      compute();
    }
  }
}

// ------------------------------------------------------------------ diagonal tile


// Factor the 64x64 tile D (lower triangle; LDS, row stride ldd) with one wave
// of a larger workgroup: the logs of its pivots that fall in the S part go to
// dR, the inverse of the factor to Li (LDS, row stride lip).  2x2 blocks of 32, lane i owns row i:
//   1. eliminate columns 0..31 over all 64 rows  -> L11 (lanes 0..31), L21 (lanes 32..63)
//   2. D22 - L21 L21^T, eliminate columns 32..63  -> L22 (lanes 32..63)
//   3. columns of L11^-1 (lanes 0..31) and L22^-1 (lanes 32..63) by forward
//      substitution that pushes each solved entry into the later ones
//   4. Y = -L22^-1 (L21 L11^-1) as two products on fp32 MFMA:
//      Linv = [[L11^-1, 0], [Y, L22^-1]]
// (step 2's product L21 L21^T also runs on fp32 MFMA)
// Each elimination step broadcasts the pivot with one readlane and the scaled
// column through LDS; lanes above the diagonal also run the updates, on
// entries of the upper triangle that are never read.  Reciprocal square roots
// replace divisions; LDS rows are 16-byte aligned and read 4 floats at a time.
// sW is LDS scratch of kFactorLds floats (16-byte aligned).
constexpr int kF = 36;  // row stride of the 32-wide LDS blocks
constexpr int kFactorLds = 64 + 64 + 64 * kF + 2 * 32 * kF;

__device__ __forceinline__ void ld4(const float* p, float* dst) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
}

// LDS ordering among the lanes of the one wave running factor64 (no barrier:
// the other waves of the workgroup do not take part)
__device__ __forceinline__ void wave_lds_sync() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup"); }

__device__ __forceinline__ void factor64(const float* __restrict__ D, int ldd, float* __restrict__ sW,
                                         float* __restrict__ Li, int lip, float* __restrict__ dR_blk,
                                         int rr0, int cj, int32_t* __restrict__ status) {
  float* col = sW;                 // [64]    column broadcast
  float* rinv = sW + 64;           // [64]    reciprocals of the diagonal of L
  float* sL = sW + 128;            // [64][kF] rows of L11 (0..31) and L21 (32..63)
  float* sT11 = sL + 64 * kF;      // [32][kF] L11^T, later L11^-1 (row-major)
  float* sT22 = sT11 + 32 * kF;    // [32][kF] L22^T, later L22^-1 (row-major)
  const int i = threadIdx.x & 63, ih = i & 31;
  const bool hi = i >= 32;
  float piv = 1.f, rd = 1.f;
  bool bad = false;
  float a[32], cv[32];
#pragma unroll
  for (int q = 0; q < 32; q += 4) ld4(D + i * ldd + q, a + q);
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) {
    const float pv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[jj]), jj));
    bad |= !(pv > 0.f);
    const float r = __builtin_amdgcn_rsqf(pv);
    const float l = pv * r;
    if (i == jj) { piv = l; rd = r; }
    a[jj] = i == jj ? l : a[jj] * r;
    col[i] = a[jj];
#pragma unroll
    for (int v = (jj + 1) / 4; v < 8; ++v) ld4(col + 4 * v, cv + 4 * v);
#pragma unroll
    for (int kk = jj + 1; kk < 32; ++kk) a[kk] = fmaf(-a[jj], cv[kk], a[kk]);
  }
#pragma unroll
  for (int q = 0; q < 32; q += 4)
    *reinterpret_cast<float4*>(sL + i * kF + q) =
        make_float4((hi || q <= i) ? a[q] : 0.f, (hi || q + 1 <= i) ? a[q + 1] : 0.f,
                    (hi || q + 2 <= i) ? a[q + 2] : 0.f, (hi || q + 3 <= i) ? a[q + 3] : 0.f);
  if (!hi) {
#pragma unroll
    for (int q = 0; q < 32; ++q) sT11[q * kF + i] = q <= i ? a[q] : 0.f;
  }
  wave_lds_sync();
  float b[32];
#pragma unroll
  for (int q = 0; q < 32; q += 4) ld4(D + i * ldd + 32 + q, b + q);
  {
    // L21 L21^T on fp32 MFMA (32x32x2: in step st lane l supplies column
    // 2 st + l / 32 of row l % 32 as both operands), rows back through sT22
    floatx16 c = zero16();
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const float v = sL[(32 + ih) * kF + 2 * st + (i >> 5)];
      c = mfma32(v, v, c);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sT22[crow(r, i) * kF + ih] = c[r];
    wave_lds_sync();
    if (hi) {
      float cr[32];
#pragma unroll
      for (int q = 0; q < 32; q += 4) ld4(sT22 + ih * kF + q, cr + q);
#pragma unroll
      for (int q = 0; q < 32; ++q) b[q] -= cr[q];
    }
    wave_lds_sync();
  }
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) {
    const float pv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b[jj]), 32 + jj));
    bad |= !(pv > 0.f);
    const float r = __builtin_amdgcn_rsqf(pv);
    const float l = pv * r;
    if (ih == jj && hi) { piv = l; rd = r; }
    b[jj] = ih == jj ? l : b[jj] * r;
    col[i] = b[jj];
#pragma unroll
    for (int v = (jj + 1) / 4; v < 8; ++v) ld4(col + 32 + 4 * v, cv + 4 * v);
#pragma unroll
    for (int kk = jj + 1; kk < 32; ++kk) b[kk] = fmaf(-b[jj], cv[kk], b[kk]);
  }
  if (bad && status && i == 0) atomicOr(status, BLLM_S_NONFINITE);
  if (hi) {
#pragma unroll
    for (int q = 0; q < 32; ++q) sT22[q * kF + ih] = q <= ih ? b[q] : 0.f;
  }
  rinv[i] = rd;
  wave_lds_sync();
  // 3. lane m < 32: column m of L11^-1; lane 32+m: column m of L22^-1.
  // sT holds L^T, so column p of L is the contiguous row p of sT.
  float x[32];
  {
    const float* Tm = hi ? sT22 : sT11;
    float ri[32];
#pragma unroll
    for (int p = 0; p < 32; p += 4) ld4(rinv + (hi ? 32 : 0) + p, ri + p);
#pragma unroll
    for (int r = 0; r < 32; ++r) x[r] = r == ih ? 1.f : 0.f;
#pragma unroll
    for (int p = 0; p < 32; ++p) {
      x[p] *= ri[p];
#pragma unroll
      for (int v = (p + 1) / 4; v < 8; ++v) ld4(Tm + p * kF + 4 * v, cv + 4 * v);
#pragma unroll
      for (int r = p + 1; r < 32; ++r) x[r] = fmaf(-cv[r], x[p], x[r]);
    }
  }
  wave_lds_sync();
  {
    // inverses to LDS (row-major, over the consumed transposes) and to Li
    float* Tw = hi ? sT22 : sT11;
#pragma unroll
    for (int r = 0; r < 32; ++r) Tw[r * kF + ih] = x[r];
    if (!hi) {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        Li[r * lip + i] = x[r];
        Li[r * lip + 32 + i] = 0.f;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 32; ++r) Li[(32 + r) * lip + 32 + ih] = x[r];
    }
  }
  wave_lds_sync();
  {
    // 4. Z = L21 L11^-1 and Y = -L22^-1 Z on fp32 MFMA; Z goes row-major over
    // the rows of L11 in sL (no longer read), Y to the lower left block of Li
    floatx16 z = zero16();
#pragma unroll
    for (int st = 0; st < 16; ++st)
      z = mfma32(sL[(32 + ih) * kF + 2 * st + (i >> 5)], sT11[(2 * st + (i >> 5)) * kF + ih], z);
#pragma unroll
    for (int r = 0; r < 16; ++r) sL[crow(r, i) * kF + ih] = z[r];
    wave_lds_sync();
    floatx16 y = zero16();
#pragma unroll
    for (int st = 0; st < 16; ++st)
      y = mfma32(sT22[ih * kF + 2 * st + (i >> 5)], sL[(2 * st + (i >> 5)) * kF + ih], y);
#pragma unroll
    for (int r = 0; r < 16; ++r) Li[(32 + crow(r, i)) * lip + ih] = -y[r];
  }
  if (dR_blk != nullptr) {
    const int rr = rr0 + i;  // row of the block (S part)
    if (rr >= 0 && rr < cj) dR_blk[rr] = __logf(piv);  // hardware log2 scaled by ln 2
  }
}

// ------------------------------------------------------------------ factorization
// Left-looking by 64-column panels, two launches per panel over all block
// matrices at once:
//   cr_diag(k)   one wave per matrix factors the diagonal tile D_k (the Gram
//                prefix for k = 0, else written by cr_panel(k-1)), stores
//                Linv_k and, in the S part, the logs of the pivots
//   cr_panel(k)  workgroups of each matrix build every tile below the diagonal
//                of panel k, in passes of kPassTiles tiles (pp consecutive
//                passes per workgroup; the passes are independent):
//                  ACC_i = orig(i, k) -/+ sum_{cols < 64k} L[i, :] L[k, :]^T
//                  L[i, k] = ACC_i Linv_k^T                            (TRSM)
//                from row strips of L staged through LDS kChunk columns at a
//                time (the panel's rows once per pass, every other strip row
//                once), and the next diagonal tile
//                  D_{k+1} = orig -/+ sum_{cols <= 64k+63} L[k+1, :] L[k+1, :]^T
// Waves hold ACC_i^T (panel columns x tile rows), so the TRSM is
// Linv_k * ACC_i^T with the accumulator registers as the MFMA B operand: with
// the k index of MFMA step st taken as crow(st, lane), register st of a C/D
// tile is exactly the B element that lane supplies.
constexpr int kChunk = 16;                      // columns per staged strip chunk
constexpr int kWaitVmcnt0 = 0x0F70;             // s_waitcnt vmcnt(0), other counters unconstrained
constexpr int kSRow = 56;                       // LDS row of a strip chunk: 3 x 16 bf16 parts + 8 pad
constexpr int kPassTiles = 2;                   // tiles below the diagonal per pass
constexpr int kSlots = kPassTiles / 2;          // pass tiles per wave
constexpr int kStripRows = 64 * (kPassTiles + 1);
constexpr int kXP = 68;                         // LDS row pitch of 64x64 tiles
// one strip stage, also large enough for the staged X_{k+1} tile
constexpr int kStripFloats = kStripRows * kSRow / 2 > 64 * kXP ? kStripRows * kSRow / 2 : 64 * kXP;
constexpr int kPanelFloats = kStripFloats + 64 * kXP;
static_assert(64 * kXP <= kStripFloats, "X staging must fit in the strip buffers");
static_assert(kPassTiles == 2, "the strip loader below issues kPassTiles + 1 = 3 loads per set");

// Strip products on bf16 MFMA: an fp32 value x is the exact sum of three
// bf16 parts, x = hi + mid + lo (hi = x with its low 16 bits cleared, mid the
// same of x - hi, lo = x - hi - mid, which has at most 8 significant bits).
// A product takes the six part products down to 2^-24 of |x y| (hi hi, hi mid,
// mid hi, hi lo, lo hi, mid mid), each exact in the fp32 accumulator, so the
// sums keep fp32 accuracy at 6 x 32 instead of 8 x 64 MFMA cycles per 16 columns.
// LDS strip row (kSRow bf16): [hi 0..15][mid 0..15][lo 0..15][pad 8].
__device__ inline void stash_split(uint16_t* dst, const float4& v) {
  const float x[4] = {v.x, v.y, v.z, v.w};
  uint32_t hw[4], mw[4], lw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h = __float_as_uint(x[e]) & 0xFFFF0000u;
    const float r = x[e] - __uint_as_float(h);
    const uint32_t m = __float_as_uint(r) & 0xFFFF0000u;
    hw[e] = h;
    mw[e] = m;
    lw[e] = __float_as_uint(r - __uint_as_float(m));
  }
  // perm(s0, s1, sel): result low half = high half of s1, result high half = high half of s0
  const uint32_t sel = 0x07060302u;
  *reinterpret_cast<uint2*>(dst) =
      make_uint2(__builtin_amdgcn_perm(hw[1], hw[0], sel), __builtin_amdgcn_perm(hw[3], hw[2], sel));
  *reinterpret_cast<uint2*>(dst + 16) =
      make_uint2(__builtin_amdgcn_perm(mw[1], mw[0], sel), __builtin_amdgcn_perm(mw[3], mw[2], sel));
  *reinterpret_cast<uint2*>(dst + 32) =
      make_uint2(__builtin_amdgcn_perm(lw[1], lw[0], sel), __builtin_amdgcn_perm(lw[3], lw[2], sel));
}

// part p of the 8 columns 8 hh .. 8 hh + 7 of staged row r (16-byte LDS read)
__device__ inline uint4 frag(const uint16_t* sb, int r, int p, int hh) {
  return *reinterpret_cast<const uint4*>(sb + r * kSRow + 16 * p + 8 * hh);
}

__device__ inline uint4 xor4(uint4 v, uint32_t m) {
  v.x ^= m; v.y ^= m; v.z ^= m; v.w ^= m;
  return v;
}

__device__ inline floatx16 mfma_bf(const uint4& a, const uint4& b, const floatx16& c) {
  bf16x8 x, y;
  __builtin_memcpy(&x, &a, 16);
  __builtin_memcpy(&y, &b, 16);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
}

// sum over 16 columns of a[m][k] b[n][k] from the parts of both operands
__device__ inline floatx16 mfma_split(const uint4* a, const uint4* b, floatx16 c) {
  c = mfma_bf(a[1], b[1], c);
  c = mfma_bf(a[0], b[2], c);
  c = mfma_bf(a[2], b[0], c);
  c = mfma_bf(a[0], b[1], c);
  c = mfma_bf(a[1], b[0], c);
  return mfma_bf(a[0], b[0], c);
}

// elements (row, col .. col+3), col % 4 == 0; a group lies wholly in one part
template <int DT>
__device__ inline float4 orig4(const void* h, const float* Mx, const CRGeom& g, int64_t hrow0, int cj,
                               float salpha, int row, int col) {
  if (col >= g.dp)
    return make_float4(row == col ? 1.f : 0.f, row == col + 1 ? 1.f : 0.f, row == col + 2 ? 1.f : 0.f,
                       row == col + 3 ? 1.f : 0.f);
  if (row < g.dp) return *reinterpret_cast<const float4*>(Mx + static_cast<int64_t>(row) * g.ldm + col);
  const int rr = row - g.dp;
  if (rr >= cj || col >= g.d) return make_float4(0.f, 0.f, 0.f, 0.f);
  const int64_t e = (hrow0 + rr) * g.d + col;
  if (DT == BLLM_F32) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(h) + e);
    return make_float4(salpha * v.x, salpha * v.y, salpha * v.z, salpha * v.w);
  }
  const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(h) + e);
  return make_float4(salpha * bf16_to_f32(static_cast<uint16_t>(v.x & 0xFFFFu)),
                     salpha * bf16_to_f32(static_cast<uint16_t>(v.x >> 16)),
                     salpha * bf16_to_f32(static_cast<uint16_t>(v.y & 0xFFFFu)),
                     salpha * bf16_to_f32(static_cast<uint16_t>(v.y >> 16)));
}

// C/D tile registers of one lane from the row segments orig(row, col0 + crow(q, lane))
template <int DT>
__device__ inline floatx16 orig_tile_t(const void* h, const float* Mx, const CRGeom& g, int64_t hrow0,
                                       int cj, float salpha, int row, int col0, int hh) {
  floatx16 a;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const float4 v = orig4<DT>(h, Mx, g, hrow0, cj, salpha, row, col0 + 8 * q4 + 4 * hh);
    a[4 * q4] = v.x; a[4 * q4 + 1] = v.y; a[4 * q4 + 2] = v.z; a[4 * q4 + 3] = v.w;
  }
  return a;
}

__global__ __launch_bounds__(64) void cr_diag(float* __restrict__ ws, float* __restrict__ linv,
                                              float* __restrict__ dR, int32_t* __restrict__ status,
                                              CRGeom g, int k) {
  __shared__ __attribute__((aligned(16))) float sW[kFactorLds];
  const int m = blockIdx.x;
  const int s = m / g.nblk, j = m % g.nblk;
  if (NB * k >= block_n(g, j)) return;
  const float* D = ws + static_cast<int64_t>(m) * g.ldm * g.ldm + static_cast<int64_t>(NB * k) * g.ldm + NB * k;
  float* dRb = NB * k >= g.dp ? dR + static_cast<int64_t>(s) * g.T + static_cast<int64_t>(j) * g.c : nullptr;
  factor64(D, g.ldm, sW, linv + static_cast<int64_t>(m) * NB * NB, NB, dRb, NB * k - g.dp,
           block_rows(g, j), status);
}

template <int DT>
__global__ __launch_bounds__(256, 3) void cr_panel(const void* __restrict__ h, float* __restrict__ ws,
                                                   const float* __restrict__ linv, CRGeom g,
                                                   float salpha, int k, int pp) {
  __shared__ __attribute__((aligned(16))) float lds[kPanelFloats];
  float* sLi = lds + kStripFloats;      // Linv_k
  float* sX = lds;                      // X_{k+1} (over the strip buffers)
  uint16_t* sst = reinterpret_cast<uint16_t*>(lds);  // staged strip chunk, split into bf16 parts
  // the workgroups of one matrix are consecutive on one XCD (block b runs on XCD b % 8)
  const int ngrp = (g.ldm / NB - k - 1 + kPassTiles * pp - 1) / (kPassTiles * pp);
  const int bq = blockIdx.x >> 3, grp = bq % ngrp;
  const int m = (bq / ngrp) * 8 + (blockIdx.x & 7);
  if (m >= g.nmat) return;
  const int s = m / g.nblk, j = m % g.nblk;
  const int npan = block_n(g, j) / NB;
  if (k + 1 >= npan) return;
  const int nt = npan - k - 1;
  const int tbeg = grp * pp * kPassTiles, tend = min(nt, tbeg + pp * kPassTiles);
  if (tbeg >= nt) return;
  const bool look = grp == 0;  // this workgroup also builds the next diagonal tile
  const int cj = block_rows(g, j);
  const int64_t hrow0 = static_cast<int64_t>(s) * g.T + static_cast<int64_t>(j) * g.c;
  float* Mx = ws + static_cast<int64_t>(m) * g.ldm * g.ldm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wp = w >> 1, wn = w & 1;  // pass tiles u = wp + 2 sl; tile-row half wn
  const int dm = w >> 1, dn = w & 1;  // block of the lookahead tile
  const bool panelS = NB * k >= g.dp;
  const bool rowS1 = NB * (k + 1) >= g.dp;
  const int nch = NB * k / kChunk;
  {
    const float* Li = linv + static_cast<int64_t>(m) * NB * NB;
    for (int e = tid; e < NB * NB / 4; e += 256) {
      const int r = e >> 4, cc = (e & 15) * 4;
      *reinterpret_cast<float4*>(sLi + r * kXP + cc) = *reinterpret_cast<const float4*>(Li + r * NB + cc);
    }
  }
  // lookahead tile, symmetric: read orig transposed for row-contiguous loads
  floatx16 accD = zero16();
  if (look)
    accD = orig_tile_t<DT>(h, Mx, g, hrow0, cj, salpha, NB * (k + 1) + 32 * dn + l32, NB * (k + 1) + 32 * dm, hh);
  for (int t0 = tbeg; t0 < tend; t0 += kPassTiles) {
    const int npt = min(kPassTiles, nt - t0);
    const bool first = t0 == 0;
    floatx16 acc[kSlots][2];  // [slot][panel-column half]
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int u = wp + 2 * sl;
      const int row = NB * (k + 1 + t0 + u) + 32 * wn + l32;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        acc[sl][mb] = u < npt ? orig_tile_t<DT>(h, Mx, g, hrow0, cj, salpha, row, NB * k + 32 * mb, hh)
                              : zero16();
    }
    // strip rows: the panel's 64 rows, then the pass tiles' rows.  Two sets of
    // named prefetch registers: chunk ch + 2 is loaded while chunk ch is
    // staged and multiplied.  Rows past the pass load a valid panel row
    // instead and chunks past the end load the panel's own columns (inside
    // the row, never staged), so the loads are unconditional and the wait
    // counts static.
    const int nrows = NB * (npt + 1);
    const int lr = tid >> 2, lc = (tid & 3) * 4;
    int go[3];
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int r = lr + 64 * it;
      const int grow = r < NB ? NB * k + r : (r < nrows ? NB * (k + 1 + t0) + (r - NB) : NB * k + (r & 63));
      go[it] = grow * g.ldm + lc;
    }
    float4 qa0, qa1, qa2, qb0, qb1, qb2;
    auto ldq = [&](int it, int co) { return *reinterpret_cast<const float4*>(Mx + go[it] + co); };
    auto fetch_a = [&](int ch) {
      const int co = ch * kChunk;
      qa0 = ldq(0, co); qa1 = ldq(1, co); qa2 = ldq(2, co);
    };
    auto fetch_b = [&](int ch) {
      const int co = ch * kChunk;
      qb0 = ldq(0, co); qb1 = ldq(1, co); qb2 = ldq(2, co);
    };
    auto stash = [&](uint16_t* sb, const float4& v0, const float4& v1, const float4& v2) {
      stash_split(sb + lr * kSRow + lc, v0);
      stash_split(sb + (lr + 64) * kSRow + lc, v1);
      stash_split(sb + (lr + 128) * kSRow + lc, v2);
    };
    auto compute = [&](const uint16_t* sb, int ch) {
      const bool chA = ch * kChunk < g.dp;
      const uint32_t sg = (panelS && chA) ? 0u : 0x80008000u;  // sign flip of the panel rows
      uint4 a0[3], a1[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        a0[p] = xor4(frag(sb, l32, p, hh), sg);
        a1[p] = xor4(frag(sb, 32 + l32, p, hh), sg);
      }
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl) {
        const int u = wp + 2 * sl;
        if (u < npt) {
          uint4 b[3];
#pragma unroll
          for (int p = 0; p < 3; ++p) b[p] = frag(sb, NB + NB * u + 32 * wn + l32, p, hh);
          acc[sl][0] = mfma_split(a0, b, acc[sl][0]);
          acc[sl][1] = mfma_split(a1, b, acc[sl][1]);
        }
      }
      if (first) {
        const uint32_t sd = (rowS1 && chA) ? 0u : 0x80008000u;
        uint4 da[3], db[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          da[p] = xor4(frag(sb, NB + 32 * dm + l32, p, hh), sd);
          db[p] = frag(sb, NB + 32 * dn + l32, p, hh);
        }
        accD = mfma_split(da, db, accD);
      }
    };
    // the accumulators were loaded from memory: wait here once, so that the
    // loop's only outstanding loads are the prefetches
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (nch > 0) {
      fetch_a(0);
      fetch_b(1);
    }
    // one LDS stage, two LDS-only barriers per chunk (the prefetches stay in
    // flight across them)
    for (int ch = 0; ch < nch; ch += 2) {
      lds_barrier();
      stash(sst, qa0, qa1, qa2);
      lds_barrier();
      fetch_a(ch + 2);
      compute(sst, ch);
      if (ch + 1 < nch) {
        lds_barrier();
        stash(sst, qb0, qb1, qb2);
        lds_barrier();
        fetch_b(ch + 3);
        compute(sst, ch + 1);
      }
    }
    __syncthreads();  // strip buffers free (sX lives there); sLi staged
    // TRSM: X_u^T = Linv_k * ACC_u^T, written as rows of L
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int u = wp + 2 * sl;
      if (u < npt) {
        floatx16 x0 = zero16(), x1 = zero16();
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float l00[4], l10[4], l11[4];
          const int kc = 8 * q4 + 4 * hh;  // crow(4*q4 + e, lane) = kc + e
          ld4(sLi + l32 * kXP + kc, l00);
          ld4(sLi + (32 + l32) * kXP + kc, l10);
          ld4(sLi + (32 + l32) * kXP + 32 + kc, l11);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int st = 4 * q4 + e;
            x0 = mfma32(l00[e], acc[sl][0][st], x0);
            x1 = mfma32(l10[e], acc[sl][0][st], x1);
            x1 = mfma32(l11[e], acc[sl][1][st], x1);
          }
        }
        const int row = NB * (k + 1 + t0 + u) + 32 * wn + l32;
        float* Lr = Mx + static_cast<int64_t>(row) * g.ldm + NB * k;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int kc = 8 * q4 + 4 * hh;
          *reinterpret_cast<float4*>(Lr + kc) =
              make_float4(x0[4 * q4], x0[4 * q4 + 1], x0[4 * q4 + 2], x0[4 * q4 + 3]);
          *reinterpret_cast<float4*>(Lr + 32 + kc) =
              make_float4(x1[4 * q4], x1[4 * q4 + 1], x1[4 * q4 + 2], x1[4 * q4 + 3]);
        }
        if (first && u == 0) {
          float* xr = sX + (32 * wn + l32) * kXP;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int kc = 8 * q4 + 4 * hh;
            *reinterpret_cast<float4*>(xr + kc) =
                make_float4(x0[4 * q4], x0[4 * q4 + 1], x0[4 * q4 + 2], x0[4 * q4 + 3]);
            *reinterpret_cast<float4*>(xr + 32 + kc) =
                make_float4(x1[4 * q4], x1[4 * q4 + 1], x1[4 * q4 + 2], x1[4 * q4 + 3]);
          }
        }
      }
    }
    if (first) {
      // D_{k+1} -/+= X_{k+1} X_{k+1}^T over the panel's columns
      __syncthreads();
      const float sd = (rowS1 && !panelS) ? 1.f : -1.f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float da[16], db[16];
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
          ld4(sX + (32 * dm + l32) * kXP + 32 * half + 16 * hh + e, da + e);
          ld4(sX + (32 * dn + l32) * kXP + 32 * half + 16 * hh + e, db + e);
        }
#pragma unroll
        for (int st = 0; st < 16; ++st) accD = mfma32(sd * da[st], db[st], accD);
      }
    }
    __syncthreads();  // sX and the strip buffers are reused next
  }
  if (!look) return;
  // D_{k+1} over the diagonal tile (k+1, k+1), whose original is consumed
  float* Dt = Mx + static_cast<int64_t>(NB * (k + 1) + 32 * dm) * g.ldm + NB * (k + 1) + 32 * dn;
#pragma unroll
  for (int q = 0; q < 16; ++q) Dt[static_cast<int64_t>(crow(q, lane)) * g.ldm + l32] = accD[q];
}

CRGeom cr_geometry(int64_t nseq, int64_t T, int64_t d) {
  CRGeom g;
  g.T = static_cast<int>(T);
  g.d = static_cast<int>(d);
  g.dp = static_cast<int>((d + NB - 1) / NB * NB);
  // c near d/2 minimises the factorization flops per row, (d' + c)^3 / (3c)
  int c = (g.dp / 2 + NB - 1) / NB * NB;
  c = c < NB ? NB : (c > 256 ? 256 : c);
  g.c = c;
  g.nblk = static_cast<int>((T + c - 1) / c);
  g.ldm = g.dp + c;
  g.nmat = static_cast<int>(nseq) * g.nblk;
  g.nseq = static_cast<int>(nseq);
  return g;
}

size_t cr_ws_bytes(const CRGeom& g) {
  return static_cast<size_t>(g.nmat) * (static_cast<size_t>(g.ldm) * g.ldm + NB * NB) * 4 + 256;
}

// Passes of one panel launch per workgroup: one (a workgroup per pass, the
// passes of a matrix consecutive on one XCD so that they share the panel
// rows in its L2) unless the launch would exceed kPanelGroups workgroups.
#ifndef BLLM_CR_PANEL_GROUPS
#define BLLM_CR_PANEL_GROUPS (1 << 20)
#endif
constexpr int kPanelGroups = BLLM_CR_PANEL_GROUPS;
int passes_per_group(int nmat, int npass) {
  const int ngrp = std::max(1, std::min(npass, kPanelGroups / std::max(nmat, 1)));
  return (npass + ngrp - 1) / ngrp;
}

// The launches of one factorization as numbered steps: 0 the Gram prefix,
// then 2k + 1 the diagonal factor of panel k and 2k + 2 panel k.
struct CRCall {
  const void* h;
  CRGeom g;
  double alpha;
  float *dR, *ws, *linv, *sout;
  const float* sin;
  int32_t* status;
  hipStream_t st;
};

inline int cr_steps(const CRGeom& g) { return 2 * (g.ldm / NB); }  // gram + 12 diag + 11 panel at ldm 768

template <int DT>
void cr_step(const CRCall& c, int i) {
  const CRGeom& g = c.g;
  if (i == 0) {
    const int nt = g.dp / NB;
    const unsigned ggrid = static_cast<unsigned>((g.nseq + 7) / 8 * 8 * (nt * (nt + 1) / 2));
    if (DT == BLLM_BF16)
      hipLaunchKernelGGL(cr_gram_prefix_bf16, dim3(ggrid), dim3(256), 0, c.st, static_cast<const uint16_t*>(c.h),
                         c.ws, g, static_cast<float>(c.alpha), c.sin, c.sout);
    else
      hipLaunchKernelGGL(cr_gram_prefix<DT>, dim3(ggrid), dim3(256), 0, c.st, c.h, c.ws, g,
                         static_cast<float>(c.alpha), c.sin, c.sout);
    return;
  }
  const int k = (i - 1) / 2, npan = g.ldm / NB;
  if (i % 2 == 1) {
    hipLaunchKernelGGL(cr_diag, dim3(g.nmat), dim3(64), 0, c.st, c.ws, c.linv, c.dR, c.status, g, k);
  } else if (k + 1 < npan) {
    const int npass = (npan - k - 1 + kPassTiles - 1) / kPassTiles;
    const int pp = passes_per_group(g.nmat, npass);
    const int ngrp = (npass + pp - 1) / pp;
    hipLaunchKernelGGL(cr_panel<DT>, dim3((g.nmat + 7) / 8 * 8 * ngrp), dim3(256), 0, c.st, c.h, c.ws, c.linv, g,
                       static_cast<float>(std::sqrt(c.alpha)), k, pp);
  }
}

// The second stream of a split batch: one per device, created on first use
// and kept until the process ends, with the two events of the fork and join.
constexpr int kSplitMatrices = 512;
constexpr int kMaxDevices = 64;

struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool tried = false;
};

std::mutex g_side_mu;  // guards g_side and orders the fork / launches / join of one call
SideStream g_side[kMaxDevices];

// the side stream of the device that runs st (caller holds g_side_mu); nullptr
// if it could not be made, and then the batch runs on st alone
SideStream* side_stream(hipStream_t st) {
  hipDevice_t dev = 0;
  if (hipStreamGetDevice(st, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  SideStream& x = g_side[dev];
  if (!x.tried) {
    x.tried = true;
    int cur = 0;
    bool ok = hipGetDevice(&cur) == hipSuccess && hipSetDevice(dev) == hipSuccess;
    ok = ok && hipStreamCreateWithFlags(&x.st, hipStreamNonBlocking) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&x.fork, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&x.join, hipEventDisableTiming) == hipSuccess;
    if (hipSetDevice(cur) != hipSuccess) ok = false;
    if (!ok) {
      x.st = nullptr;
      (void)hipGetLastError();  // clear the failure just met (the call then runs on st alone)
    }
  }
  return x.st ? &x : nullptr;
}

}  // namespace
}  // namespace bllm

using namespace bllm;

extern "C" size_t bllm_coding_rate_workspace(int64_t nseq, int64_t T, int64_t d) {
  if (nseq < 1 || T < 1 || d < 1) return 0;
  return cr_ws_bytes(cr_geometry(nseq, T, d));
}

static int coding_rate_entry(const void* h, int dtype, int64_t nseq, int64_t T, int64_t d, double eps2,
                             const float* state_in, float* state_out, float* dR_out, int32_t* status,
                             void* ws, size_t ws_bytes, void* stream) {
  if (!h || !dR_out || nseq < 1 || T < 1 || d < 1 || !(eps2 > 0.0)) return BLLM_E_INVAL;
  if (!valid_dtype(dtype)) return BLLM_E_NOTSUP;
  if (d > 640 || nseq > 65535 || T > (int64_t(1) << 24)) return BLLM_E_NOTSUP;
  if ((d * elem_size(dtype)) % 16 != 0 || !aligned16(h)) return BLLM_E_NOTSUP;
  const CRGeom g = cr_geometry(nseq, T, d);
  if (static_cast<int64_t>(g.nmat) * g.nblk > (int64_t(1) << 31)) return BLLM_E_NOTSUP;
  if (!ws || ws_bytes < cr_ws_bytes(g) || !aligned16(ws)) return BLLM_E_WS;
  const double alpha = static_cast<double>(d) / eps2;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* wsf = static_cast<float*>(ws);
  float* linv = wsf + static_cast<int64_t>(g.nmat) * g.ldm * g.ldm;
  const int64_t es = elem_size(dtype);
  // sequences [s0, s0 + ns) on stream sx: their matrices, inverse slots, rows
  // of h, dR and carried state are contiguous slices of the batch's
  auto part = [&](int64_t s0, int64_t ns, hipStream_t sx) {
    CRCall c;
    c.g = cr_geometry(ns, T, d);
    c.h = static_cast<const char*>(h) + s0 * T * d * es;
    c.alpha = alpha;
    c.dR = dR_out + s0 * T;
    c.ws = wsf + s0 * g.nblk * static_cast<int64_t>(g.ldm) * g.ldm;
    c.linv = linv + s0 * g.nblk * static_cast<int64_t>(NB) * NB;
    c.sin = state_in ? state_in + s0 * d * d : nullptr;
    c.sout = state_out ? state_out + s0 * d * d : nullptr;
    c.status = status;
    c.st = sx;
    return c;
  };
  auto step = [&](const CRCall& c, int i) {
    if (dtype == BLLM_F32)
      cr_step<BLLM_F32>(c, i);
    else
      cr_step<BLLM_BF16>(c, i);
  };
  if (g.nmat < kSplitMatrices || nseq < 2) {
    const CRCall c = part(0, nseq, st);
    for (int i = 0; i < cr_steps(g); ++i) step(c, i);
    return launch_status();
  }
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* side = side_stream(st);
  if (!side) {
    const CRCall c = part(0, nseq, st);
    for (int i = 0; i < cr_steps(g); ++i) step(c, i);
    return launch_status();
  }
  const int64_t half = (nseq + 1) / 2;
  if (hipEventRecord(side->fork, st) != hipSuccess || hipStreamWaitEvent(side->st, side->fork, 0) != hipSuccess)
    return BLLM_E_HIP;
  // the halves' launches are queued alternately, so both start at once
  const CRCall a = part(0, half, st), b = part(half, nseq - half, side->st);
  for (int i = 0; i < cr_steps(g); ++i) {
    step(a, i);
    step(b, i);
  }
  if (hipEventRecord(side->join, side->st) != hipSuccess || hipStreamWaitEvent(st, side->join, 0) != hipSuccess)
    return BLLM_E_HIP;
  return launch_status();
}

extern "C" int bllm_coding_rate(const void* h, int dtype, int64_t nseq, int64_t T, int64_t d,
                                double eps2, float* dR_out, int32_t* status, void* ws,
                                size_t ws_bytes, void* stream) {
  return coding_rate_entry(h, dtype, nseq, T, d, eps2, nullptr, nullptr, dR_out, status, ws, ws_bytes, stream);
}

extern "C" int bllm_coding_rate_stream(const void* h, int dtype, int64_t nseq, int64_t W, int64_t d,
                                       double eps2, const float* state_in, float* state_out, float* dR_out,
                                       int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  return coding_rate_entry(h, dtype, nseq, W, d, eps2, state_in, state_out, dR_out, status, ws, ws_bytes, stream);
}
