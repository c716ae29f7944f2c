// Block scoring kernels for gfx950 (CDNA4, wave64).
//
// score[i][b] = sum_h sum_d q[i][h][d] * kblk[b][h][d]  (page "#3108 perf(hip):
// optimize exact QSA block scoring and top-k selection on gfx12", Summary
// item 1: per-head reductions summed into one block score).  Two regimes:
//
// * few queries (decode): a GEMV.  Every byte of the active summaries is read
//   once, arithmetic intensity is ~0.5 FLOP/B, so the kernel is HBM-bound.  One
//   wave covers a 2 KB summary row per load wave-instruction pair; q sits in
//   registers.
// * many queries (prompt): a dense fp32 contraction S = Q * Kblk^T with
//   M = nq, N = active blocks, K = heads*dim, run on the fp32 matrix cores
//   (v_mfma_f32_16x16x4_f32).  With nq = 256 the intensity is ~80 FLOP/B, past
//   the fp32-MFMA ridge, so the kernel is MFMA-bound.
//
// Both keep every block's arithmetic independent of its position in a tile,
// so identical summaries give bitwise-identical scores.
#include <hip/hip_runtime.h>

#include "qsa_internal.h"

namespace qsa {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 load_f4(const float *p) { return *reinterpret_cast<const f4 *>(p); }

// ---------------------------------------------------------------------------
// GEMV scorer: NQ queries (padded), NC float4 chunks of K per lane, U rows per
// wave.  Lane l owns elements [4*(c*64 + l), +4) of every row for c < NC.
// Per lane: an fp32 FMA chain over its chunks; then a 64-lane butterfly.  The
// butterfly is symmetric, so every lane ends with the same value and every row
// gets the same operation tree.
// ---------------------------------------------------------------------------
template <int NQ, int NC, int U>
__global__ __launch_bounds__(256) void scores_gemv_kernel(const float *__restrict__ q,
                                                          const float *__restrict__ kblk,
                                                          int nq, int K, int A,
                                                          float *__restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t(blockIdx.x) * 4 + wave) * U;
  if (row0 >= A) return;  // wave-uniform; no barriers in this kernel

  f4 qf[NQ][NC];
#pragma unroll
  for (int n = 0; n < NQ; ++n)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = 4 * (c * 64 + lane);
      qf[n][c] = (n < nq && e < K) ? load_f4(q + int64_t(n) * K + e) : f4{0.f, 0.f, 0.f, 0.f};
    }

  f4 kf[U][NC];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = 4 * (c * 64 + lane);
      const int64_t r = row0 + u;
      kf[u][c] = (r < A && e < K) ? load_f4(kblk + r * K + e) : f4{0.f, 0.f, 0.f, 0.f};
    }

  float p[U][NQ];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc = __builtin_fmaf(qf[n][c].x, kf[u][c].x, acc);
        acc = __builtin_fmaf(qf[n][c].y, kf[u][c].y, acc);
        acc = __builtin_fmaf(qf[n][c].z, kf[u][c].z, acc);
        acc = __builtin_fmaf(qf[n][c].w, kf[u][c].w, acc);
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
      p[u][n] = acc;
    }

#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const int64_t r = row0 + u;
      if (lane == u * NQ + n && r < A && n < nq) scores[int64_t(n) * A + r] = p[u][n];
    }
}

// ---------------------------------------------------------------------------
// MFMA scorer.  A workgroup (4 waves) owns a 64-query x 64-block output tile.
// Wave w accumulates the tile over the w-th quarter of K (with heads = 4 that
// is exactly head w), as 4x4 sub-tiles of v_mfma_f32_16x16x4_f32.  The four
// partial tiles meet in LDS and are summed as (p0 + p1) + (p2 + p3).
//
// Operand layout of v_mfma_f32_16x16x4_f32 (wave64): lane l supplies
// A[row l%16][k l/16] and B[k l/16][col l%16]; the 16x16 result sits in lane
// l as rows 4*(l/16) + r, r = 0..3, of column l%16.  Each lane loads a float4
// of 4 consecutive K elements of its row; MFMA step c of an iteration takes
// component c, so one iteration covers 16 K elements: lane group g (= l/16)
// contributes elements kk + 4g + c.  A and B use the same assignment, so the
// contraction is exact in which products meet; only the fp32 rounding order
// is fixed by it.
// ---------------------------------------------------------------------------
constexpr int TM = 64;   // queries per tile
constexpr int TN = 64;   // blocks per tile
constexpr int PSTRIDE = 68;  // LDS row stride of a partial tile (bank spread)

__device__ __forceinline__ f4 mfma16x16x4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <bool FULL>
__device__ __forceinline__ void mfma_tile_body(const float *__restrict__ q,
                                               const float *__restrict__ kblk, int nq, int K,
                                               int A, int q0, int b0, int wave, int lane,
                                               float (*part)[TM][PSTRIDE]) {
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int KQ = ((K + 15) / 16) * 4;  // quarter of K, rounded up to a multiple of 4
  const int kbeg = wave * KQ;
  const int kend = min(K, kbeg + KQ);
  // Sub-tiles along N that hold at least one active block (all 4 when FULL).
  const int nni = FULL ? 4 : min(4, (A - b0 + 15) / 16);

  const float *qrow[4];
  const float *krow[4];
  bool qok[4], kok[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int qi = q0 + 16 * mi + r16;
    qok[mi] = qi < nq;
    qrow[mi] = q + int64_t(qok[mi] ? qi : 0) * K;
  }
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int bj = b0 + 16 * ni + r16;
    kok[ni] = FULL || bj < A;
    krow[ni] = kblk + int64_t(kok[ni] ? bj : 0) * K;
  }

  f4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f4{0.f, 0.f, 0.f, 0.f};

  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  f4 a[4], b[4], an[4], bn[4];
  auto load = [&](f4 *aa, f4 *bb, int kk) {
    const int e = kk + 4 * g;
    const bool kin = e < kend;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) aa[mi] = (kin && qok[mi]) ? load_f4(qrow[mi] + e) : zero;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      bb[ni] = (kin && kok[ni] && (FULL || ni < nni)) ? load_f4(krow[ni] + e) : zero;
  };

  if (kbeg < kend) load(a, b, kbeg);
  for (int kk = kbeg; kk < kend; kk += 16) {
    const bool more = kk + 16 < kend;
    if (more) load(an, bn, kk + 16);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          if (FULL || ni < nni) acc[mi][ni] = mfma16x16x4(a[mi][c], b[ni][c], acc[mi][ni]);
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = an[i];
        b[i] = bn[i];
      }
    }
  }

#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wave][16 * mi + 4 * g + r][16 * ni + r16] = acc[mi][ni][r];
}

// blockIdx -> tile: consecutive workgroup ids go round-robin over the 8 XCDs,
// so each XCD gets a contiguous run of tiles (query tiles fastest) and the
// query tiles that share a block tile share that XCD's L2.
__global__ __launch_bounds__(256, 2) void scores_mfma_kernel(const float *__restrict__ q,
                                                             const float *__restrict__ kblk,
                                                             int nq, int K, int A,
                                                             float *__restrict__ scores,
                                                             int nqt, int ntiles,
                                                             int tiles_per_xcd) {
  __shared__ float part[4][TM][PSTRIDE];
  const int tile = (blockIdx.x & 7) * tiles_per_xcd + (blockIdx.x >> 3);
  if (tile >= ntiles) return;  // whole workgroup leaves before any barrier
  const int q0 = (tile % nqt) * TM;
  const int b0 = (tile / nqt) * TN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  if (b0 + TN <= A)
    mfma_tile_body<true>(q, kblk, nq, K, A, q0, b0, wave, lane, part);
  else
    mfma_tile_body<false>(q, kblk, nq, K, A, q0, b0, wave, lane, part);
  __syncthreads();

#pragma unroll 4
  for (int e = threadIdx.x; e < TM * TN; e += 256) {
    const int i = e / TN, j = e % TN;
    const float s = (part[0][i][j] + part[1][i][j]) + (part[2][i][j] + part[3][i][j]);
    if (q0 + i < nq && b0 + j < A) scores[int64_t(q0 + i) * A + b0 + j] = s;
  }
}

template <int NQ, int NC>
hipError_t launch_gemv(const float *q, const float *kblk, int nq, int K, int A, float *scores,
                       hipStream_t stream) {
  constexpr int U = NC >= 8 ? 1 : NC >= 4 ? 2 : 4;  // ~8 float4 loads in flight per lane
  const int rows_per_wg = 4 * U;
  const int grid = (A + rows_per_wg - 1) / rows_per_wg;
  scores_gemv_kernel<NQ, NC, U><<<grid, 256, 0, stream>>>(q, kblk, nq, K, A, scores);
  return hipGetLastError();
}

template <int NQ>
hipError_t launch_gemv_nc(const float *q, const float *kblk, int nq, int K, int A,
                          float *scores, hipStream_t stream) {
  const int nc = (K + 255) / 256;
  if (nc <= 1) return launch_gemv<NQ, 1>(q, kblk, nq, K, A, scores, stream);
  if (nc <= 2) return launch_gemv<NQ, 2>(q, kblk, nq, K, A, scores, stream);
  if constexpr (NQ <= 4) {
    if (nc <= 4) return launch_gemv<NQ, 4>(q, kblk, nq, K, A, scores, stream);
  }
  if constexpr (NQ <= 2) {
    if (nc <= 8) return launch_gemv<NQ, 8>(q, kblk, nq, K, A, scores, stream);
  }
  if constexpr (NQ <= 1) {
    if (nc <= 16) return launch_gemv<NQ, 16>(q, kblk, nq, K, A, scores, stream);
  }
  return hipErrorInvalidValue;  // caller routes these shapes to the MFMA kernel
}

// Whether the GEMV kernel keeps this (nq, K) in registers (NQ * NC <= 16).
bool gemv_fits(int nq, int K) {
  if (nq > kGemvMaxQueries) return false;
  const int nqp = nq <= 1 ? 1 : nq <= 2 ? 2 : nq <= 4 ? 4 : 8;
  const int nc = (K + 255) / 256;
  const int ncp = nc <= 1 ? 1 : nc <= 2 ? 2 : nc <= 4 ? 4 : nc <= 8 ? 8 : 16;
  return nqp * ncp <= 16;
}

}  // namespace

hipError_t launch_block_scores(const float *q, const float *kblk, int nq, int K, int A,
                               float *scores, hipStream_t stream) {
  if (gemv_fits(nq, K)) {
    if (nq <= 1) return launch_gemv_nc<1>(q, kblk, nq, K, A, scores, stream);
    if (nq <= 2) return launch_gemv_nc<2>(q, kblk, nq, K, A, scores, stream);
    if (nq <= 4) return launch_gemv_nc<4>(q, kblk, nq, K, A, scores, stream);
    return launch_gemv_nc<8>(q, kblk, nq, K, A, scores, stream);
  }
  const int nqt = (nq + TM - 1) / TM;
  const int nct = (A + TN - 1) / TN;
  const int ntiles = nqt * nct;
  const int per_xcd = (ntiles + 7) / 8;
  scores_mfma_kernel<<<8 * per_xcd, 256, 0, stream>>>(q, kblk, nq, K, A, scores, nqt, ntiles,
                                                      per_xcd);
  return hipGetLastError();
}

}  // namespace qsa
