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

#include <algorithm>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 load_f4(const float *p) { return *reinterpret_cast<const f4 *>(p); }
// Block summaries streamed once per call: non-temporal loads keep them from
// displacing reusable lines in the caches (measured 10 % faster on a 67 MB
// decode stream).
__device__ __forceinline__ f4 load_f4_stream(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
}

// Sum over the 64 lanes by an XOR butterfly (strides 32, 16, ..., 1): every
// lane adds the same two values in the same order at each level, so all lanes
// end with the bitwise-same sum.  The exchanges are lane swaps and DPP moves,
// not LDS permutes.
__device__ __forceinline__ float butterfly_sum(float v) {
  v += __uint_as_float(lane_xor<32>(__float_as_uint(v)));
  v += __uint_as_float(lane_xor<16>(__float_as_uint(v)));
  v += __uint_as_float(lane_xor<8>(__float_as_uint(v)));
  v += __uint_as_float(lane_xor<4>(__float_as_uint(v)));
  v += __uint_as_float(lane_xor<2>(__float_as_uint(v)));
  v += __uint_as_float(lane_xor<1>(__float_as_uint(v)));
  return v;
}

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
      kf[u][c] = (r < A && e < K) ? load_f4_stream(kblk + r * K + e) : f4{0.f, 0.f, 0.f, 0.f};
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
      p[u][n] = butterfly_sum(acc);
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
// Decode scorer with the first step of the whole-GPU top-k fused in.  A
// workgroup of NW waves scores one group of 64 consecutive blocks (wave w:
// blocks (64/NW) w .. (64/NW)(w+1) - 1, U at a time, with exactly the
// arithmetic of scores_gemv_kernel), stores the scores, and then waves
// publish each query's M best rank words of the group -- what the top-k's
// first kernel would compute from the stored scores, without reading them
// back.
// ---------------------------------------------------------------------------
// Eight waves per SIMD when the registers allow (at most 64 VGPRs): with
// 16-wave workgroups one per CU would leave the CU idle through each
// workgroup's barrier and sort.  The widest rows (NC = 16: a query and a
// summary row of 4096 floats, 128 VGPRs of operands) take 8-wave workgroups
// at two waves per SIMD, so nothing spills.
template <int NQ, int NC, int U, int NW>
constexpr int gemv_tops_min_waves() {
  return (NQ + U) * NC <= 10 ? 8 : NC >= 16 ? 2 : 4;
}

template <int NQ, int NC, int U, int NW>
__global__ __launch_bounds__(64 * NW, (gemv_tops_min_waves<NQ, NC, U, NW>())) void scores_gemv_tops_kernel(const float *__restrict__ q,
                                                                const float *__restrict__ kblk,
                                                                int nq, int K, int A,
                                                                float *__restrict__ scores,
                                                                uint64_t *__restrict__ tops,
                                                                int ngroups, int M) {
  __shared__ float sc[NQ][64 + NW];  // the group's scores, then the merged tail's
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t g = blockIdx.x;
  // The last workgroup also takes the final group when the launch leaves it
  // out (at most NW rows: one per wave).
  const bool tail = blockIdx.x == gridDim.x - 1 && int(gridDim.x) < ngroups;

  f4 qf[NQ][NC];
#pragma unroll
  for (int n = 0; n < NQ; ++n)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = 4 * (c * 64 + lane);
      qf[n][c] = (n < nq && e < K) ? load_f4(q + int64_t(n) * K + e) : f4{0.f, 0.f, 0.f, 0.f};
    }

  constexpr int RPW = 64 / NW;  // rows per wave
#pragma unroll
  for (int it = 0; it < RPW / U; ++it) {
    const int64_t row0 = g * 64 + wave * RPW + it * U;
    f4 kf[U][NC];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int e = 4 * (c * 64 + lane);
        const int64_t r = row0 + u;
        kf[u][c] = (r < A && e < K) ? load_f4_stream(kblk + r * K + e) : f4{0.f, 0.f, 0.f, 0.f};
      }
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
        acc = butterfly_sum(acc);
        const int64_t r = row0 + u;
        if (lane == u * NQ + n && r < A && n < nq) scores[int64_t(n) * A + r] = acc;
        if (lane == 0) sc[n][wave * RPW + it * U + u] = acc;
      }
  }
  if (tail) {
    const int64_t r = (g + 1) * 64 + wave;
    if (r < A) {  // wave-uniform
      f4 kf[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int e = 4 * (c * 64 + lane);
        kf[c] = e < K ? load_f4_stream(kblk + r * K + e) : f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          acc = __builtin_fmaf(qf[n][c].x, kf[c].x, acc);
          acc = __builtin_fmaf(qf[n][c].y, kf[c].y, acc);
          acc = __builtin_fmaf(qf[n][c].z, kf[c].z, acc);
          acc = __builtin_fmaf(qf[n][c].w, kf[c].w, acc);
        }
        acc = butterfly_sum(acc);
        if (lane == n && n < nq) scores[int64_t(n) * A + r] = acc;
        if (lane == 0) sc[n][64 + wave] = acc;
      }
    }
  }
  __syncthreads();
  // Wave j publishes query j % nq's words of the group (j < nq) or of the
  // merged tail group (nq <= j < 2 nq).
  const int npub = tail ? 2 * nq : nq;
  for (int j = wave; j < npub; j += NW) {  // wave-uniform
    const int n = j < nq ? j : j - nq;
    const int64_t gg = j < nq ? g : g + 1;
    const uint32_t id = uint32_t(gg * 64 + lane);
    const bool live = id < uint32_t(A) && (j < nq || lane < NW);
    const uint32_t key = live ? score_key(__float_as_uint(sc[n][j < nq ? lane : 64 + lane])) : 0u;
    publish_group_tops(key, id, M, tops + (int64_t(n) * ngroups + gg) * M);
  }
}

template <int NQ, int NC>
hipError_t launch_gemv_tops_nc(const float *q, const float *kblk, int nq, int K, int A,
                               float *scores, uint64_t *tops, int M, hipStream_t stream) {
  // rows per batch: the loaded summaries (U x NC float4s) and the queries
  // (NQ x NC) together stay near 16 float4s per lane
  constexpr int U = NQ * NC >= 8 ? 1 : NQ * NC >= 4 ? 2 : 4;
  const int ngroups = (A + 63) / 64;
  // waves per 64-block group: 16 (four rows each) for one or two queries;
  // 8 (eight rows each, half the registers per workgroup, so the barrier and
  // the sort of one workgroup stall fewer waves) from four queries on
  // (measured: 4 queries 29.4 -> 27.2 us per select; 1 and 2 slower), and for
  // 4096-float rows, whose operands need more than the 128 VGPRs of four
  // waves per SIMD.
  constexpr int NW = (NQ >= 4 || NC >= 16) ? 8 : 16;
  // With 16 waves per workgroup (two workgroups per CU, 512 at once), a final
  // group of at most NW blocks -- the capacity-shaped rows of 2^n + 2 blocks
  // end in one of 2 -- rides on the last full group's workgroup instead of
  // queueing as workgroup 513 behind the first 512 (measured, select per
  // call: two queries 21.2 -> 20.0 us, one query unchanged; with eight waves
  // four workgroups fit per CU and nothing queues, so nothing is merged).
  const bool merge = NW == 16 && ngroups >= 2 && A - 64 * (ngroups - 1) <= NW;
  scores_gemv_tops_kernel<NQ, NC, U, NW><<<merge ? ngroups - 1 : ngroups, 64 * NW, 0, stream>>>(
      q, kblk, nq, K, A, scores, tops, ngroups, M);
  return hipGetLastError();
}

template <int NQ>
hipError_t launch_gemv_tops_q(const float *q, const float *kblk, int nq, int K, int A,
                              float *scores, uint64_t *tops, int M, hipStream_t stream) {
  const int nc = (K + 255) / 256;
  if (nc <= 1) return launch_gemv_tops_nc<NQ, 1>(q, kblk, nq, K, A, scores, tops, M, stream);
  if (nc <= 2) return launch_gemv_tops_nc<NQ, 2>(q, kblk, nq, K, A, scores, tops, M, stream);
  if constexpr (NQ <= 4) {
    if (nc <= 4) return launch_gemv_tops_nc<NQ, 4>(q, kblk, nq, K, A, scores, tops, M, stream);
  }
  if constexpr (NQ <= 2) {
    if (nc <= 8) return launch_gemv_tops_nc<NQ, 8>(q, kblk, nq, K, A, scores, tops, M, stream);
  }
  if constexpr (NQ <= 1) {
    if (nc <= 16) return launch_gemv_tops_nc<NQ, 16>(q, kblk, nq, K, A, scores, tops, M, stream);
  }
  return hipErrorInvalidValue;  // the caller checks gemv_fits first
}

// ---------------------------------------------------------------------------
// MFMA scorer.  A workgroup (4 waves) owns a 64-query x 64-block output tile.
// Wave w accumulates the tile over the w-th quarter of K (with heads = 4 that
// is exactly head w), as 4x4 sub-tiles of v_mfma_f32_16x16x4_f32.  The four
// partial tiles are summed as (p0 + p1) + (p2 + p3) through two pairwise
// exchanges in LDS.
//
// Operand layout of v_mfma_f32_16x16x4_f32 (wave64): lane l supplies
// A[row l%16][k l/16] and B[k l/16][col l%16]; the 16x16 result sits in lane
// l as rows 4*(l/16) + r, r = 0..3, of column l%16.  Each lane loads a float4
// of 4 consecutive K elements of its row; MFMA step c of an iteration takes
// component c, so one iteration covers 16 K elements: lane group g (= l/16)
// contributes elements kk + 4g + c.  A and B use the same assignment, so the
// contraction pairs the right products; only the fp32 rounding order is fixed
// by it.
//
// Loads are raw buffer loads whose resource covers just the tile's valid rows:
// the hardware returns zeros for rows past nq or past the active blocks, and
// for K elements outside the wave's quarter the offset is pushed out of range.
// Zero operands add exact zeros, so a tile's ragged edge runs the same
// instruction stream as a full tile and every score is computed the same way
// wherever its block sits.  Iterations alternate between two register sets,
// so the loads for the next 16 K elements are in flight while the MFMAs of
// the current ones issue.
// ---------------------------------------------------------------------------
constexpr int TM = 64;       // queries per tile
constexpr int TN = 64;       // blocks per tile
constexpr uint32_t kOutOfRange = 0x40000000u;  // byte offset past any tile resource

__device__ __forceinline__ f4 mfma16x16x4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const float *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, int(bytes), 0x00020000);
}

__device__ __forceinline__ f4 buffer_f4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Epilogue of one wave of a tile (see score_tile).  W is the wave index.
template <int W>
__device__ __forceinline__ void combine_store(const f4 (&acc)[4][4], f4 *xbuf,
                                              float *__restrict__ scores, int nq, int A, int q0,
                                              int b0, int lane) {
  constexpr int keep1 = (W & 1) ? 2 : 0;  // row blocks kept after stage 1: keep1, keep1 + 1
  constexpr int send1 = 2 - keep1;
  constexpr int keep2 = (W >> 1) & 1;     // which of the two stays after stage 2
  constexpr int mi = keep1 + keep2;
  const int r16 = lane & 15;
  const int g = lane >> 4;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) xbuf[((W * 2 + m) * 4 + ni) * 64 + lane] = acc[send1 + m][ni];
  __syncthreads();
  f4 half[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      half[m][ni] = acc[keep1 + m][ni] + xbuf[(((W ^ 1) * 2 + m) * 4 + ni) * 64 + lane];
  f4 *x2 = xbuf + 4 * 2 * 4 * 64;
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) x2[(W * 4 + ni) * 64 + lane] = half[1 - keep2][ni];
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const f4 v = half[keep2][ni] + x2[((W ^ 2) * 4 + ni) * 64 + lane];
    const int col = b0 + 16 * ni + r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = q0 + 16 * mi + 4 * g + r;
      if (row < nq && col < A) scores[int64_t(row) * A + col] = v[r];
    }
  }
}

// One 64 x 64 output tile.  FULL: all 64 block rows are active.  A ragged last
// tile (FULL = false) skips the 16-block sub-tiles that hold no active block;
// the sub-tiles it does run execute the same instruction stream as in a full
// tile, so every score is bitwise the same wherever its block sits.
template <bool FULL>
__device__ __forceinline__ void score_tile(const float *__restrict__ q,
                                           const float *__restrict__ kblk, int nq, int K, int A,
                                           float *__restrict__ scores, int q0, int b0,
                                           f4 *xbuf) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int nni = FULL ? 4 : min(4, (A - b0 + 15) / 16);  // sub-tiles with an active block

  const uint32_t row_bytes = uint32_t(K) * 4u;
  const __amdgpu_buffer_rsrc_t rq = tile_rsrc(q + int64_t(q0) * K, uint32_t(min(TM, nq - q0)) * row_bytes);
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kblk + int64_t(b0) * K, uint32_t(min(TN, A - b0)) * row_bytes);

  const int KQ = ((K + 15) / 16) * 4;  // quarter of K, rounded up to a multiple of 4
  const int kbeg = wave * KQ;
  const int kend = min(K, kbeg + KQ);

  // Byte offset of this lane's float4 at iteration base kk (row part added per sub-tile).
  auto koff = [&](int kk) -> uint32_t {
    const int e = kk + 4 * g;
    return e < kend ? uint32_t(e) * 4u : kOutOfRange;
  };
  const uint32_t rowoff = uint32_t(r16) * row_bytes;
  const uint32_t sub = 16u * row_bytes;  // byte stride between 16-row sub-tiles

  f4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f4{0.f, 0.f, 0.f, 0.f};

  auto load = [&](f4 *a, f4 *b, int kk) {
    const uint32_t o = koff(kk) + rowoff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = buffer_f4(rq, o + uint32_t(i) * sub);
      if (FULL || i < nni) b[i] = buffer_f4(rk, o + uint32_t(i) * sub);
    }
  };
  auto mma = [&](const f4 *a, const f4 *b) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          if (FULL || ni < nni) acc[mi][ni] = mfma16x16x4(a[mi][c], b[ni][c], acc[mi][ni]);
  };

  // Ping-pong over 16-element steps; a step past kend loads zeros (no memory
  // access) and its MFMAs add exact zeros.
  f4 a0[4], b0v[4], a1[4], b1v[4];
  load(a0, b0v, kbeg);
  for (int kk = kbeg; kk < kend; kk += 32) {
    load(a1, b1v, kk + 16);
    mma(a0, b0v);
    load(a0, b0v, kk + 32);
    mma(a1, b1v);
  }

  // Combine the four quarter partials as (p0 + p1) + (p2 + p3) in two
  // pairwise exchanges through LDS (float4 per lane, one 1 KB row of lanes
  // per access, conflict-free); fp32 addition is commutative, so which wave
  // of a pair adds does not change a bit.
  //   stage 1, pairs (0,1) and (2,3): the even wave keeps row blocks 0-1 and
  //            sends 2-3, the odd wave the reverse -> p0+p1 / p2+p3 halves;
  //   stage 2, pairs (0,2) and (1,3): each keeps one row block -> the sum.
  // Wave w ends with row block {0, 2, 1, 3}[w] and stores it from registers.
  // The wave's role is a template argument so every register-array index is
  // a compile-time constant (a runtime index would demote acc to scratch).
  switch (wave) {
    case 0: combine_store<0>(acc, xbuf, scores, nq, A, q0, b0, lane); break;
    case 1: combine_store<1>(acc, xbuf, scores, nq, A, q0, b0, lane); break;
    case 2: combine_store<2>(acc, xbuf, scores, nq, A, q0, b0, lane); break;
    default: combine_store<3>(acc, xbuf, scores, nq, A, q0, b0, lane); break;
  }
}

// Tiles are 64 queries x 64 blocks: nqt query tiles by nct block tiles, the
// last block tile ragged when A is not a multiple of 64 (e.g. the 32,770 =
// 512 * 64 + 2 blocks of a 131K context).  Workgroup ids go round-robin over
// the 8 XCDs (XCD = blockIdx % 8), each XCD dispatching its own ids in order.
// Each XCD gets an equal share of the full tiles (query tiles fastest, so the
// query tiles of one block tile share that XCD's L2) and every eighth ragged
// tile; its ragged tiles -- the cheapest -- go first, so no XCD is left with a
// lone full tile in a last partial round.
__global__ __launch_bounds__(256, 3) void scores_mfma_kernel(const float *__restrict__ q,
                                                             const float *__restrict__ kblk,
                                                             int nq, int K, int A,
                                                             float *__restrict__ scores,
                                                             int nqt, int nct, int ntail) {
  __shared__ f4 xbuf[(4 * 2 * 4 + 4 * 4) * 64];  // 48 KB: three workgroups fit a CU
  const int x = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int tails_here = ntail > x ? (ntail - x + 7) / 8 : 0;
  if (slot < tails_here) {
    const int qt = x + 8 * slot;
    score_tile<false>(q, kblk, nq, K, A, scores, qt * TM, (nct - 1) * TN, xbuf);
    return;
  }
  const int64_t nfull = int64_t(nqt) * (nct - (ntail > 0 ? 1 : 0));
  const int64_t f = nfull * x / 8 + (slot - tails_here);
  if (f >= nfull * (x + 1) / 8) return;  // whole workgroup leaves before any barrier
  score_tile<true>(q, kblk, nq, K, A, scores, int(f % nqt) * TM, int(f / nqt) * TN, xbuf);
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

}  // namespace

// Whether the GEMV kernel keeps this (nq, K) in registers (NQ * NC <= 16).
bool gemv_fits(int nq, int K) {
  if (nq > kGemvMaxQueries) return false;
  const int nqp = nq <= 1 ? 1 : nq <= 2 ? 2 : nq <= 4 ? 4 : 8;
  const int nc = (K + 255) / 256;
  const int ncp = nc <= 1 ? 1 : nc <= 2 ? 2 : nc <= 4 ? 4 : nc <= 8 ? 8 : 16;
  return nqp * ncp <= 16;
}


hipError_t launch_gemv_tops(const float *q, const float *kblk, int nq, int K, int A,
                            float *scores, uint64_t *tops, int M, hipStream_t stream) {
  if (!gemv_fits(nq, K)) return hipErrorInvalidValue;
  if (nq <= 1) return launch_gemv_tops_q<1>(q, kblk, nq, K, A, scores, tops, M, stream);
  if (nq <= 2) return launch_gemv_tops_q<2>(q, kblk, nq, K, A, scores, tops, M, stream);
  if (nq <= 4) return launch_gemv_tops_q<4>(q, kblk, nq, K, A, scores, tops, M, stream);
  return launch_gemv_tops_q<8>(q, kblk, nq, K, A, scores, tops, M, stream);
}

hipError_t launch_block_scores_fp32(const float *q, const float *kblk, int nq, int K, int A,
                                    float *scores, hipStream_t stream) {
  if (gemv_fits(nq, K)) {
    if (nq <= 1) return launch_gemv_nc<1>(q, kblk, nq, K, A, scores, stream);
    if (nq <= 2) return launch_gemv_nc<2>(q, kblk, nq, K, A, scores, stream);
    if (nq <= 4) return launch_gemv_nc<4>(q, kblk, nq, K, A, scores, stream);
    return launch_gemv_nc<8>(q, kblk, nq, K, A, scores, stream);
  }
  const int nqt = (nq + TM - 1) / TM;
  const int nct = (A + TN - 1) / TN;
  const int ntail = (A % TN) ? nqt : 0;
  const int64_t nfull = int64_t(nqt) * (nct - (ntail ? 1 : 0));
  int64_t per = 0;  // workgroups per XCD: the largest share
  for (int x = 0; x < 8; ++x) {
    const int64_t tails = ntail > x ? (ntail - x + 7) / 8 : 0;
    per = std::max(per, tails + nfull * (x + 1) / 8 - nfull * x / 8);
  }
  scores_mfma_kernel<<<int(8 * per), 256, 0, stream>>>(q, kblk, nq, K, A, scores, nqt, nct, ntail);
  return hipGetLastError();
}

// Mode dispatch (modes of include/qsa.h).  AUTO: few queries are bandwidth-
// bound and take the fp32 dot-product kernel; larger batches take the fp16
// two-piece split MFMA tiles, whose error against FP64 is of the same order
// as the fp32 MFMA path's (prompt-128k scorer: 47.5 us against 62.5 us for
// the bf16 three-way split and 91 us for fp32 MFMA).
hipError_t launch_block_scores(const float *q, const float *kblk, int nq, int K, int A,
                               float *scores, int mode, hipStream_t stream) {
  if (mode == kScoresF16x2 || (mode == kScoresAuto && !gemv_fits(nq, K)))
    return launch_block_scores_f16x2(q, kblk, nq, K, A, scores, stream);
  if (mode == kScoresBf16x3)
    return launch_block_scores_bf16x3(q, kblk, nq, K, A, scores, stream);
  return launch_block_scores_fp32(q, kblk, nq, K, A, scores, stream);
}

}  // namespace qsa
