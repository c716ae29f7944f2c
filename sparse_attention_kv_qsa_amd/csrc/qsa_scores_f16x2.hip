// Block scoring on fp16 matrix cores with a scaled two-piece split (gfx950).
//
// The score is the fp32 dot product of page "#3108 perf(hip): optimize exact
// QSA block scoring and top-k selection on gfx12", Summary item 1, evaluated
// on matrix cores the way page "#337 hip: gfx12 (RDNA4) QSA select - WMMA
// block scorer, prompt-aware top-k dispatch", What item 2 does with bf16
// slices, but with binary16 pieces: binary16 keeps 11 significant bits
// against bf16's 8, so two pieces carry 22 bits of every operand and a
// product needs three matrix products instead of six.
//
// Pieces.  Every row (a query, or a block summary) gets a power-of-two scale
// 2^-e fixed by its own first 32 elements: with m their largest magnitude,
// m * 2^-e lies in [2^8, 2^9).  A scaled element x' = x * 2^-e (exact) is cut
// into hi = fp16(x') and lo = fp16(x' - hi), both rounded to nearest, so
// |x' - hi - lo| <= 2^-22 |x'| while x' stays in binary16's normal range; an
// element below it (more than ~2^22 under the row's first-step maximum)
// keeps an absolute error of at most 2^-25 in the scaled domain.  For a query
// piece pair (a, b) and a block pair (c, d) the product is formed as
//   a*c  +  [a*d + b*c]
// dropping b*d (below 2^-22 of the term); each piece product is exact in
// fp32.  The a*c products get their own accumulator and the two corrections
// another, added once at the end, and the tile result is scaled back by
// 2^(e_q + e_b) (exact).  The error against FP64 is therefore of the order of
// fp32 accumulation's, as for the three-way bf16 split.
//
// Range.  A scaled element of at least 65520 in magnitude (more than 2^7
// times its row's first-step maximum) would become an infinite piece.  Such
// a score -- detectable as a non-finite accumulator, since finite pieces
// cannot overflow a product or a 4096-term sum -- is computed again from the
// two rows in FP64 (a fixed sequential loop) and rounded once; non-finite
// inputs take the same route and give non-finite scores.  Both the scales
// and this fallback depend on a score's two rows only, so equal summaries
// still score bitwise-equal wherever they sit.
//
// Workgroup tile: 128 queries x 64 blocks, 4 waves; wave w owns queries
// [32w, 32w + 32) against both 32-block halves over all of K, in steps of 32
// = two 16-element halves (v_mfma_f32_32x32x16_f16; lane l supplies row l%32,
// K elements 8*(l/32) .. +7 of a half, and holds rows 8*(r/4) + 4*(l/32) +
// r%4 of column l%32 of the result in register r).  Thread t loads 8
// consecutive elements of block row t/4 per step, splits them and writes the
// two 16-byte planes to LDS where the MFMA lane that needs them reads them;
// two LDS buffers alternate, one barrier per step.  Each wave splits its own
// query slices in registers; with K a multiple of 32 its query rows arrive
// through LDS by direct buffer-to-LDS loads (8 lanes per 128-byte row
// segment).  Two accumulators per 32-block column half, hi*hi and
// corrections, each receiving every 16-element K chunk in order; the score
// is (hh + c) * 2^(e_q + e_b).  At 168 VGPRs and 50 KB of LDS, three
// workgroups share a CU (one accumulator set per K half, as in the bf16
// split scorer, would need 232 VGPRs and allow two: 53 against 47 us per
// 256 x 32,770-block call).  A ragged column runs the same tile with its
// empty column half skipped, so every score sees the same MFMA sequence.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qsa_internal.h"

namespace qsa {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int BM = 128;  // queries per tile
constexpr int BN = 64;   // blocks per tile
constexpr int BK = 32;   // K elements per step
constexpr uint32_t kOutOfRange = 0x40000000u;  // byte offset past any tile resource
constexpr int kPlane = 2 * 2 * 64;             // u4 entries per plane of one step

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const float *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, int(bytes), 0x00020000);
}

__device__ __forceinline__ f4 buffer_f4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Exponent e of a row's scale 2^-e from m, the largest magnitude of its first
// 32 elements: m * 2^-e in [2^8, 2^9).  Zero (or a non-finite m) keeps the
// row unscaled; e stays in [-126, 126] so that 2^-e is a normal float.
__device__ __forceinline__ int row_exp(float m) {
  if (!(m > 0.0f) || !(m <= 3.402823466e38f)) return 0;
  const int E = __builtin_amdgcn_frexp_expf(m);  // m = f * 2^E, f in [0.5, 1)
  return std::min(std::max(E - 9, -126), 126);
}

__device__ __forceinline__ float max_abs8(f4 a, f4 b) {
  float m = fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w)));
  return fmaxf(m, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
}

// The two binary16 planes of 8 consecutive fp32 values times the row scale
// sc, each packed as 8 halves (element 2i in the low half of word i).
struct Pieces {
  u4 hi, lo;
};

// Per pair of elements: two multiplies and one packed conversion for hi, and
// the residual x * sc - hi as one mixed-precision FMA per element (exact:
// x * sc and hi share their leading bits), then one packed conversion for lo.
__device__ __forceinline__ Pieces split8(f4 a, f4 b, float sc) {
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  Pieces p;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f2 v = {x[2 * w], x[2 * w + 1]};
    const h2 hv = __builtin_convertvector(v * sc, h2);
    const f2 r = {__builtin_fmaf(v.x, sc, -float(hv.x)), __builtin_fmaf(v.y, sc, -float(hv.y))};
    p.hi[w] = __builtin_bit_cast(uint32_t, hv);
    p.lo[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, h2));
  }
  return p;
}

__device__ __forceinline__ f16v mfma_f16(u4 a, u4 b, f16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b),
                                                c, 0, 0, 0);
}

// The range fallback: one score from its two rows, FP64 products summed in
// order, rounded once.
__device__ __forceinline__ float score_f64(const float *__restrict__ qr, const float *__restrict__ kr,
                                           int K) {
  double s = 0.0;
  for (int e = 0; e < K; ++e) s = __builtin_fma(double(qr[e]), double(kr[e]), s);
  return float(s);
}

// LDS slots of a step's block planes are [ks][column half][lane]; lane l of
// K group g = 2 ks + l/32 sits at l ^ lane_swz(g), so that neither the
// quartet writes of one block row nor the MFMA-lane reads conflict.
__device__ __forceinline__ int lane_swz(int g) { return (g << 2) ^ ((g >> 1) << 1); }

// Scale back one lane's 16 results of column half ni (tile rows qr0 + 8(r/4)
// + 4h + r%4 of the wave's query group) and mark the non-finite ones.
__device__ __forceinline__ uint32_t unscale16(f16v &v, const int *eqs, int qr0, int h, int ek,
                                              int ni) {
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int4 e4 = *reinterpret_cast<const int4 *>(eqs + qr0 + 8 * j + 4 * h);
    const int ev[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * j + i;
      bad |= uint32_t(!__builtin_isfinite(v[r])) << (16 * ni + r);
      v[r] = __builtin_amdgcn_ldexpf(v[r], ev[i] + ek);
    }
  }
  return bad;
}

// After the tile's stores: scores whose accumulator was not finite are
// computed again from their rows (bit 16 ni + r of `bad`: register r of
// column half ni).  The wait orders these stores after the tile's own.
__device__ __forceinline__ void fix_range(uint32_t bad, const float *__restrict__ q,
                                          const float *__restrict__ kblk, int nq, int K, int A,
                                          float *__restrict__ scores, int qrow0, int b0, int r32,
                                          int h) {
  if (__builtin_amdgcn_ballot_w64(bad != 0) == 0) return;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tile's stores are done
  while (bad) {
    const int bit = __builtin_ctz(bad);
    bad &= bad - 1;
    const int ni = bit >> 4, r = bit & 15;
    const int row = qrow0 + 8 * (r >> 2) + 4 * h + (r & 3);
    const int col = b0 + 32 * ni + r32;
    if (row < nq && col < A)
      scores[int64_t(row) * A + col] = score_f64(q + int64_t(row) * K, kblk + int64_t(col) * K, K);
  }
}

// One 128 x 64 tile.  FULL: all 64 block rows active; otherwise a 32-block
// half without an active block skips its MFMAs.
template <bool FULL, bool QD>
__device__ __forceinline__ void split_tile(const float *__restrict__ q,
                                           const float *__restrict__ kblk, int nq, int K, int A,
                                           float *__restrict__ scores, int q0, int b0, u4 *bl,
                                           u4 *qst, int *eqs, int *eks) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int r32 = lane & 31;
  const int h = lane >> 5;
  const int nni = FULL ? 2 : min(2, (A - b0 + 31) / 32);

  const uint32_t row_bytes = uint32_t(K) * 4u;
  const __amdgpu_buffer_rsrc_t rq = tile_rsrc(q + int64_t(q0) * K, uint32_t(min(BM, nq - q0)) * row_bytes);
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kblk + int64_t(b0) * K, uint32_t(min(BN, A - b0)) * row_bytes);

  const uint32_t qrow = uint32_t(32 * wave + r32) * row_bytes;
  const int brow = t >> 2;
  const int bkg = t & 3;
  const uint32_t boff = uint32_t(brow) * row_bytes;
  const int bslot = ((bkg >> 1) * 2 + (brow >> 5)) * 64 + (((brow & 31) + 32 * (bkg & 1)) ^ lane_swz(bkg));

  auto eoff = [&](int e) -> uint32_t { return e < K ? uint32_t(e) * 4u : kOutOfRange; };

  // acc[set][ni]: set 0 = hi*hi, set 1 = corrections.
  f16v acc[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[c][ni] = f16v{};

  f4 qa[2][2], kb[2];
  // QD: the wave's 32 query rows of a step go global -> LDS by direct loads,
  // 8 lanes per 128-byte row segment, piece p of row r at slot p ^ ((r >> 1)
  // & 7); the lanes then read their MFMA slices.
  uint32_t dq[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int p = (lane & 7) ^ ((r >> 1) & 7);
    dq[i] = uint32_t(32 * wave + (lane >> 3)) * row_bytes + uint32_t(p) * 16u;
  }
  auto dma_q = [&](int buf, int kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void *)(qst + buf * 256 + i * 64), 16, dq[i & 1],
                                               kk * 4 + 8 * i * int(row_bytes), 0, 0);
  };
  auto read_q = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int p = 4 * ks + 2 * h + half;
        qa[ks][half] = __builtin_bit_cast(f4, qst[buf * 256 + r32 * 8 + (p ^ ((r32 >> 1) & 7))]);
      }
  };
  auto load = [&](int kk) {
    if (QD) {
      if (kk < K) dma_q((kk / BK) & 1, kk);
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        qa[ks][0] = buffer_f4(rq, qrow + eoff(kk + 16 * ks + 8 * h));
        qa[ks][1] = buffer_f4(rq, qrow + eoff(kk + 16 * ks + 8 * h + 4));
      }
    }
    kb[0] = buffer_f4(rk, boff + eoff(kk + 8 * bkg));
    kb[1] = buffer_f4(rk, boff + eoff(kk + 8 * bkg + 4));
  };
  float sq = 1.0f, sk = 1.0f;  // this lane's query scale, this thread's block scale
  auto publish = [&](u4 *buf) {
    const Pieces pb = split8(kb[0], kb[1], sk);
    buf[0 * kPlane + bslot] = pb.hi;
    buf[1 * kPlane + bslot] = pb.lo;
  };

  // Software pipeline over 32-element steps, as in the bf16 split scorer: at
  // the top of step s the wave splits the raw data of step s + 1 and issues
  // the loads of step s + 2; one workgroup barrier per step.
  const int nsteps = (K + BK - 1) / BK;
  auto step = [&](int s, const Pieces (&use)[2], Pieces (&fill)[2]) {
    const u4 *cur = bl + (s & 1) * (2 * kPlane);
    u4 *nxt = bl + ((s + 1) & 1) * (2 * kPlane);
    if (QD) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this step's staged queries and blocks
      read_q((s + 1) & 1);
      publish(nxt);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) fill[ks] = split8(qa[ks][0], qa[ks][1], sq);
    if (!QD) publish(nxt);
    load((s + 2) * BK);  // past K: out-of-range offsets, no memory access
    __builtin_amdgcn_sched_barrier(0);
    Pieces pbv[2][2];  // [ks][ni]
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        if (FULL || ni < nni) {
          const int o = (ks * 2 + ni) * 64 + (lane ^ lane_swz(2 * ks + h));
          pbv[ks][ni].hi = cur[0 * kPlane + o];
          pbv[ks][ni].lo = cur[1 * kPlane + o];
        }
      }
    // Product order, fixed for every element: hi*hi of both K halves into
    // the hh set; then hi*lo of both halves and lo*hi of both halves into
    // the correction set.
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          if (!(FULL || ni < nni)) continue;
          const Pieces &x = use[ks];
          const Pieces &y = pbv[ks][ni];
          if (p == 0) acc[0][ni] = mfma_f16(x.hi, y.hi, acc[0][ni]);
          else if (p == 1) acc[1][ni] = mfma_f16(x.hi, y.lo, acc[1][ni]);
          else acc[1][ni] = mfma_f16(x.lo, y.hi, acc[1][ni]);
        }
    if (QD) {
      // Barrier for the block planes only: this wave's LDS reads and writes
      // are done (lgkmcnt); the direct loads of step s + 2 stay in flight
      // across it (a full __syncthreads() waits for them too), and the wait
      // at the top of step s + 1 covers them (44.5 against 45.9 us per 256 x
      // 32K-block call).  The empty asm statements keep the compiler from
      // moving LDS accesses across the barrier instruction.
      __builtin_amdgcn_s_waitcnt(0xC07F);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      __syncthreads();
    }
  };

  Pieces pa[2], pn[2];
  load(0);
  if (QD) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    read_q(0);
  }
  {
    // Row scales from the first step: a query row's 32 elements sit in lanes
    // l and l ^ 32, a block row's in four consecutive threads.
    float mq = fmaxf(max_abs8(qa[0][0], qa[0][1]), max_abs8(qa[1][0], qa[1][1]));
    mq = fmaxf(mq, __shfl_xor(mq, 32));
    const int eq = row_exp(mq);
    sq = __builtin_amdgcn_ldexpf(1.0f, -eq);
    if (h == 0) eqs[32 * wave + r32] = eq;
    float mk = max_abs8(kb[0], kb[1]);
    mk = fmaxf(mk, __shfl_xor(mk, 1));
    mk = fmaxf(mk, __shfl_xor(mk, 2));
    const int ek = row_exp(mk);
    sk = __builtin_amdgcn_ldexpf(1.0f, -ek);
    if (bkg == 0) eks[brow] = ek;
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) pa[ks] = split8(qa[ks][0], qa[ks][1], sq);
  publish(bl);
  load(BK);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    step(s, pa, pn);
    if (s + 1 < nsteps) step(s + 1, pn, pa);
  }

  // The loop's barriers have published eqs/eks.
  f16v v[2];
  uint32_t bad = 0;
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    v[ni] = acc[0][ni] + acc[1][ni];
    bad |= unscale16(v[ni], eqs, 32 * wave, h, eks[32 * ni + r32], ni);
  }

  if (FULL && QD) {
    // Full tile: the wave's 32 x 64 results go through its own staging area
    // (free now: no query row is in flight) so each lane stores whole float4s
    // of a row; rows that are not 16-byte aligned store the four floats one
    // by one.
    float *tl = reinterpret_cast<float *>(qst);  // [32 rows][64 columns]
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) tl[(8 * (r >> 2) + 4 * h + (r & 3)) * 64 + 32 * ni + r32] = v[ni][r];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes are done
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = j * 64 + lane;  // float4 e of 512: row e / 16, columns 4 (e % 16) ..
      const int row = e >> 4, c4 = (e & 15) * 4;
      const f4 val = *reinterpret_cast<const f4 *>(tl + row * 64 + c4);
      const int grow = q0 + 32 * wave + row;
      if (grow < nq) {
        float *dst = scores + int64_t(grow) * A + b0 + c4;
        if ((A & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0) {
          *reinterpret_cast<f4 *>(dst) = val;
        } else {
          dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
        }
      }
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = b0 + 32 * ni + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = q0 + 32 * wave + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < nq && col < A) scores[int64_t(row) * A + col] = v[ni][r];
      }
    }
  }
  fix_range(bad, q, kblk, nq, K, A, scores, q0 + 32 * wave, b0, r32, h);
}

// Tile assignment as in the bf16 split scorer: workgroup ids go round-robin
// over the 8 XCDs; each XCD takes an equal share of the full tiles (query
// tiles of one block tile adjacent) and then every eighth ragged tile (the
// last, partial 64-block column, for each query tile).  QD (K a multiple of
// 32, every workload here) stages the query rows through LDS and runs three
// workgroups per CU; other K load the query slices into registers, two
// workgroups per CU.
template <bool QD>
__global__ __launch_bounds__(256, QD ? 3 : 2) void scores_f16x2_kernel(const float *__restrict__ q,
                                                                       const float *__restrict__ kblk,
                                                                       int nq, int K, int A,
                                                                       float *__restrict__ scores,
                                                                       int nqt, int nct, int ntail) {
  __shared__ u4 bl[2 * 2 * kPlane];              // 16 KB: two steps x two planes
  __shared__ u4 qst[QD ? 4 * 2 * 256 : 1];       // 32 KB: per wave, two steps of 32 query rows
  __shared__ __attribute__((aligned(16))) int eqs[BM];  // row scale exponents of the tile's queries
  __shared__ int eks[BN];                                // ... and of its blocks
  const int x = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  u4 *mq = qst + (QD ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 512 : 0);
  const int tails_here = ntail > x ? (ntail - x + 7) / 8 : 0;
  const int64_t nfull = int64_t(nqt) * (nct - (ntail > 0 ? 1 : 0));
  const int64_t fhere = nfull * (x + 1) / 8 - nfull * x / 8;
  if (slot >= fhere) {
    const int ts = int(slot - fhere);
    if (ts >= tails_here) return;
    const int u = x + 8 * ts;  // ragged tile: query tile u of the last block column
    split_tile<false, QD>(q, kblk, nq, K, A, scores, u * BM, (nct - 1) * BN, bl, mq, eqs, eks);
    return;
  }
  const int64_t f = nfull * x / 8 + slot;
  split_tile<true, QD>(q, kblk, nq, K, A, scores, int(f % nqt) * BM, int(f / nqt) * BN, bl, mq,
                       eqs, eks);
}

}  // namespace

hipError_t launch_block_scores_f16x2(const float *q, const float *kblk, int nq, int K, int A,
                                     float *scores, hipStream_t stream) {
  const int nqt = (nq + BM - 1) / BM;
  const int nct = (A + BN - 1) / BN;
  const int ntail = A % BN == 0 ? 0 : nqt;
  const int64_t nfull = int64_t(nqt) * (nct - (ntail ? 1 : 0));
  int64_t per = 0;  // workgroups per XCD: the largest share
  for (int x = 0; x < 8; ++x) {
    const int64_t tails = ntail > x ? (ntail - x + 7) / 8 : 0;
    per = std::max(per, tails + nfull * (x + 1) / 8 - nfull * x / 8);
  }
  if (K % BK == 0)
    scores_f16x2_kernel<true><<<int(8 * per), 256, 0, stream>>>(q, kblk, nq, K, A, scores, nqt,
                                                                nct, ntail);
  else
    scores_f16x2_kernel<false><<<int(8 * per), 256, 0, stream>>>(q, kblk, nq, K, A, scores, nqt,
                                                                 nct, ntail);
  return hipGetLastError();
}

}  // namespace qsa
