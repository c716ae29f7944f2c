// Block scoring on bf16 matrix cores with an exact three-way split (gfx950).
//
// Page "#337 hip: gfx12 (RDNA4) QSA select - WMMA block scorer, prompt-aware
// top-k dispatch", What item 2: every fp32 operand x is cut into three bf16
// numbers hi + mid + lo == x exactly (each holds the next 8 significant bits:
// hi is x truncated to bf16, mid is (x - hi) truncated, lo = x - hi - mid),
// and a product q*k is formed from the six slice products of order <= 2:
//   hi*hi  +  [hi*mid + mid*hi + hi*lo + mid*mid + lo*hi],
// dropping mid*lo, lo*mid and lo*lo (each below 2^-24 of |q*k|).  Every slice
// product is exact in fp32.  The hi*hi products get their own accumulator and
// the five corrections another, added once at the end, so the corrections are
// not rounded at the large accumulator's ulp.
//
// On CDNA4 the dense bf16 matrix rate is 16x the fp32 one, so six bf16 MFMAs
// per fp32-equivalent product still run ~2.7x faster than fp32 MFMA.
//
// Workgroup tile: 128 queries x 64 blocks, 4 waves.  Wave w owns queries
// [32w, 32w + 32) against both 32-block halves of the tile over the whole of
// K, in steps of 32 = two 16-element halves (v_mfma_f32_32x32x16_bf16; lane l
// supplies row l%32, K elements 8*(l/32) .. +7 of a half, and holds rows
// 8*(r/4) + 4*(l/32) + r%4 of column l%32 of the result in register r).  The
// block summaries of a step are shared by the four waves: thread t loads 8
// consecutive elements of block row t/4, splits them and writes the three
// 16-byte planes to LDS exactly where the MFMA lane that needs them will read
// them; two LDS buffers alternate, one barrier per step.  Each wave splits its
// own query slices in registers.  When K is a multiple of 32 the wave's query
// rows reach it through LDS: direct buffer-to-LDS loads in which 8 lanes read
// one 128-byte row segment (a load instruction touches 8 cache lines instead
// of 32), then one ds_read per MFMA slice.  A wave keeps eight accumulators per tile
// column half: hi*hi and corrections, each separately for the two K halves
// of a step (so that no accumulator is reused within four MFMAs); the score
// is (hh_0 + hh_1) + (c_0 + c_1).  No cross-wave combine: each wave stores
// its 32 x 64 results from registers.
//
// Position invariance: a ragged tile runs the same per-element instruction
// sequence (hardware-bounded buffer loads return zeros past the valid rows;
// zero slices add exact zeros), so equal summaries score bitwise-equal.  A
// ragged column of at most 32 blocks is split by K half (split_tail) without
// changing any accumulator's sequence of MFMAs.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qsa_internal.h"

namespace qsa {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int BM = 128;  // queries per tile
constexpr int BN = 64;   // blocks per tile
constexpr int BK = 32;   // K elements per step
constexpr int BT = 64;   // queries per narrow ragged tile (split_tail)
constexpr uint32_t kOutOfRange = 0x40000000u;  // byte offset past any tile resource

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const float *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, int(bytes), 0x00020000);
}

__device__ __forceinline__ f4 buffer_f4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The three bf16 planes of 8 consecutive fp32 values (x[0..3] = a, x[4..7] = b),
// each packed as 8 bf16 (element 2i in the low half of word i).
struct Planes {
  u4 hi, mid, lo;
};

__device__ __forceinline__ uint32_t pack_hi16(uint32_t even, uint32_t odd) {
  // low half <- even[31:16], high half <- odd[31:16]
  return __builtin_amdgcn_perm(odd, even, 0x07060302u);
}

__device__ __forceinline__ Planes split8(f4 a, f4 b) {
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t hb[8], mb[8], lb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t u = __float_as_uint(x[i]);
    hb[i] = u;                                          // hi = top 16 bits of u
    const float r1 = x[i] - __uint_as_float(u & 0xFFFF0000u);  // exact: <= 16 significant bits
    const uint32_t v = __float_as_uint(r1);
    mb[i] = v;                                          // mid = top 16 bits of r1
    const float r2 = r1 - __uint_as_float(v & 0xFFFF0000u);    // exact: <= 8 significant bits
    lb[i] = __float_as_uint(r2);                        // lo = r2, exact in bf16
  }
  Planes p;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    p.hi[w] = pack_hi16(hb[2 * w], hb[2 * w + 1]);
    p.mid[w] = pack_hi16(mb[2 * w], mb[2 * w + 1]);
    p.lo[w] = pack_hi16(lb[2 * w], lb[2 * w + 1]);
  }
  return p;
}

__device__ __forceinline__ f16v mfma_bf16(u4 a, u4 b, f16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8, a),
                                                 __builtin_bit_cast(bf8, b), c, 0, 0, 0);
}

// LDS slots of a step's block planes are [ks][column half][lane]; lane l of
// K group g = 2 ks + l/32 sits at l ^ lane_swz(g).  Without the swizzle the
// four K groups a thread quartet writes (one block row) fall on the same
// banks; with it, both the writes (8 or 16 lanes per pass) and the MFMA-lane
// reads (a permutation of consecutive slots) are free of bank conflicts for
// 32 or 64 four-byte banks.
__device__ __forceinline__ int lane_swz(int g) { return (g << 2) ^ ((g >> 1) << 1); }

// One 128 x 64 tile.  FULL: all 64 block rows active; otherwise a 32-block
// half without an active block skips its MFMAs.
typedef __attribute__((address_space(3))) void lds_void;

template <bool FULL, bool QD>
__device__ __forceinline__ void split_tile(const float *__restrict__ q,
                                           const float *__restrict__ kblk, int nq, int K, int A,
                                           float *__restrict__ scores, int q0, int b0, u4 *bl,
                                           u4 *qst) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int r32 = lane & 31;
  const int h = lane >> 5;
  const int nni = FULL ? 2 : min(2, (A - b0 + 31) / 32);

  const uint32_t row_bytes = uint32_t(K) * 4u;
  const __amdgpu_buffer_rsrc_t rq = tile_rsrc(q + int64_t(q0) * K, uint32_t(min(BM, nq - q0)) * row_bytes);
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kblk + int64_t(b0) * K, uint32_t(min(BN, A - b0)) * row_bytes);

  // Query slices: lane supplies row 32*wave + r32, elements kk + 16*ks + 8h .. +7.
  const uint32_t qrow = uint32_t(32 * wave + r32) * row_bytes;
  // Block share: thread t loads row t/4, elements kk + 8*(t%4) .. +7, i.e. K
  // half ks = (t%4)/2 of MFMA lane (row%32) + 32*((t%4)%2) of column half row/32.
  const int brow = t >> 2;
  const int bkg = t & 3;
  const uint32_t boff = uint32_t(brow) * row_bytes;
  const int bslot = ((bkg >> 1) * 2 + (brow >> 5)) * 64 + (((brow & 31) + 32 * (bkg & 1)) ^ lane_swz(bkg));
  constexpr int kPlane = 2 * 2 * 64;  // u4 entries per plane of one step

  auto eoff = [&](int e) -> uint32_t { return e < K ? uint32_t(e) * 4u : kOutOfRange; };

  // acc[ks][set][ni]: set 0 = hi*hi, set 1 = corrections; ks = K half of a step.
  f16v acc[2][2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[a][c][ni] = f16v{};

  f4 qa[2][2], kb[2];
  // QD (K a multiple of 32): the wave's 32 query rows of a step go global ->
  // LDS by direct loads, 8 lanes per 128-byte row segment, piece p of row r
  // at slot p ^ ((r >> 1) & 7); the lanes then read their MFMA slices.
  // Row 8i + lane/8 of the wave: the swizzle depends on i only through its
  // parity, so two lane offsets serve the four loads and the row step 8i goes
  // into the scalar offset.
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
  auto publish = [&](u4 *buf) {
    const Planes pb = split8(kb[0], kb[1]);
    buf[0 * kPlane + bslot] = pb.hi;
    buf[1 * kPlane + bslot] = pb.mid;
    buf[2 * kPlane + bslot] = pb.lo;
  };

  // Software pipeline over 32-element steps.  At the top of step s the wave
  // splits the raw data of step s + 1 (its query slices into registers, its
  // share of the block slices into the other LDS buffer) and at once issues
  // the loads of step s + 2, so they have the whole MFMA section of step s to
  // arrive; a scheduling barrier keeps the compiler from sinking them.  With
  // QD the query rows of step s + 2 land in the wave's other staging buffer
  // (the workgroup barrier at the end of step s waits for them, as for any
  // LDS write).  One
  // workgroup barrier per step publishes the next buffer and retires the
  // reads of the buffer it will overwrite.  The loop is unrolled by two so
  // the query planes of consecutive steps alternate between two register
  // sets instead of being copied.
  const int nsteps = (K + BK - 1) / BK;
  auto step = [&](int s, const Planes (&use)[2], Planes (&fill)[2]) {
    const u4 *cur = bl + (s & 1) * (3 * kPlane);
    u4 *nxt = bl + ((s + 1) & 1) * (3 * kPlane);
    if (QD) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this step's staged queries and blocks
      read_q((s + 1) & 1);
      publish(nxt);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) fill[ks] = split8(qa[ks][0], qa[ks][1]);
    if (!QD) publish(nxt);
    load((s + 2) * BK);  // past K: out-of-range offsets, no memory access
    __builtin_amdgcn_sched_barrier(0);
    Planes pbv[2][2];  // [ks][ni]
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        if (FULL || ni < nni) {
          const int o = (ks * 2 + ni) * 64 + (lane ^ lane_swz(2 * ks + h));
          pbv[ks][ni].hi = cur[0 * kPlane + o];
          pbv[ks][ni].mid = cur[1 * kPlane + o];
          pbv[ks][ni].lo = cur[2 * kPlane + o];
        }
      }
    // Product order, fixed for every element: hi*hi into the hh set; then
    // hi*mid, mid*hi, hi*lo, mid*mid, lo*hi into the correction set.
#pragma unroll
    for (int p = 0; p < 6; ++p)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          if (!(FULL || ni < nni)) continue;
          const Planes &x = use[ks];
          const Planes &y = pbv[ks][ni];
          switch (p) {
            case 0: acc[ks][0][ni] = mfma_bf16(x.hi, y.hi, acc[ks][0][ni]); break;
            case 1: acc[ks][1][ni] = mfma_bf16(x.hi, y.mid, acc[ks][1][ni]); break;
            case 2: acc[ks][1][ni] = mfma_bf16(x.mid, y.hi, acc[ks][1][ni]); break;
            case 3: acc[ks][1][ni] = mfma_bf16(x.hi, y.lo, acc[ks][1][ni]); break;
            case 4: acc[ks][1][ni] = mfma_bf16(x.mid, y.mid, acc[ks][1][ni]); break;
            default: acc[ks][1][ni] = mfma_bf16(x.lo, y.hi, acc[ks][1][ni]); break;
          }
        }
    __syncthreads();
  };

  Planes pa[2], pn[2];
  load(0);
  if (QD) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    read_q(0);
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) pa[ks] = split8(qa[ks][0], qa[ks][1]);
  publish(bl);
  load(BK);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    step(s, pa, pn);
    if (s + 1 < nsteps) step(s + 1, pn, pa);
  }

  if (FULL && QD) {
    // Full tile: the wave's 32 x 64 results go through its own staging area
    // (free now: no query row is in flight) so each lane stores whole float4s
    // of a row -- 8 wide stores per lane instead of 32 single floats (1-2 us
    // less per 256 x 32K-block select).  Rows that are not 16-byte aligned
    // store the four floats one by one.
    float *tl = reinterpret_cast<float *>(qst);  // [32 rows][64 columns]
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const f16v v = (acc[0][0][ni] + acc[1][0][ni]) + (acc[0][1][ni] + acc[1][1][ni]);
#pragma unroll
      for (int r = 0; r < 16; ++r) tl[(8 * (r >> 2) + 4 * h + (r & 3)) * 64 + 32 * ni + r32] = v[r];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes are done
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = j * 64 + lane;          // float4 e of 512: row e / 16, columns 4 (e % 16) ..
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
    return;
  }
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const f16v v = (acc[0][0][ni] + acc[1][0][ni]) + (acc[0][1][ni] + acc[1][1][ni]);
    const int col = b0 + 32 * ni + r32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = q0 + 32 * wave + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < nq && col < A) scores[int64_t(row) * A + col] = v[r];
    }
  }
}

// A ragged tile whose active blocks fit one 32-block column half (A % 64 in
// 1..32), for 64 queries.  The two K halves of every step are independent
// accumulations until the final sum (hh_0, c_0 and hh_1, c_1 above), so wave
// w takes query group w / 2 and K half w % 2 only: each wave runs half the
// MFMAs and half the query split of a full-width ragged tile, and the tail
// spreads over twice as many workgroups.  Each accumulator receives the same
// MFMAs in the same order as in split_tile, and the halves meet in LDS in the
// same expression, so the scores are bitwise those of a full tile.
__device__ __forceinline__ void split_tail(const float *__restrict__ q,
                                           const float *__restrict__ kblk, int nq, int K, int A,
                                           float *__restrict__ scores, int q0, int b0, u4 *bl) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int qg = wave >> 1;  // query group: rows q0 + 32 qg ..
  const int kh = wave & 1;   // K half of every step
  const int r32 = lane & 31;
  const int h = lane >> 5;

  const uint32_t row_bytes = uint32_t(K) * 4u;
  const __amdgpu_buffer_rsrc_t rq = tile_rsrc(q + int64_t(q0) * K, uint32_t(min(BT, nq - q0)) * row_bytes);
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kblk + int64_t(b0) * K, uint32_t(min(BN, A - b0)) * row_bytes);
  const uint32_t qrow = uint32_t(32 * qg + r32) * row_bytes;
  const int brow = t >> 2;
  const int bkg = t & 3;
  const uint32_t boff = uint32_t(brow) * row_bytes;
  const int bslot = ((bkg >> 1) * 2 + (brow >> 5)) * 64 + (((brow & 31) + 32 * (bkg & 1)) ^ lane_swz(bkg));
  constexpr int kPlane = 2 * 2 * 64;
  auto eoff = [&](int e) -> uint32_t { return e < K ? uint32_t(e) * 4u : kOutOfRange; };

  f16v hh = f16v{}, cc = f16v{};
  f4 qa[2], kb[2];
  auto load = [&](int kk) {
    qa[0] = buffer_f4(rq, qrow + eoff(kk + 16 * kh + 8 * h));
    qa[1] = buffer_f4(rq, qrow + eoff(kk + 16 * kh + 8 * h + 4));
    kb[0] = buffer_f4(rk, boff + eoff(kk + 8 * bkg));
    kb[1] = buffer_f4(rk, boff + eoff(kk + 8 * bkg + 4));
  };
  auto publish = [&](u4 *buf) {
    const Planes pb = split8(kb[0], kb[1]);
    buf[0 * kPlane + bslot] = pb.hi;
    buf[1 * kPlane + bslot] = pb.mid;
    buf[2 * kPlane + bslot] = pb.lo;
  };
  const int nsteps = (K + BK - 1) / BK;
  auto step = [&](int s, const Planes &use, Planes &fill) {
    const u4 *cur = bl + (s & 1) * (3 * kPlane);
    u4 *nxt = bl + ((s + 1) & 1) * (3 * kPlane);
    fill = split8(qa[0], qa[1]);
    publish(nxt);
    load((s + 2) * BK);
    __builtin_amdgcn_sched_barrier(0);
    const int o = (kh * 2) * 64 + (lane ^ lane_swz(2 * kh + h));
    Planes y;
    y.hi = cur[0 * kPlane + o];
    y.mid = cur[1 * kPlane + o];
    y.lo = cur[2 * kPlane + o];
    hh = mfma_bf16(use.hi, y.hi, hh);
    cc = mfma_bf16(use.hi, y.mid, cc);
    cc = mfma_bf16(use.mid, y.hi, cc);
    cc = mfma_bf16(use.hi, y.lo, cc);
    cc = mfma_bf16(use.mid, y.mid, cc);
    cc = mfma_bf16(use.lo, y.hi, cc);
    __syncthreads();
  };
  Planes pa, pn;
  load(0);
  pa = split8(qa[0], qa[1]);
  publish(bl);
  load(BK);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    step(s, pa, pn);
    if (s + 1 < nsteps) step(s + 1, pn, pa);
  }
  // The K-half-1 waves hand their accumulators over through LDS (free after
  // the last step's barrier): [query group][register][lane].
  float *xch = reinterpret_cast<float *>(bl);
  if (kh == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      xch[(qg * 32 + r) * 64 + lane] = hh[r];
      xch[(qg * 32 + 16 + r) * 64 + lane] = cc[r];
    }
  }
  __syncthreads();
  if (kh == 0) {
    const int col = b0 + r32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = (hh[r] + xch[(qg * 32 + r) * 64 + lane]) + (cc[r] + xch[(qg * 32 + 16 + r) * 64 + lane]);
      const int row = q0 + 32 * qg + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < nq && col < A) scores[int64_t(row) * A + col] = v;
    }
  }
}

// Tile assignment: workgroup ids go round-robin over the 8 XCDs; each XCD
// takes an equal share of the full tiles (query tiles of one block tile
// adjacent) and then every eighth ragged unit.  A ragged unit is a 64-query
// split_tail tile when the ragged column has at most 32 active blocks
// (narrow), else a 128-query split_tile<false> tile.  The ragged units come
// last: on a 131K context they fill slots freed at the end of the full tiles'
// second round (scorer 63.2 -> 62.3 us; 23.0 -> 21.9 us on a 32K context).
// QD (K a multiple of 32, every workload here) stages the query rows through
// LDS with direct loads and runs at two waves per SIMD; the other K take the
// register-loaded queries in an instance of their own with the whole
// register file per wave, so neither instance spills.
template <bool QD>
__global__ __launch_bounds__(256, QD ? 2 : 1) void scores_bf16x3_kernel(const float *__restrict__ q,
                                                               const float *__restrict__ kblk,
                                                               int nq, int K, int A,
                                                               float *__restrict__ scores,
                                                               int nqt, int nct, int ntail,
                                                               int narrow) {
  __shared__ u4 bl[2 * 3 * 2 * 2 * 64];  // 24 KB: two steps x three planes x (2 K halves x 2 column halves x 64 lanes)
  __shared__ u4 qst[QD ? 4 * 2 * 256 : 1];  // 32 KB: per wave, two steps of 32 query rows x 128 bytes
  const int x = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  u4 *mq = qst + (QD ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 512 : 0);
  const int tails_here = ntail > x ? (ntail - x + 7) / 8 : 0;
  const int64_t nfull = int64_t(nqt) * (nct - (ntail > 0 ? 1 : 0));
  const int64_t fhere = nfull * (x + 1) / 8 - nfull * x / 8;
  if (slot >= fhere) {
    const int ts = int(slot - fhere);
    if (ts >= tails_here) return;
    const int u = x + 8 * ts;  // ragged unit
    if (narrow) split_tail(q, kblk, nq, K, A, scores, u * BT, (nct - 1) * BN, bl);
    else split_tile<false, QD>(q, kblk, nq, K, A, scores, u * BM, (nct - 1) * BN, bl, mq);
    return;
  }
  const int64_t f = nfull * x / 8 + slot;
  split_tile<true, QD>(q, kblk, nq, K, A, scores, int(f % nqt) * BM, int(f / nqt) * BN, bl, mq);
}

}  // namespace

hipError_t launch_block_scores_bf16x3(const float *q, const float *kblk, int nq, int K, int A,
                                      float *scores, hipStream_t stream) {
  const int nqt = (nq + BM - 1) / BM;
  const int nct = (A + BN - 1) / BN;
  const int rag = A % BN;
  const int narrow = rag > 0 && rag <= 32;
  const int ntail = rag == 0 ? 0 : narrow ? (nq + BT - 1) / BT : nqt;
  const int64_t nfull = int64_t(nqt) * (nct - (ntail ? 1 : 0));
  int64_t per = 0;  // workgroups per XCD: the largest share
  for (int x = 0; x < 8; ++x) {
    const int64_t tails = ntail > x ? (ntail - x + 7) / 8 : 0;
    per = std::max(per, tails + nfull * (x + 1) / 8 - nfull * x / 8);
  }
  if (K % BK == 0)
    scores_bf16x3_kernel<true><<<int(8 * per), 256, 0, stream>>>(q, kblk, nq, K, A, scores, nqt,
                                                                 nct, ntail, narrow);
  else
    scores_bf16x3_kernel<false><<<int(8 * per), 256, 0, stream>>>(q, kblk, nq, K, A, scores, nqt,
                                                                  nct, ntail, narrow);
  return hipGetLastError();
}

}  // namespace qsa
