// Per-query radix top-k of block scores for gfx950 (CDNA4, wave64).
//
// Pages: "#3108 perf(hip): optimize exact QSA block scoring and top-k selection
// on gfx12", Summary item 2 (radix selection with 256-bin digit histograms and
// parallel prefix scans; keys held in registers with a per-thread width set by
// the number of blocks); "#337 hip: gfx12 (RDNA4) QSA select ...", What item 1
// (the width follows the ACTIVE block count, never the capacity).
//
// One workgroup of 1024 threads (16 waves) selects one row.  Steps:
//   1. key transform: fp32 score -> uint32 whose unsigned order is the score
//      order (-0.0 folded onto +0.0);
//   2. up to four MSB-first passes over 8-bit digits: a 256-bin LDS histogram
//      of the candidates still sharing the threshold prefix (one sub-histogram
//      per wave), a suffix scan to find the bin holding the k-th largest key,
//      then the prefix grows by that digit.  A pass whose bin is taken whole
//      ends the search early;
//   3. if more keys equal the threshold key T than are still needed, the same
//      passes run over the block id (lowest ids first) among keys == T -- so
//      ties go to the lower block id;
//   4. the k winners are gathered into LDS as (key, id) pairs and
//      bitonic-sorted into rank order: key descending, then id ascending.
// Keys live in registers, PER per thread plus one slot in LDS (thread t holds
// ids t + j*1024), PER chosen from the active block count.  Rows longer than
// the largest width stream their keys from global memory on every pass.
#include <hip/hip_runtime.h>

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int NT = kTopkThreads;
constexpr int NWAVES = NT / 64;
constexpr int MAXK = kTopkMaxK;

struct TopkShared {
  uint32_t hsub[NWAVES][256];  // per-wave digit histograms
  uint32_t wtot[4];            // scan carry of the four scanning waves
  uint32_t bcast[3];           // chosen digit, remaining k, count in the bin
  uint32_t count;              // gathered winners
  uint32_t extra[NT];          // each thread's last key slot (kept in LDS, not VGPRs)
  uint32_t bkey[MAXK];         // winners' keys ...
  uint32_t bid[MAXK];          // ... and ids, sorted into rank order
};

// Order-preserving map of an fp32 score to uint32: a larger score gives a
// larger key.  -0.0 is folded onto +0.0.  Key 0 is kept free as the "no
// block" sentinel of register slots past the row end; the one score that
// would map there is a NaN (whose rank is unspecified), so it moves to 1.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return key == 0u ? 1u : key;
}

// Given the histogram of the current digit in sh.hsub (complete: the caller
// has passed a barrier), find the digit d* holding the kr-th largest
// candidate.  Returns d*, the rank left inside that bin and the bin's size.
// `sub0` sentinel keys were counted in bin 0 and are taken out of it.
// Threads 0..255 reduce the per-wave histograms (clearing them for the next
// pass) and scan from the top digit down.  Contains two barriers; every
// thread of the workgroup must call it.
__device__ __forceinline__ void find_digit(TopkShared &sh, uint32_t sub0, uint32_t &kr,
                                           uint32_t &digit, uint32_t &cnt) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  uint32_t h = 0, v = 0;
  if (t < 256) {
    const int d = 255 - t;  // thread t scans digits from the top
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
      h += sh.hsub[w][d];
      sh.hsub[w][d] = 0;
    }
    if (d == 0) h -= sub0;
    v = h;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(v, off, 64);
      if (lane >= off) v += y;
    }
    if (lane == 63) sh.wtot[wave] = v;
  }
  __syncthreads();
  if (t < 256) {
    for (int w = 0; w < wave; ++w) v += sh.wtot[w];
    // v = number of candidates whose digit is >= d; exactly one d satisfies this.
    if (v >= kr && v - h < kr) {
      sh.bcast[0] = 255 - t;
      sh.bcast[1] = kr - (v - h);
      sh.bcast[2] = h;
    }
  }
  __syncthreads();
  digit = sh.bcast[0];
  kr = sh.bcast[1];
  cnt = sh.bcast[2];
}

template <int PER>
struct RowKeys {
  uint32_t key[PER > 0 ? PER : 1];
};

template <int PER>
__global__ __launch_bounds__(NT) void topk_kernel(const float *__restrict__ scores, int A, int k,
                                                  int *__restrict__ ids) {
  __shared__ TopkShared sh;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const float *srow = scores + int64_t(blockIdx.x) * A;
  int *orow = ids + int64_t(blockIdx.x) * k;
  const int m = min(k, A);

  if (m == 0) {  // no active blocks: every slot is padding
    for (int r = t; r < k; r += NT) orow[r] = -1;
    return;
  }

  for (int i = t; i < NWAVES * 256; i += NT) (&sh.hsub[0][0])[i] = 0;
  if (t == 0) sh.count = 0;

  // Thread t owns ids t + j*NT: slots j < PER in VGPRs, slot PER in LDS
  // (sh.extra[t]), so a row of (PER+1)*NT ids needs only PER registers -- the
  // capacity-sized rows of 2^n + 2 blocks spill just two ids into the extra
  // slot.  Slots past the row end hold the sentinel key 0: it never matches a
  // threshold (real keys are >= 1), is never gathered, and the n_sentinel of
  // them are taken out of bin 0 while the prefix is still 0.  This keeps
  // per-slot validity masks out of the hot loops.
  RowKeys<PER> rk;
  uint32_t n_sentinel = 0;
  if constexpr (PER >= 0) {
    n_sentinel = uint32_t((PER + 1) * NT - A);
#pragma unroll
    for (int j = 0; j <= PER; ++j) {
      const int id = j * NT + t;
      const uint32_t key = id < A ? score_key(srow[id]) : 0u;
      if (j < PER)
        rk.key[j < PER ? j : 0] = key;
      else
        sh.extra[t] = key;
    }
  }
  // Visit every (id, key) this thread owns (sentinel slots included).  The
  // empty asm hides that `tv` equals t, so ids are recomputed in each visit
  // (one add) instead of being hoisted into PER more live registers.
  auto for_each = [&](auto &&f) {
    if constexpr (PER >= 0) {
      int tv = t;
      asm volatile("" : "+v"(tv));
#pragma unroll
      for (int j = 0; j < PER; ++j) f(j * NT + tv, rk.key[j]);
      f(PER * NT + tv, sh.extra[tv]);
    } else {
      for (int id = t; id < A; id += NT) f(id, score_key(srow[id]));
    }
  };
  __syncthreads();

  uint32_t pref = 0, mask = 0;      // threshold key prefix and the bits it fixes
  uint32_t idpref = 0, idmask = 0;  // the same for reversed ids among keys == T
  uint32_t idtop = 0;               // ids map to rid = idtop - id (larger rid = lower id)
  bool by_id = false;

  if (k < A) {
    uint32_t kr = uint32_t(k);
    bool done = false;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for_each([&](int, uint32_t key) {
        if ((key & mask) == pref) atomicAdd(&sh.hsub[wave][(key >> shift) & 255u], 1u);
      });
      __syncthreads();
      uint32_t d, cnt;
      find_digit(sh, pref == 0 ? n_sentinel : 0u, kr, d, cnt);
      pref |= d << shift;
      mask |= 0xFFu << shift;
      if (cnt == kr) {
        done = true;
        break;
      }
    }
    if (!done) {
      // More keys equal T = pref than are still needed: take the kr lowest ids.
      by_id = true;
      const int idbits = 32 - __clz(uint32_t(A - 1));
      idtop = idbits >= 32 ? 0xFFFFFFFFu : ((1u << idbits) - 1u);
      for (int shift = 8 * ((idbits + 7) / 8 - 1); shift >= 0; shift -= 8) {
        for_each([&](int id, uint32_t key) {
          const uint32_t rid = idtop - uint32_t(id);
          if (key == pref && (rid & idmask) == idpref)
            atomicAdd(&sh.hsub[wave][(rid >> shift) & 255u], 1u);
        });
        __syncthreads();
        uint32_t d, cnt;
        find_digit(sh, 0u, kr, d, cnt);
        idpref |= d << shift;
        idmask |= 0xFFu << shift;
        if (cnt == kr) break;
      }
    }
  }

  // Gather the winners: one LDS atomic per wave and visit.
  for_each([&](int id, uint32_t key) {
    const uint32_t kp = key & mask;
    bool sel = kp > pref;
    if (kp == pref) sel = !by_id || (((idtop - uint32_t(id)) & idmask) >= idpref);
    sel = sel && key != 0u;
    const uint64_t bal = __ballot(sel);
    if (bal) {
      const int leader = __ffsll((unsigned long long)bal) - 1;
      uint32_t base = 0;
      if (lane == leader) base = atomicAdd(&sh.count, uint32_t(__popcll(bal)));
      base = __shfl(base, leader, 64);
      const uint32_t below = __builtin_amdgcn_mbcnt_hi(uint32_t(bal >> 32),
                                                       __builtin_amdgcn_mbcnt_lo(uint32_t(bal), 0u));
      if (sel && base + below < uint32_t(MAXK)) {  // exactly m <= MAXK are selected
        sh.bkey[base + below] = key;
        sh.bid[base + below] = uint32_t(id);
      }
    }
  });

  int P = 1;
  while (P < m) P <<= 1;
  __syncthreads();
  for (int i = m + t; i < P; i += NT) {  // padding ranks after every winner
    sh.bkey[i] = 0u;
    sh.bid[i] = 0xFFFFFFFFu;
  }
  __syncthreads();

  // Bitonic sort of [0, P) into rank order.  "x before y" is the strict
  // total order key desc, id asc; a block of the network whose index has the
  // `size` bit clear sorts forward, otherwise backward.
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = t; p < (P >> 1); p += NT) {
        const int i = ((p & ~(stride - 1)) << 1) | (p & (stride - 1));
        const int j = i + stride;
        const uint32_t ki = sh.bkey[i], kj = sh.bkey[j];
        const uint32_t ii = sh.bid[i], ij = sh.bid[j];
        const bool j_first = kj > ki || (kj == ki && ij < ii);
        const bool forward = (i & size) == 0;
        if (j_first == forward) {
          sh.bkey[i] = kj;
          sh.bkey[j] = ki;
          sh.bid[i] = ij;
          sh.bid[j] = ii;
        }
      }
      __syncthreads();
    }
  }

  for (int r = t; r < k; r += NT) orow[r] = r < m ? int(sh.bid[r]) : -1;
}

template <int PER>
hipError_t launch_topk(const float *scores, int nq, int A, int k, int *ids, hipStream_t stream) {
  topk_kernel<PER><<<nq, NT, 0, stream>>>(scores, A, k, ids);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_topk(const float *scores, int nq, int A, int k, int *ids,
                             hipStream_t stream) {
  // Register width from the active block count only: the smallest PER with
  // (PER + 1) * NT >= A; longer rows stream from memory on every pass.
  const int slots = (A + NT - 1) / NT;  // PER + 1 needed
  if (slots <= 1) return launch_topk<0>(scores, nq, A, k, ids, stream);
  if (slots <= 2) return launch_topk<1>(scores, nq, A, k, ids, stream);
  if (slots <= 4) return launch_topk<3>(scores, nq, A, k, ids, stream);
  if (slots <= 8) return launch_topk<7>(scores, nq, A, k, ids, stream);
  if (slots <= 16) return launch_topk<15>(scores, nq, A, k, ids, stream);
  if (slots <= 24) return launch_topk<23>(scores, nq, A, k, ids, stream);
  if (slots <= 33) return launch_topk<32>(scores, nq, A, k, ids, stream);
  if (slots <= 48) return launch_topk<47>(scores, nq, A, k, ids, stream);
  if (slots <= 65) return launch_topk<64>(scores, nq, A, k, ids, stream);
  return launch_topk<-1>(scores, nq, A, k, ids, stream);
}

}  // namespace qsa
