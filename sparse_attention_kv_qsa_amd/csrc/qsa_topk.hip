// Per-query radix top-k of block scores for gfx950 (CDNA4, wave64).
//
// Pages: "#3108 perf(hip): optimize exact QSA block scoring and top-k selection
// on gfx12", Summary item 2 (radix selection with 256-bin digit histograms and
// parallel prefix scans; keys held in registers with a per-thread width set by
// the number of blocks); "#337 hip: gfx12 (RDNA4) QSA select ...", What item 1
// (the width follows the ACTIVE block count, never the capacity).
//
// One workgroup of 1024 threads (16 waves) selects one row.
//   1. key transform: fp32 score -> uint32 whose unsigned order is the score
//      order (-0.0 folded onto +0.0).  Keys live in VGPRs, PER per thread plus
//      one slot in LDS (thread t holds ids t + j*1024), PER chosen from the
//      active block count; rows past the largest width stream from memory.
//   2. a lower bound on the threshold from the threads' own maxima (distinct
//      elements): each wave sorts its 64 maxima in registers and offers its
//      ceil(k/16)-th; the smallest offer is <= the k-th largest key.  Only
//      keys at or above the bound can win; they are compacted into LDS (a few
//      percent of an N(0,1) row at k/A = 1/64).
//   3. if at most 1024 keys are candidates (the usual case), they are sorted
//      whole (step 4) and the first k kept.  Otherwise a radix select on the
//      candidates: up to four MSB-first passes over 8-bit digits, each a
//      256-bin LDS histogram (one sub-histogram per wave), a suffix scan to
//      find the bin holding the k-th largest key, and the prefix grows by that
//      digit; a pass whose bin is taken whole ends early.  If more keys equal
//      the threshold key T than are still needed, the same passes run over the
//      block id (lowest first) among keys == T, so ties go to the lower block
//      id.  (If the candidates overflow LDS, the passes run over the
//      register-resident row instead; the result is the same.)
//   4. rank order (key desc, id asc): a counting rank -- buckets by key, one
//      prefix sum over the bucket counts, then a count of the larger words
//      inside each pair's own bucket (1, 2 or 4 pairs per thread) -- unless a
//      bucket takes more than kBucketCap pairs (bulk ties); then a bitonic
//      sort: in registers with lane exchanges for strides < 64, through LDS
//      above that.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <type_traits>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int NT = kTopkThreads;
constexpr int NWAVES = NT / 64;
constexpr int MAXK = kTopkMaxK;
constexpr int CAP = 8192;  // LDS candidate capacity

struct TopkShared {
  uint64_t wbuf[2 * NT];       // rank words of the sort's cross-wave steps (two buffers)
  uint32_t hsub[NWAVES][256];  // per-wave digit histograms
  uint32_t wtot[4];            // scan carry of the four scanning waves
  uint32_t bcast[3];           // chosen digit, remaining k, count in the bin
  uint32_t ncand;              // candidates gathered
  uint32_t nwin;               // winners gathered
  uint32_t wmin[NWAVES];       // per-wave candidate bound; per-wave smallest key of the counting rank
  uint32_t wmax[NWAVES];       // per-wave largest key of the counting rank
  uint32_t big;                // the counting rank met a bucket past its cap
  uint32_t wsum[NWAVES];       // wave totals of the wide counting rank's prefix sum
  union {
    struct {
      uint32_t ckey[CAP];      // candidates: keys ...
      uint32_t cid[CAP];       // ... and block ids
    } c;
    uint64_t xbuf[CAP];        // the large sort's two exchange buffers, once the candidates are used
  } cu;
  uint32_t bkey[MAXK];         // winners: keys ...
  uint32_t bid[MAXK];          // ... and ids, sorted into rank order
  uint32_t extra[NT];          // each thread's last key slot (kept in LDS, not VGPRs)
};

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
    v = wave_incl_scan(h);
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

// Outcome of a radix select: an element (id, key) is a winner iff
//   (key & mask) >  pref, or
//   (key & mask) == pref and (!by_id or ((idtop - id) & idmask) >= idpref).
struct Threshold {
  uint32_t pref = 0, mask = 0;
  uint32_t idpref = 0, idmask = 0, idtop = 0;
  uint32_t tied = 0;  // winners that share the whole key T (pref, with a full mask)
  bool by_id = false;
  __device__ bool wins(uint32_t id, uint32_t key) const {
    const uint32_t kp = key & mask;
    const bool id_ok = !by_id | (((idtop - id) & idmask) >= idpref);
    return (kp > pref) | ((kp == pref) & id_ok);
  }
};

// Count `bin` into the wave's sub-histogram for the lanes where `take` holds.
// The lanes sharing the first such lane's bin add their count with one
// atomic: radix digits are often shared by most of the wave (the leading
// digit of keys of one magnitude, mass ties), and same-address LDS atomics
// serialise.  Every lane of the wave must call it.
__device__ __forceinline__ void hist_add(uint32_t *hsub, bool take, uint32_t bin) {
  const uint64_t act = __ballot(take);
  if (act == 0) return;  // wave-uniform
  const int first = __builtin_ctzll(act);
  const uint32_t lead = __builtin_amdgcn_readlane(bin, first);
  const bool same = take && bin == lead;
  const uint64_t nsame = __popcll(__ballot(same));
  if ((threadIdx.x & 63) == first) atomicAdd(&hsub[lead], uint32_t(nsame));
  else if (take && !same) atomicAdd(&hsub[bin], 1u);
}

// Radix select of the k largest (key, id) pairs among those `visit` yields
// (key 0 = sentinel; n_sentinel of them among the visited).  k must be less
// than the number of real keys.  ids are block ids < A.  With `keys_only`,
// a select that meets more keys equal to T than it still needs returns after
// the key passes (by_id set, tied = the number of them to take, lowest ids
// first) and leaves the id passes to the caller.
template <class Visit>
__device__ __forceinline__ Threshold radix_select(TopkShared &sh, Visit &&visit, uint32_t k, uint32_t n_sentinel,
                                  int A, bool keys_only = false) {
  const int wave = threadIdx.x >> 6;
  Threshold th;
  uint32_t kr = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    const uint32_t mask = th.mask, pref = th.pref;
    visit([&](uint32_t, uint32_t key) {
      hist_add(sh.hsub[wave], (key & mask) == pref, (key >> shift) & 255u);
    });
    __syncthreads();
    uint32_t d, cnt;
    find_digit(sh, th.pref == 0 ? n_sentinel : 0u, kr, d, cnt);
    th.pref |= d << shift;
    th.mask |= 0xFFu << shift;
    if (cnt == kr) {
      if (shift == 0) th.tied = kr;
      return th;
    }
  }
  // More keys equal T = pref than are still needed: take the kr lowest ids.
  th.by_id = true;
  th.tied = kr;
  if (keys_only) return th;
  const int idbits = 32 - __clz(uint32_t(A - 1));
  th.idtop = idbits >= 32 ? 0xFFFFFFFFu : ((1u << idbits) - 1u);
  for (int shift = 8 * ((idbits + 7) / 8 - 1); shift >= 0; shift -= 8) {
    const uint32_t T = th.pref, idmask = th.idmask, idpref = th.idpref, idtop = th.idtop;
    visit([&](uint32_t id, uint32_t key) {
      const uint32_t rid = idtop - id;
      hist_add(sh.hsub[wave], key == T && (rid & idmask) == idpref, (rid >> shift) & 255u);
    });
    __syncthreads();
    uint32_t d, cnt;
    find_digit(sh, 0u, kr, d, cnt);
    th.idpref |= d << shift;
    th.idmask |= 0xFFu << shift;
    if (cnt == kr) break;
  }
  return th;
}

// Append the (id, key) pairs for which pred holds to LDS arrays at
// counter `*count`, one LDS atomic per wave.  `visit` must visit every lane
// of the wave the same number of times (all lanes active).  Writes past
// `cap` are dropped; the counter still counts them.
// Append the (id, key) pairs for which pred holds to LDS arrays at counter
// `*count`, one LDS atomic per wave.  `visit` must visit every lane of the
// wave the same number of times (all lanes active).  If a wave's pairs would
// pass `cap`, that wave writes none of them; the counter still counts them.
// PER_THREAD: each thread counts its own pairs (vector adds, no per-slot wave
// operations), one prefix sum over the wave places them and each thread
// appends its own -- fewer instructions per slot, more registers (used up to
// 32 register slots per thread).  Otherwise a ballot per slot places them.
// The order of the pairs differs between the two; no caller depends on it.
//
// The per-thread form evaluates the predicate twice (count, then append)
// rather than keep every slot's result alive (two scalar registers a slot).
// To keep the compiler from reusing the first results, `hide` runs between
// the passes: it hides a value the predicate reads (one register move); the
// default hides each key instead (a move per slot).
struct HideKeys {
  __device__ void operator()() const {}
};
template <bool PER_THREAD, class Visit, class Pred, class Hide = HideKeys>
__device__ __forceinline__ void compact(Visit &&visit, Pred &&pred, uint32_t *count, uint32_t *dkey,
                        uint32_t *did, uint32_t cap, Hide &&hide = Hide{}) {
  const int lane = threadIdx.x & 63;
  if constexpr (PER_THREAD) {
    constexpr bool kHideKeys = std::is_same_v<std::decay_t<Hide>, HideKeys>;
    uint32_t mine = 0;
    visit([&](uint32_t id, uint32_t key) { mine += pred(id, key) ? 1u : 0u; });
    const uint32_t incl = wave_incl_scan(mine);
    const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
    uint32_t base = 0;
    if (lane == 0 && total) base = atomicAdd(count, total);
    base = __builtin_amdgcn_readfirstlane(base);
    if (base + total > cap) return;  // wave-uniform
    hide();
    // One LDS address per thread, advanced per pair; the id array's offset
    // from the key array is a constant (the store's immediate offset).
    uint32_t *kp = dkey + (base + incl - mine);
    const ptrdiff_t idoff = did - dkey;
    visit([&](uint32_t id, uint32_t key) {
      if constexpr (kHideKeys) asm volatile("" : "+v"(key));
      if (pred(id, key)) {
        kp[0] = key;
        kp[idoff] = id;
        ++kp;
      }
    });
  } else {
    uint32_t total = 0;
    visit([&](uint32_t id, uint32_t key) { total += __popcll(__ballot(pred(id, key))); });
    uint32_t base = 0;
    if (lane == 0 && total) base = atomicAdd(count, total);
    base = __builtin_amdgcn_readfirstlane(base);
    if (base + total > cap) return;  // wave-uniform
    visit([&](uint32_t id, uint32_t key) {
      asm volatile("" : "+v"(key));
      const bool p = pred(id, key);
      const uint64_t bal = __ballot(p);
      if (p) {
        const uint32_t pos = base + lanes_below(bal);
        dkey[pos] = key;
        did[pos] = id;
      }
      base += __popcll(bal);
    });
  }
}

// Bitonic sort of P = W NT rank words (descending), W words per thread: word r
// of thread t is element i = t + NT r.  Strides of NT and more pair words of
// one thread, strides 64 .. NT/2 go through LDS (two buffers alternating, one
// barrier per step), smaller ones are lane exchanges.  The compare-exchange
// rule is the one of the other sorts.
template <int W>
struct WideSort {
  uint64_t w[W];
  uint64_t *xbuf;  // 2 W NT words
  int t;
  int phase = 0;

  template <int SIZE, int STRIDE>
  __device__ __forceinline__ void step() {
    if constexpr (STRIDE >= NT) {
      constexpr int S = STRIDE / NT;  // the partner word of the same thread
#pragma unroll
      for (int r = 0; r < W; ++r) {
        if constexpr (true) {
          if ((r & S) == 0) {
            const bool desc = ((t + NT * r) & SIZE) == 0;  // the lower element keeps the larger
            const uint64_t a = w[r], b = w[r + S];
            const uint64_t big = a > b ? a : b, small = a > b ? b : a;
            w[r] = desc ? big : small;
            w[r + S] = desc ? small : big;
          }
        }
      }
    } else {
      uint64_t *buf = xbuf + (phase & 1) * (W * NT);
      ++phase;
#pragma unroll
      for (int r = 0; r < W; ++r) buf[t + NT * r] = w[r];
      __syncthreads();
#pragma unroll
      for (int r = 0; r < W; ++r) {
        const int i = t + NT * r;
        const uint64_t p = buf[i ^ STRIDE];
        const bool keep_larger = ((i & STRIDE) == 0) == ((i & SIZE) == 0);
        w[r] = ((p > w[r]) == keep_larger) ? p : w[r];
      }
    }
  }

  // Stage SIZE: strides SIZE/2 .. 64 here, then 32 .. 1 inside each wave.
  template <int SIZE, int STRIDE = SIZE / 2>
  __device__ __forceinline__ void stage() {
    if constexpr (STRIDE >= 64) {
      step<SIZE, STRIDE>();
      stage<SIZE, STRIDE / 2>();
    } else {
#pragma unroll
      for (int r = 0; r < W; ++r) bitonic_word_stage<SIZE, (SIZE < 64 ? SIZE / 2 : 32)>(w[r], t + NT * r);
    }
  }
};

// The n (NT < n <= W NT) pairs of skey/sid in rank order: the first m ids to
// orow, then -1 up to k.  `xbuf` holds 2 W NT words and does not overlap
// skey/sid.
template <int W>
__device__ __forceinline__ void sort_wide(const uint32_t *skey, const uint32_t *sid, int n, int m, int k,
                          int *__restrict__ orow, uint64_t *xbuf) {
  WideSort<W> ws;
  ws.xbuf = xbuf;
  ws.t = threadIdx.x;
  const int t = ws.t;
#pragma unroll
  for (int r = 0; r < W; ++r) {
    const int i = t + NT * r;
    ws.w[r] = i < n ? rank_word(skey[i], sid[i]) : 0ull;  // padding: word 0, after every element
  }
  ws.template stage<2>();
  ws.template stage<4>();
  ws.template stage<8>();
  ws.template stage<16>();
  ws.template stage<32>();
  ws.template stage<64>();
  ws.template stage<128>();
  ws.template stage<256>();
  ws.template stage<512>();
  ws.template stage<1024>();
  ws.template stage<2048>();
  if constexpr (W >= 4) ws.template stage<4096>();
#pragma unroll
  for (int r = 0; r < W; ++r) {
    const int i = t + NT * r;
    if (i < m) orow[i] = int(~uint32_t(ws.w[r]));
  }
  for (int r = m + t; r < k; r += NT) orow[r] = -1;
}

// Exclusive prefix sum of v over the workgroup (NT threads) and the total.
// One barrier; `wsum` is NWAVES words of scratch.  Every thread must call it.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wsum, uint32_t &total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  const uint32_t ws = wave_incl_scan(lane < NWAVES ? wsum[lane] : 0u);
  total = __builtin_amdgcn_readlane(ws, NWAVES - 1);
  const uint32_t before = wave > 0 ? __builtin_amdgcn_readlane(ws, wave - 1) : 0u;
  return before + incl - v;
}

// Keys known to lie in [lo, hi].
struct KeyRange {
  uint32_t lo, hi;
};

// Buckets of the counting rank, and the most pairs it lets one bucket take.
constexpr int kRankBuckets = NT;
constexpr uint32_t kBucketCap = 64;

// Rank-order store of n <= NT (key, id) pairs (skey/sid in LDS) by counting
// instead of a sorting network: each pair goes to one of NT buckets by key
// (equal ranges of key values from the largest key down to the smallest, so
// every key of bucket b is larger than every key of bucket b + 1), one prefix
// sum over the bucket counts gives each bucket's first rank, and a pair's
// rank is that plus the number of larger rank words in its own bucket.  The
// pair of rank r < m stores its id at orow[r]; orow[m, k) gets -1.  Returns
// false, having stored nothing, when a bucket receives more than kBucketCap
// pairs (ties or near-ties in bulk): the caller then sorts with the network.
// Five barriers; every thread of the workgroup must call it.
__device__ __forceinline__ bool counting_rank_store(const uint32_t *skey, const uint32_t *sid, int n,
                                                    int m, int k, int *__restrict__ orow,
                                                    TopkShared &sh, bool known, KeyRange range) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const bool live = t < n;
  const uint32_t key = live ? skey[t] : 0u;
  const uint32_t id = live ? sid[t] : 0u;
  uint32_t *cnt = &sh.hsub[0][0];  // bucket counts, then each bucket's first rank
  uint32_t *wsum = cnt + kRankBuckets;
  uint32_t hi, lo;
  if (known) {
    // The candidates of one row: keys in [bound, row maximum]; the counts
    // and the flag were cleared when the row started.
    lo = range.lo;
    hi = range.hi;
  } else {
    hi = key;
    lo = live ? key : 0xFFFFFFFFu;
    hi = max(hi, lane_xor<1>(hi)); lo = min(lo, lane_xor<1>(lo));
    hi = max(hi, lane_xor<2>(hi)); lo = min(lo, lane_xor<2>(lo));
    hi = max(hi, lane_xor<4>(hi)); lo = min(lo, lane_xor<4>(lo));
    hi = max(hi, lane_xor<8>(hi)); lo = min(lo, lane_xor<8>(lo));
    hi = max(hi, lane_xor<16>(hi)); lo = min(lo, lane_xor<16>(lo));
    hi = max(hi, lane_xor<32>(hi)); lo = min(lo, lane_xor<32>(lo));
    if (lane == 0) {
      sh.wmin[wave] = lo;
      sh.wmax[wave] = hi;
    }
    cnt[t] = 0u;
    if (t == 0) sh.big = 0u;
    __syncthreads();
    hi = 0u;
    lo = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
      hi = max(hi, sh.wmax[w]);
      lo = min(lo, sh.wmin[w]);
    }
  }
  // Bucket of a key: (hi - key) >> shift, below kRankBuckets for every key in [lo, hi].
  const uint32_t span = hi - lo;
  const int shift = max(0, 32 - __builtin_clz(span | 1u) - 10);
  const uint32_t b = (hi - key) >> shift;
  uint32_t within = 0;
  if (live) {
    within = atomicAdd(&cnt[b], 1u);
    if (within >= kBucketCap) sh.big = 1u;
  }
  __syncthreads();
  if (sh.big) return false;
  uint32_t total;
  const uint32_t first = block_excl_scan(cnt[t], wsum, total);
  cnt[t] = first;
  uint64_t *sw = sh.wbuf;
  if (t < 4) sw[n + t] = 0ull;  // the rank loop reads up to three words past the last bucket
  __syncthreads();
  const uint64_t word = rank_word(key, id);
  uint32_t start = 0, end = 0;
  if (live) {
    start = cnt[b];
    end = b + 1 < uint32_t(kRankBuckets) ? cnt[b + 1] : uint32_t(n);
    sw[start + within] = word;
  }
  __syncthreads();
  if (live) {
    // Words past the bucket's end belong to later buckets (smaller keys) or
    // are the zero padding: comparing with them adds nothing.
    uint32_t r = start;
    for (uint32_t j = start; j < end; j += 4)
      r += uint32_t(sw[j] > word) + uint32_t(sw[j + 1] > word) + uint32_t(sw[j + 2] > word) +
           uint32_t(sw[j + 3] > word);
    if (r < uint32_t(m)) orow[r] = int(id);
  }
  for (int r = m + t; r < k; r += NT) orow[r] = -1;
  return true;
}

// The counting rank for NT < n <= W NT pairs (the winners of k > NT), W of
// them per thread (pair t + j NT for j < W): W NT buckets, each thread owning
// W consecutive ones in the prefix sum; the pairs are placed bucket by bucket
// in the candidates' area (free once the winners are gathered).  The rest as
// counting_rank_store.  Returns false, having stored nothing, when a bucket
// receives more than kBucketCap pairs.  Every thread must call it.
template <int W>
__device__ __forceinline__ bool counting_rank_store_wide(const uint32_t *skey, const uint32_t *sid,
                                                         int n, int m, int k,
                                                         int *__restrict__ orow, TopkShared &sh) {
  constexpr int NB = W * NT;  // <= the NWAVES * 256 words of hsub
  constexpr int LGNB = W == 2 ? 11 : 12;
  static_assert(NB <= NWAVES * 256 && (W == 2 || W == 4), "bucket counts live in hsub");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  uint32_t key[W], id[W];
  uint32_t hi = 0u, lo = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < W; ++j) {
    const int i = t + j * NT;
    const bool live = i < n;
    key[j] = live ? skey[i] : 0u;
    id[j] = live ? sid[i] : 0u;
    if (live) {
      hi = max(hi, key[j]);
      lo = min(lo, key[j]);
    }
  }
  hi = max(hi, lane_xor<1>(hi)); lo = min(lo, lane_xor<1>(lo));
  hi = max(hi, lane_xor<2>(hi)); lo = min(lo, lane_xor<2>(lo));
  hi = max(hi, lane_xor<4>(hi)); lo = min(lo, lane_xor<4>(lo));
  hi = max(hi, lane_xor<8>(hi)); lo = min(lo, lane_xor<8>(lo));
  hi = max(hi, lane_xor<16>(hi)); lo = min(lo, lane_xor<16>(lo));
  hi = max(hi, lane_xor<32>(hi)); lo = min(lo, lane_xor<32>(lo));
  uint32_t *cnt = &sh.hsub[0][0];  // bucket counts, then each bucket's first rank
  if (lane == 0) {
    sh.wmin[wave] = lo;
    sh.wmax[wave] = hi;
  }
#pragma unroll
  for (int j = 0; j < W; ++j) cnt[t + j * NT] = 0u;
  if (t == 0) sh.big = 0u;
  __syncthreads();
  hi = 0u;
  lo = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    hi = max(hi, sh.wmax[w]);
    lo = min(lo, sh.wmin[w]);
  }
  const uint32_t span = hi - lo;
  const int shift = max(0, 32 - __builtin_clz(span | 1u) - LGNB);
  uint32_t b[W], within[W];
#pragma unroll
  for (int j = 0; j < W; ++j) {
    b[j] = (hi - key[j]) >> shift;
    within[j] = 0u;
    if (t + j * NT < n) {
      within[j] = atomicAdd(&cnt[b[j]], 1u);
      if (within[j] >= kBucketCap) sh.big = 1u;
    }
  }
  __syncthreads();
  if (sh.big) return false;
  uint32_t c[W], local = 0u;
#pragma unroll
  for (int j = 0; j < W; ++j) {
    c[j] = cnt[W * t + j];
    local += c[j];
  }
  uint32_t total;
  uint32_t first = block_excl_scan(local, sh.wsum, total);
#pragma unroll
  for (int j = 0; j < W; ++j) {
    cnt[W * t + j] = first;
    first += c[j];
  }
  uint64_t *sw = sh.cu.xbuf;  // CAP words >= n + 3
  if (t < 4) sw[n + t] = 0ull;  // the rank loop reads up to three words past the last bucket
  __syncthreads();
  uint32_t start[W], end[W];
  uint64_t word[W];
#pragma unroll
  for (int j = 0; j < W; ++j) {
    word[j] = rank_word(key[j], id[j]);
    start[j] = end[j] = 0u;
    if (t + j * NT < n) {
      start[j] = cnt[b[j]];
      end[j] = b[j] + 1 < uint32_t(NB) ? cnt[b[j] + 1] : uint32_t(n);
      sw[start[j] + within[j]] = word[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < W; ++j) {
    if (t + j * NT < n) {
      uint32_t r = start[j];
      for (uint32_t q = start[j]; q < end[j]; q += 4)
        r += uint32_t(sw[q] > word[j]) + uint32_t(sw[q + 1] > word[j]) +
             uint32_t(sw[q + 2] > word[j]) + uint32_t(sw[q + 3] > word[j]);
      if (r < uint32_t(m)) orow[r] = int(id[j]);
    }
  }
  for (int r = m + t; r < k; r += NT) orow[r] = -1;
  return true;
}

// Rank-order sort of the n (key, id) pairs in LDS arrays skey/sid, then the
// store of one row of ids: the first m in rank order, then -1 up to k.
// `wbuf` is 2 NT words of LDS scratch; `xbuf`, 2 MAXK words, is used only
// for n > NT and must not overlap skey/sid.  Every thread of the workgroup
// must call it.
__device__ __forceinline__ void sort_and_store(uint32_t *skey, uint32_t *sid, int n, int m, int k,
                               int *__restrict__ orow, TopkShared &sh, uint64_t *xbuf,
                               bool try_count = true, bool known = false,
                               KeyRange range = KeyRange{0u, 0u}) {
  const int t = threadIdx.x;
  uint64_t *wbuf = sh.wbuf;
  int P = 1;
  while (P < n) P <<= 1;
  if (P <= NT) {
    if (try_count && counting_rank_store(skey, sid, n, m, k, orow, sh, known, range)) return;
    // One rank word per thread (padding: word 0, after every element).
    // Strides below 64 exchange inside the wave, larger strides through LDS.
    // Waves past the P elements only keep the barriers.
    const bool busy = (t & ~63) < P;  // wave-uniform
    uint64_t w = t < n ? rank_word(skey[t], sid[t]) : 0ull;
    // Cross-wave steps alternate between two buffers, so each needs one
    // barrier: a buffer is rewritten two steps after it was read, and every
    // thread has passed the step in between.
    int phase = 0;
    auto lds_step = [&](int size, int stride) {
      uint64_t *buf = wbuf + (phase & 1) * NT;
      ++phase;
      if (busy) buf[t] = w;
      __syncthreads();
      if (busy) {
        const uint64_t p = buf[t ^ stride];
        const bool keep_larger = ((t & stride) == 0) == ((t & size) == 0);
        w = ((p > w) == keep_larger) ? p : w;
      }
    };
    // Stages 2..64 run whole inside each wave; later stages start with their
    // cross-wave strides, then finish with the in-wave ones.
    if (busy) {
      if (P >= 2) bitonic_word_stage<2, 1>(w, t);
      if (P >= 4) bitonic_word_stage<4, 2>(w, t);
      if (P >= 8) bitonic_word_stage<8, 4>(w, t);
      if (P >= 16) bitonic_word_stage<16, 8>(w, t);
      if (P >= 32) bitonic_word_stage<32, 16>(w, t);
      if (P >= 64) bitonic_word_stage<64, 32>(w, t);
    }
    if (P >= 128) {
      lds_step(128, 64);
      if (busy) bitonic_word_stage<128, 32>(w, t);
    }
    if (P >= 256) {
      lds_step(256, 128);
      lds_step(256, 64);
      if (busy) bitonic_word_stage<256, 32>(w, t);
    }
    if (P >= 512) {
      lds_step(512, 256);
      lds_step(512, 128);
      lds_step(512, 64);
      if (busy) bitonic_word_stage<512, 32>(w, t);
    }
    if (P >= 1024) {
      lds_step(1024, 512);
      lds_step(1024, 256);
      lds_step(1024, 128);
      lds_step(1024, 64);
      bitonic_word_stage<1024, 32>(w, t);
    }
    if (t < m) orow[t] = int(~uint32_t(w));
    for (int r = m + t; r < k; r += NT) orow[r] = -1;
    return;
  }
  // P in (NT, MAXK]: W = P / NT words per thread.
  if (P == 2 * NT) {
    if (try_count && counting_rank_store_wide<2>(skey, sid, n, m, k, orow, sh)) return;
    sort_wide<2>(skey, sid, n, m, k, orow, xbuf);
  } else {
    if (try_count && counting_rank_store_wide<4>(skey, sid, n, m, k, orow, sh)) return;
    sort_wide<4>(skey, sid, n, m, k, orow, xbuf);
  }
}

// Register slots of width PER that lie inside every row the dispatcher gives
// that width: rows longer than (next smaller width + 1) * NT.
constexpr int topk_full_slots(int per) {
  return per >= 64 ? 48 : per >= 47 ? 33 : per >= 32 ? 24 : per >= 23 ? 16 : per >= 15 ? 8
       : per >= 7 ? 4 : per >= 3 ? 2 : per >= 1 ? 1 : 0;
}

template <int PER>
struct RowKeys {
  uint32_t key[PER > 0 ? PER : 1];
};

// Selects one row with the whole workgroup (NT threads): srow[0, A) -> the
// k ids of orow.  Every thread of the workgroup must call it.
template <int PER>
__device__ __forceinline__ void topk_row(const float *__restrict__ srow, int A, int k,
                                         int *__restrict__ orow, TopkShared &sh) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int m = min(k, A);
  // Up to 32 register slots per thread the leaner per-slot code fits the
  // register file; the wider rows keep the code that needs fewer registers.
  constexpr bool kLean = PER >= 0 && PER <= 32;

  if (m == 0) {  // no active blocks: every slot is padding
    for (int r = t; r < k; r += NT) orow[r] = -1;
    return;
  }

  for (int i = t; i < NWAVES * 256; i += NT) (&sh.hsub[0][0])[i] = 0;
  if (t == 0) {
    sh.ncand = 0;
    sh.nwin = 0;
    sh.big = 0;
  }

  // Raw buffer loads: the hardware returns 0 past the row end, so every
  // slot's load is issued unconditionally and in flight together.
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)srow, 0, A * 4, 0x00020000);
  auto load_key = [&](int id) -> uint32_t {
    const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(rs, id * 4, 0, 0);
    return id < A ? score_key(u) : 0u;
  };

  // Thread t owns ids t + j*NT: slots j < PER in VGPRs, slot PER in LDS
  // (sh.extra[t]), so a row of (PER+1)*NT ids needs only PER registers -- the
  // capacity-sized rows of 2^n + 2 blocks spill just two ids into the extra
  // slot.  Slots past the row end hold the sentinel key 0: it never passes
  // the candidate bound, never matches a threshold (real keys are >= 1), and
  // the n_sentinel of them are taken out of bin 0 while the prefix is still 0.
  RowKeys<PER> rk;
  uint32_t n_sentinel = 0;
  if constexpr (PER >= 0) {
    n_sentinel = uint32_t((PER + 1) * NT - A);
    // Slots below kFull hold ids inside every row this width is chosen for
    // (the dispatcher takes the smallest width that holds the row, so the
    // row is longer than the next smaller width's slots): no id check there,
    // and their loads take the slot's offset from a scalar register (one
    // vector offset for all of them instead of one vector add per slot).
    constexpr int kFull = kLean ? topk_full_slots(PER) : 0;
    const bool full = kFull > 0 && A >= kFull * NT;  // workgroup-uniform; always true from the dispatcher
    if (full) {
#pragma unroll
      for (int j = 0; j < PER; ++j)
        rk.key[j] = j < kFull ? __builtin_amdgcn_raw_buffer_load_b32(rs, t * 4, j * NT * 4, 0)
                              : __builtin_amdgcn_raw_buffer_load_b32(rs, (j * NT + t) * 4, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) rk.key[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, (j * NT + t) * 4, 0, 0);
    }
    uint32_t xr = __builtin_amdgcn_raw_buffer_load_b32(rs, (PER * NT + t) * 4, 0, 0);
    // All loads first (raw bits), then the transform: the empty asm makes each
    // loaded value live unconditionally, so the compiler cannot sink a load
    // into the id < A branch and wait on it there.
    if (full) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        asm volatile("" : "+v"(rk.key[j]));
        rk.key[j] = (j < kFull || j * NT + t < A) ? score_key(rk.key[j]) : 0u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        asm volatile("" : "+v"(rk.key[j]));
        rk.key[j] = j * NT + t < A ? score_key(rk.key[j]) : 0u;
      }
    }
    asm volatile("" : "+v"(xr));
    sh.extra[t] = PER * NT + t < A ? score_key(xr) : 0u;
  } else {
    n_sentinel = uint32_t((A + NT - 1) / NT * NT - A);
  }
  // Visit every (id, key) this thread owns, sentinel slots included, with all
  // lanes active.  The empty asm hides that `tv` equals t, so ids are
  // recomputed in each visit (one add) instead of being hoisted into PER more
  // live registers; the scheduling barriers keep the compiler from hoisting
  // every slot's wave-wide masks ahead of their use (scalar-register spills).
  auto visit_row = [&](auto &&f) {
    int tv = t;
    asm volatile("" : "+v"(tv));
    if constexpr (PER >= 0) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        f(uint32_t(j * NT + tv), rk.key[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
      f(uint32_t(PER * NT + tv), sh.extra[tv]);
    } else {
      for (int base = 0; base < A; base += NT) f(uint32_t(base + tv), load_key(base + tv));
    }
  };
  // No barrier here when the bound is taken: a thread reads back only its own
  // extra slot, and the bound's barrier below orders the cleared histograms
  // and counters before any use, so each wave starts on its keys as soon as
  // its own loads arrive.
  const bool take_bound = k < A && k <= 4 * NT;  // workgroup-uniform
  if (!take_bound) __syncthreads();

  // Candidate bound.  Every thread's two (k > NT: four) largest keys over its
  // own slots are distinct elements of the row (or sentinels).  Each wave
  // finds the kw-th largest, kw = ceil(k / 16), of its 128 (256) such values
  // (a bisection on the key bits with wave ballots, cheaper than sorting
  // them): at least kw elements of the wave are >= it.  The smallest of the 16 wave values is
  // then exceeded-or-equalled by at least 16 * kw >= k elements, so it is <=
  // the k-th largest key and every winner lies at or above it.  (With one
  // value per thread the bound sat lower: about 3 % of an N(0,1) row passed
  // it and one row in ten overflowed the direct sort; with two, about 2 %.)
  // Beyond k = 4 NT the bound is 1: every real key is a candidate.
  uint32_t bound = 1u;
  KeyRange range{0u, 0u};  // the candidates' keys, set with the bound
  bool ranged = false;
  if (take_bound) {
    // Up to k = NT each thread keeps its two largest keys, beyond that its
    // four (kw <= 64 or 256 values of the wave are then enough).
    const bool four = k > NT;  // workgroup-uniform
    uint32_t v0 = 0u, v1 = 0u, v2 = 0u, v3 = 0u;  // this thread's largest keys, descending
    // The median of three: with v0 >= v1 the new second largest is
    // med3(v0, x, v1); the compiler emits one v_med3_u32 for this form.
    auto med3 = [](uint32_t a, uint32_t b, uint32_t c) { return max(min(a, b), min(max(a, b), c)); };
    auto take2 = [&](uint32_t x) {
      v1 = med3(v0, x, v1);
      v0 = max(v0, x);
    };
    auto take4 = [&](uint32_t x) {
      v3 = med3(v2, x, v3);
      v2 = med3(v1, x, v2);
      take2(x);
    };
    if constexpr (PER >= 0) {
      if (four) {
#pragma unroll
        for (int j = 0; j < PER; ++j) take4(rk.key[j]);
        take4(sh.extra[t]);
      } else {
#pragma unroll
        for (int j = 0; j < PER; ++j) take2(rk.key[j]);
        take2(sh.extra[t]);
      }
    } else {
      for (int base = 0; base < A; base += NT) {
        const uint32_t x = load_key(base + t);
        if (four) take4(x);
        else take2(x);
      }
    }
    // The wave's kw-th largest of its 128 (or 256) values, bit by bit from
    // the top: the largest x with at least kw values >= x (counted with wave
    // ballots; x stays wave-uniform).  Only the top 16 key bits are settled
    // (sign, exponent and 7 mantissa bits of the score): the low bits stay 0,
    // so the offer is at most the kw-th value -- still a valid bound, about 2 %
    // more candidates, half the steps.
    const int kw = (k + NWAVES - 1) / NWAVES;
    uint32_t vw = 0u;
    for (int bit = 31; bit >= 16; --bit) {
      const uint32_t c = vw | (1u << bit);
      uint32_t n = uint32_t(__popcll(__ballot(v0 >= c))) + uint32_t(__popcll(__ballot(v1 >= c)));
      if (four) n += uint32_t(__popcll(__ballot(v2 >= c))) + uint32_t(__popcll(__ballot(v3 >= c)));
      if (n >= uint32_t(kw)) vw = c;
    }
    // The row's largest key (each thread's largest is v0).
    uint32_t mx = v0;
    mx = max(mx, lane_xor<1>(mx));
    mx = max(mx, lane_xor<2>(mx));
    mx = max(mx, lane_xor<4>(mx));
    mx = max(mx, lane_xor<8>(mx));
    mx = max(mx, lane_xor<16>(mx));
    mx = max(mx, lane_xor<32>(mx));
    if (lane == 0) {
      sh.wmin[wave] = vw;
      sh.wmax[wave] = mx;
    }
    __syncthreads();
    uint32_t b = 0xFFFFFFFFu;
    mx = 0u;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
      b = min(b, sh.wmin[w]);
      mx = max(mx, sh.wmax[w]);
    }
    bound = max(b, 1u);
    range.lo = bound;
    range.hi = max(mx, bound);
    ranged = true;
  }

  compact<kLean>(visit_row, [&](uint32_t, uint32_t key) { return key >= bound; }, &sh.ncand, sh.cu.c.ckey,
          sh.cu.c.cid, CAP, [&] { asm volatile("" : "+v"(bound)); });
  __syncthreads();
  const uint32_t C = sh.ncand;

  if (C <= uint32_t(NT)) {
    // Few candidates (the usual case): sort them all into rank order and
    // keep the first m -- every winner is a candidate.
    sort_and_store(sh.cu.c.ckey, sh.cu.c.cid, int(C), m, k, orow, sh, nullptr, true, ranged,
                   range);
    return;
  }
  bool try_count = true;
  if (C <= uint32_t(CAP)) {
    // Select among the LDS candidates (all of them when k >= C).
    const uint32_t padC = (C + NT - 1) / NT * NT;
    auto visit_cand = [&](auto &&f) {
      for (uint32_t i = t; i < padC; i += NT) {
        const bool ok = i < C;
        f(ok ? sh.cu.c.cid[i] : 0u, ok ? sh.cu.c.ckey[i] : 0u);
      }
    };
    // Rows of up to 32 x 4096 blocks resolve a tie at the threshold with a
    // bitmap of the tied ids in the sort's exchange words (free until the
    // sort): one pass of atomic ORs and one prefix sum instead of up to three
    // radix passes over the ids, and the tied winners leave in id order with
    // no sorting; only the keys above the tie are ranked.
    uint32_t *tbits = reinterpret_cast<uint32_t *>(sh.wbuf);
    constexpr int kTieWordsPerThread = int(sizeof(sh.wbuf)) / 4 / NT;
    const bool tie_bitmap = A <= 32 * kTieWordsPerThread * NT;  // workgroup-uniform
    const int nbw = (A + 31) / 32;
    if (tie_bitmap)  // cleared here; the select's barriers order it before use
      for (int w = t; w < nbw; w += NT) tbits[w] = 0u;
    Threshold th;
    if (uint32_t(k) < C) th = radix_select(sh, visit_cand, uint32_t(k), padC - C, A, tie_bitmap);
    if (th.by_id && tie_bitmap) {
      const uint32_t T = th.pref;  // the whole threshold key
      visit_cand([&](uint32_t id, uint32_t key) {
        if (key == T && key != 0u) atomicOr(&tbits[id >> 5], 1u << (id & 31u));
      });
      compact<kLean>(visit_cand, [&](uint32_t, uint32_t key) { return key > T; }, &sh.nwin, sh.bkey,
                     sh.bid, MAXK);
      __syncthreads();
      const int nabove = int(sh.nwin);  // = k - th.tied: they take ranks [0, nabove)
      // Thread t owns bitmap words [W t, W t + W): ids in ascending order
      // across the threads; the tied winners are the first th.tied set bits.
      uint32_t wv[kTieWordsPerThread];
      uint32_t cnt = 0;
#pragma unroll
      for (int j = 0; j < kTieWordsPerThread; ++j) {
        const int w = kTieWordsPerThread * t + j;
        wv[j] = w < nbw ? tbits[w] : 0u;
        cnt += uint32_t(__popc(wv[j]));
      }
      uint32_t total;
      uint32_t p = block_excl_scan(cnt, sh.wsum, total);
#pragma unroll
      for (int j = 0; j < kTieWordsPerThread; ++j) {
        uint32_t x = wv[j];
        while (x != 0u && p < th.tied) {
          const uint32_t b = uint32_t(__builtin_ctz(x));
          x &= x - 1u;
          orow[nabove + int(p)] = int(uint32_t(kTieWordsPerThread * t + j) * 32u + b);
          ++p;
        }
      }
      __syncthreads();  // the bitmap is read; the sort may reuse its words
      // A row tied in bulk at its threshold is usually tied in bulk above it
      // too, where the counting rank would refuse a bucket (about a
      // microsecond lost): rank the keys above with the network directly.
      if (nabove > 0)
        sort_and_store(sh.bkey, sh.bid, nabove, nabove, nabove, orow, sh, sh.cu.xbuf, false);
      return;
    }
    compact<kLean>(visit_cand, [&](uint32_t id, uint32_t key) { return key != 0u && th.wins(id, key); },
            &sh.nwin, sh.bkey, sh.bid, MAXK);
    try_count = !th.by_id && th.tied <= kBucketCap;
  } else {
    // Too many candidates for LDS: select over the whole row.
    const Threshold th = radix_select(sh, visit_row, uint32_t(k), n_sentinel, A);
    compact<kLean>(visit_row, [&](uint32_t id, uint32_t key) { return key != 0u && th.wins(id, key); },
            &sh.nwin, sh.bkey, sh.bid, MAXK);
    try_count = !th.by_id && th.tied <= kBucketCap;
  }
  __syncthreads();
  // A select that had to split the keys equal to its threshold by id met
  // ties in bulk, and winners that share one key share one bucket of the
  // counting rank: past its cap, go straight to the network (a failed
  // attempt costs about a microsecond on rows of thousand-way ties).
  sort_and_store(sh.bkey, sh.bid, m, m, k, orow, sh, sh.cu.xbuf, try_count);
}

template <int PER>
__global__ __launch_bounds__(NT) void topk_kernel(const float *__restrict__ scores, int A, int k,
                                                  int *__restrict__ ids) {
  __shared__ TopkShared sh;
  topk_row<PER>(scores + int64_t(blockIdx.x) * A, A, k, ids + int64_t(blockIdx.x) * k, sh);
}

// ---------------------------------------------------------------------------
// Few-row top-k across the whole GPU.
//
// One row of tens of thousands of scores on one workgroup leaves 255 of 256
// CUs idle and takes a chain of barriers.  With few rows (decode), the row is
// instead cut into groups of GS = 64 E scores (one wave each) and selected in
// two launches, with no cross-workgroup synchronisation inside a launch:
//
//   1. group_tops_kernel: every group publishes its M best elements, exactly,
//      as rank words rw = key << 32 | ~id (a larger word ranks first; 0 is an
//      empty slot).
//   2. wide_rank_kernel (NB workgroups per row, each doing the same first
//      steps):
//      a. a bound: the k-th largest key among the published words lies in
//         some 4096-bin (top 12 bits) histogram bin; B = that bin's lower
//         edge.  At least k published elements -- distinct row elements --
//         have key >= B, so every element of the row's top k has key >= B.
//      b. the candidates, all elements with key >= B: a group whose M-th
//         published word is below B ("complete") has all of them among its
//         published words; the few other groups ("rich") are re-read from
//         the scores.
//      c. exact ranks: a candidate's rank is the number of candidates whose
//         rank word is larger (every element that outranks a candidate is a
//         candidate).  The candidate list is built in the same order by
//         every workgroup (prefix sums, no atomics); workgroup j ranks the
//         j-th of NB slices of it and writes id to ids[rank] when rank < k.
//   If the candidates overflow LDS (mass ties at the bound), workgroup 0 of
//   the row runs the one-workgroup selection on the row instead; the result
//   is the same.
// ---------------------------------------------------------------------------
constexpr int WIDE_CCAP = 8192;   // LDS candidate capacity
constexpr int WIDE_UCAP = kWideMaxWordsPerRow;  // published words per row, at most
constexpr int WIDE_GCAP = WIDE_UCAP / 4;  // groups per row, at most (each publishes >= 4)
constexpr int WIDE_RCAP = 1024;   // rich groups listed (more: the one-workgroup fallback)

// Rank workgroups per row: the exact-rank step costs about C^2 / NB word
// comparisons per workgroup for C ~ k candidates, so NB grows with k (16 at
// k <= 512, 128 at k = 4096) and every workgroup's share stays the same.
int wide_nb(int k) {
  int nb = 16;
  while (nb < 128 && nb * 32 < k) nb *= 2;
  return nb;
}


// Wave maximum of a rank word held as (key, ~id) halves, using lane_xor
// (DPP within rows of 16 lanes).
__device__ __forceinline__ uint64_t wave_max_word(uint64_t v) {
  uint32_t k = uint32_t(v >> 32), i = uint32_t(v);
  auto step = [&](uint32_t pk, uint32_t pi) {
    const bool take = (pk > k) | ((pk == k) & (pi > i));
    k = take ? pk : k;
    i = take ? pi : i;
  };
  step(lane_xor<1>(k), lane_xor<1>(i));
  step(lane_xor<2>(k), lane_xor<2>(i));
  step(lane_xor<4>(k), lane_xor<4>(i));
  step(lane_xor<8>(k), lane_xor<8>(i));
  step(lane_xor<16>(k), lane_xor<16>(i));
  step(lane_xor<32>(k), lane_xor<32>(i));
  return (uint64_t(k) << 32) | i;
}

// Group g of row blockIdx.y holds ids [g*GS, g*GS + GS); lane l owns ids
// g*GS + l + 64i (i < E): each load instruction reads 256 contiguous bytes,
// and ids past the row end read as empty (a hardware-bounded buffer load of
// a dword past the row returns 0, and the id test discards it).  With E = 1
// the wave sorts its 64 elements in rank order (a bitonic network on lane
// exchanges) and lanes 0 .. M-1 hold the group's best; with E > 1 it takes
// the maximum M times, removing each winner.
template <int E>
__global__ __launch_bounds__(256) void group_tops_kernel(const float *__restrict__ scores, int A,
                                                         int ngroups, int M,
                                                         uint64_t *__restrict__ tops) {
  constexpr int GS = 64 * E;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= ngroups) return;  // wave-uniform; no barriers in this kernel
  const int row = blockIdx.y;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(scores + int64_t(row) * A), 0, A * 4, 0x00020000);
  uint32_t raw[E];
#pragma unroll
  for (int i = 0; i < E; ++i)
    raw[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, uint32_t(g * GS + lane + 64 * i) * 4u, 0, 0);
  uint64_t *dst = tops + (int64_t(row) * ngroups + g) * M;
  if constexpr (E == 1) {
    const uint32_t id = uint32_t(g * GS + lane);
    publish_group_tops(id < uint32_t(A) ? score_key(raw[0]) : 0u, id, M, dst);
  } else {
    uint64_t v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t id = uint32_t(g * GS + lane + 64 * i);
      v[i] = id < uint32_t(A) ? rank_word(score_key(raw[i]), id) : 0ull;
    }
    uint64_t mine = 0;
    for (int m = 0; m < M; ++m) {
      uint64_t best = v[0];
#pragma unroll
      for (int i = 1; i < E; ++i) best = v[i] > best ? v[i] : best;
      best = wave_max_word(best);
      if (best == 0) break;  // the group is exhausted; the rest stay empty
      if (lane == m) mine = best;
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = v[i] == best ? 0ull : v[i];  // ids are distinct
    }
    if (lane < M) dst[lane] = mine;
  }
}

struct WideShared {
  uint32_t hist[4096];
  uint32_t lastk[WIDE_GCAP];  // each group's M-th published key
  uint64_t cand[WIDE_CCAP];
  uint32_t rich[WIDE_RCAP];
  uint32_t wsum[NWAVES];
  uint32_t nvalid, bound;
};

union WideLds {
  WideShared w;
  TopkShared row;
};


template <int E, int WPT>
__global__ __launch_bounds__(NT) void wide_rank_kernel(const float *__restrict__ scores, int A,
                                                       int k, int *__restrict__ ids,
                                                       const uint64_t *__restrict__ tops,
                                                       int ngroups, int M) {
  constexpr int GS = 64 * E;
  __shared__ WideLds lds;
  WideShared &sh = lds.w;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int row = blockIdx.y;
  const float *srow = scores + int64_t(row) * A;
  int *orow = ids + int64_t(row) * k;
  const uint64_t *trow = tops + int64_t(row) * ngroups * M;
  const int U = ngroups * M;  // <= WIDE_UCAP (the launcher sizes M)
  const int m = min(k, A);

  for (int i = t; i < 4096; i += NT) sh.hist[i] = 0;
  if (t == 0) sh.nvalid = 0;
  // The published words, read once (their loads all in flight), WPT per
  // thread (WPT * NT >= U).
  uint64_t wv[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int e = t + i * NT;
    wv[i] = e < U ? trow[e] : 0ull;
  }
  __syncthreads();

  // (a) the bound: histogram of the published keys' top 12 bits, then the
  // bin where the count from the top reaches k.  Each group's M-th key goes
  // to LDS for (b).
  const int lgM = __builtin_ctz(uint32_t(M));  // M is a power of two
  uint32_t nv = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int e = t + i * NT;
    if (e >= U) break;
    const uint32_t key = uint32_t(wv[i] >> 32);
    if ((e & (M - 1)) == M - 1) sh.lastk[e >> lgM] = key;
    if (key) {
      atomicAdd(&sh.hist[key >> 20], 1u);
      ++nv;
    }
  }
  nv = wave_sum(nv);
  if (lane == 0 && nv) atomicAdd(&sh.nvalid, nv);
  __syncthreads();
  // Thread t owns bins [4096 - 4(t+1), 4096 - 4t); an exclusive prefix over
  // threads counts the published keys in higher bins.
  uint32_t c4 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) c4 += sh.hist[4095 - 4 * t - i];
  if (t == 0) sh.bound = 1u;  // fewer than k published keys: every real key qualifies
  uint32_t nvalid_total;
  uint32_t run = block_excl_scan(c4, sh.wsum, nvalid_total);
  if (sh.nvalid >= uint32_t(k)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4095 - 4 * t - i;
      const uint32_t hb = sh.hist[b];
      if (run < uint32_t(k) && run + hb >= uint32_t(k)) sh.bound = uint32_t(b) << 20;
      run += hb;
    }
  }
  __syncthreads();
  const uint32_t B = max(sh.bound, 1u);

  // (b) candidates, in an order every workgroup of the row agrees on: the
  // published words >= B of complete groups (thread order, then slot
  // order), then the elements >= B of the rich groups.
  bool take[WPT], rich[WPT];
  uint32_t ntake = 0, nrich = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int e = t + i * NT;
    take[i] = rich[i] = false;
    if (e < U) {
      const int g = e >> lgM;
      const uint32_t last = sh.lastk[g];
      const bool complete = last < B;
      take[i] = complete && uint32_t(wv[i] >> 32) >= B;
      rich[i] = !complete && (e == (g << lgM));
    }
    ntake += take[i];
    nrich += rich[i];
  }
  uint32_t total;
  const uint32_t off = block_excl_scan(ntake | (nrich << 16), sh.wsum, total);
  const uint32_t C0 = total & 0xFFFFu, nr = total >> 16;
  uint32_t oc = off & 0xFFFFu, orr = off >> 16;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    if (take[i]) {
      if (oc < uint32_t(WIDE_CCAP)) sh.cand[oc] = wv[i];
      ++oc;
    }
    if (rich[i]) {
      if (orr < uint32_t(WIDE_RCAP)) sh.rich[orr] = uint32_t((t + i * NT) >> lgM);
      ++orr;
    }
  }
  uint32_t C = C0;
  if (nr > 0 && nr <= uint32_t(WIDE_RCAP) && C0 <= uint32_t(WIDE_CCAP)) {
    __syncthreads();
    // every element of the rich groups, thread t taking t, t + NT, ...
    const uint32_t nel = nr * GS;
    constexpr int RPT = 8;  // elements per thread per pass
    for (uint32_t base = 0; base < nel; base += RPT * NT) {
      uint64_t x[RPT];
      uint32_t c = 0;
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const uint32_t i = base + uint32_t(t) + uint32_t(r) * NT;
        x[r] = 0;
        if (i < nel) {
          const uint32_t id = sh.rich[i / GS] * GS + (i % GS);
          if (id < uint32_t(A)) {
            const uint32_t key = score_key(__float_as_uint(srow[id]));
            if (key >= B) x[r] = rank_word(key, id);
          }
        }
        c += x[r] != 0;
      }
      uint32_t added;
      uint32_t o = C + block_excl_scan(c, sh.wsum, added);
#pragma unroll
      for (int r = 0; r < RPT; ++r)
        if (x[r] != 0) {
          if (o < uint32_t(WIDE_CCAP)) sh.cand[o] = x[r];
          ++o;
        }
      C += added;
      __syncthreads();  // wsum is reused by the next pass
    }
  }
  __syncthreads();

  if (C > uint32_t(WIDE_CCAP) || nr > uint32_t(WIDE_RCAP)) {
    // Mass ties at the bound: one workgroup selects the row exactly.
    if (blockIdx.x == 0) topk_row<-1>(srow, A, k, orow, lds.row);
    return;
  }

  // (c) exact ranks of candidates [C*j/NB, C*(j+1)/NB) for workgroup j.  A
  // wave takes four at a time; its lanes read the list 64 words at a time
  // and compare each word with all four.
  const uint32_t c_lo = C * blockIdx.x / gridDim.x, c_hi = C * (blockIdx.x + 1) / gridDim.x;
  const int wave = t >> 6;
  for (uint32_t i0 = c_lo + 4u * uint32_t(wave); i0 < c_hi; i0 += 4u * NWAVES) {
    uint64_t wc[4];
    uint32_t n[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      wc[c] = i0 + c < c_hi ? sh.cand[i0 + c] : ~0ull;
      n[c] = 0;
    }
    uint32_t j = uint32_t(lane);
    for (; j + 192 < C; j += 256) {
      const uint64_t a0 = sh.cand[j], a1 = sh.cand[j + 64], a2 = sh.cand[j + 128],
                     a3 = sh.cand[j + 192];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        n[c] += (a0 > wc[c] ? 1u : 0u) + (a1 > wc[c] ? 1u : 0u) + (a2 > wc[c] ? 1u : 0u) +
                (a3 > wc[c] ? 1u : 0u);
    }
    for (; j < C; j += 64) {
      const uint64_t a = sh.cand[j];
#pragma unroll
      for (int c = 0; c < 4; ++c) n[c] += a > wc[c] ? 1u : 0u;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t r = wave_sum(n[c]);
      if (lane == 0 && i0 + c < c_hi && r < uint32_t(k)) orow[r] = int(~uint32_t(wc[c]));
    }
  }
  if (blockIdx.x == 0)
    for (int r = m + t; r < k; r += NT) orow[r] = -1;
}

// The rank kernel with WPT = 8 words per thread when the row publishes at
// most 8192 (decode at k <= ~2048), else 16.
template <int E>
hipError_t launch_rank(const float *scores, int nq, int A, int k, int *ids, const uint64_t *tops,
                       int ngroups, int M, hipStream_t stream) {
  const dim3 grid(wide_nb(k), nq);
  if (ngroups * M <= 8 * NT)
    wide_rank_kernel<E, 8><<<grid, NT, 0, stream>>>(scores, A, k, ids, tops, ngroups, M);
  else
    wide_rank_kernel<E, WIDE_UCAP / NT><<<grid, NT, 0, stream>>>(scores, A, k, ids, tops, ngroups, M);
  return hipGetLastError();
}

template <int E>
hipError_t launch_wide(const float *scores, int nq, int A, int k, int *ids, hipStream_t stream,
                       ScratchFn scratch) {
  constexpr int GS = 64 * E;
  const int ngroups = (A + GS - 1) / GS;
  const int M = wide_words_per_group(ngroups, k);
  void *ws = nullptr;
  hipError_t e = scratch(stream, size_t(nq) * ngroups * M * sizeof(uint64_t), &ws);
  if (e != hipSuccess) return e;
  uint64_t *tops = static_cast<uint64_t *>(ws);
  group_tops_kernel<E><<<dim3((ngroups + 3) / 4, nq), 256, 0, stream>>>(scores, A, ngroups, M, tops);
  return launch_rank<E>(scores, nq, A, k, ids, tops, ngroups, M, stream);
}

template <int PER>
hipError_t launch_topk(const float *scores, int nq, int A, int k, int *ids, hipStream_t stream) {
  topk_kernel<PER><<<nq, NT, 0, stream>>>(scores, A, k, ids);
  return hipGetLastError();
}

}  // namespace

int wide_words_per_group(int ngroups, int k) {
  // A power of two: enough that the union holds about 4k elements, at least
  // 8 (a group then rarely holds more candidates than it publishes), at
  // most 64 and WIDE_UCAP in all.  Callers keep ngroups <= WIDE_UCAP / 4.
  int M = 8;
  while (M < 64 && M * ngroups < 4 * k) M *= 2;
  while (M > 1 && M * ngroups > WIDE_UCAP) M /= 2;
  return M;
}

hipError_t launch_wide_rank(const float *scores, int nq, int A, int k, int *ids,
                            const uint64_t *tops, int M, hipStream_t stream) {
  const int ngroups = (A + 63) / 64;
  return launch_rank<1>(scores, nq, A, k, ids, tops, ngroups, M, stream);
}

// Elements per group of the few-row top-k for a row of A scores (0: the row
// takes the one-workgroup path).  The group size grows with the row so that
// the published words stay within WIDE_UCAP (ngroups <= WIDE_UCAP / 4: every
// group publishes at least 4 words).
int wide_group_size(int nq, int A) {
  if (nq > kWideMaxRows || A <= 0 || A > 2048 * 1024) return 0;
  return A <= 2048 * 64 ? 64 : A <= 2048 * 256 ? 256 : 1024;
}

size_t select_scratch_bytes(int nq, int K, int A, int k) {
  if (nq <= 0 || A <= 0 || k <= 0) return 0;
  if (nq <= kWideMaxRows && A <= kWideMaxBlocksFused && gemv_fits(nq, K)) {
    const int ngroups = (A + 63) / 64;
    return size_t(nq) * ngroups * wide_words_per_group(ngroups, k) * sizeof(uint64_t);
  }
  const int gs = wide_group_size(nq, A);
  if (gs == 0) return 0;
  const int ngroups = (A + gs - 1) / gs;
  return size_t(nq) * ngroups * wide_words_per_group(ngroups, k) * sizeof(uint64_t);
}

hipError_t launch_block_topk(const float *scores, int nq, int A, int k, int *ids,
                             hipStream_t stream, ScratchFn scratch) {
  // Few rows: spread each row over the GPU.
  switch (wide_group_size(nq, A)) {
    case 64: return launch_wide<1>(scores, nq, A, k, ids, stream, scratch);
    case 256: return launch_wide<4>(scores, nq, A, k, ids, stream, scratch);
    case 1024: return launch_wide<16>(scores, nq, A, k, ids, stream, scratch);
    default: break;
  }
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
