// Device helpers shared by the scoring and selection kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Order-preserving map of an fp32 score (given as its bits) to uint32: a
// larger score gives a larger key.  A score with the sign bit clear maps to
// u + 2^31 (its bits with the sign bit set); a negative one to 2^32 - u (the
// two's complement negation), which reverses the order of the magnitudes and
// sends -0.0 to 2^31, the key of +0.0.  The negative range lands on
// [1, 2^31], so key 0 stays free as the "no block" sentinel.  Three vector
// instructions (negate, sign test, select with the sign set by a source
// modifier).
__device__ __forceinline__ uint32_t score_key(uint32_t u) {
  return int32_t(u) < 0 ? 0u - u : (u | 0x80000000u);
}

// Rank word of a (key, id) pair: a larger word ranks first (larger key, or
// equal key and lower id).  0 is the empty word (key 0 is never a real key).
__device__ __forceinline__ uint64_t rank_word(uint32_t key, uint32_t id) {
  return (uint64_t(key) << 32) | uint64_t(~id);
}

// v of lane (lane ^ S) for a power of two S < 64.  Strides up to 8 stay on
// DPP (quad permutes, row shifts under bank masks, a row rotate); 16 and 32
// use gfx950's lane-swap instructions (v_permlane16_swap / v_permlane32_swap:
// with both operands x, lanes with the S bit set find the partner's value in
// the first result and the others in the second).  S must be a compile-time
// constant after unrolling: a runtime switch here costs a dozen scalar
// branches per exchange.
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  const int x = int(v);
  if constexpr (S == 1) {
    return uint32_t(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    return uint32_t(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  } else if constexpr (S == 4) {
    // banks 0 and 2 (lane bit 2 clear) read lane + 4, banks 1 and 3 read lane - 4
    const int r = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0x5, false);  // row_shl:4
    return uint32_t(__builtin_amdgcn_update_dpp(r, x, 0x114, 0xF, 0xA, false));  // row_shr:4
  } else if constexpr (S == 8) {
    return uint32_t(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));  // row_ror:8
  } else if constexpr (S == 16 || S == 32) {
    const auto r = S == 32 ? __builtin_amdgcn_permlane32_swap(v, v, false, false)
                           : __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & S) ? r[0] : r[1];
  } else {
    return uint32_t(__shfl_xor(x, S, 64));
  }
}

// One compare-exchange step of a bitonic network held one element per lane,
// for a partner in the same wave (STRIDE < 64).  `pos` is the element's
// position; blocks whose position has the SIZE bit clear run in rank order.
// Ties (identical pairs) never swap.
template <int SIZE, int STRIDE, class Before>
__device__ __forceinline__ void bitonic_lane_step(uint32_t &key, uint32_t &id, int pos,
                                                  Before &&before) {
  const uint32_t pk = lane_xor<STRIDE>(key);
  const uint32_t pi = lane_xor<STRIDE>(id);
  // Branch-free: both orders are evaluated and selected with bit operations
  // (a conditional here compiles to divergent branches on every step).
  const bool take_first = ((pos & STRIDE) == 0) == ((pos & SIZE) == 0);
  const bool take = (take_first & before(pk, pi, key, id)) | (!take_first & before(key, id, pk, pi));
  key = take ? pk : key;
  id = take ? pi : id;
}

// All steps of stage SIZE with strides below 64 (STRIDE = min(SIZE, 64) / 2 down to 1).
template <int SIZE, int STRIDE, class Before>
__device__ __forceinline__ void bitonic_lane_stage(uint32_t &key, uint32_t &id, int pos,
                                                   Before &&before) {
  if constexpr (STRIDE >= 1) {
    bitonic_lane_step<SIZE, STRIDE>(key, id, pos, before);
    bitonic_lane_stage<SIZE, STRIDE / 2>(key, id, pos, before);
  }
}

// Bitonic network over 64-bit rank words (a larger word ranks first), one per
// lane: stage SIZE's in-wave steps, strides min(SIZE, 64)/2 down to 1.  A
// lane whose position has the SIZE bit clear keeps the larger word of each
// pair when it is the pair's lower position, so those blocks end in
// descending order.
template <int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_word_stage(uint64_t &w, int pos) {
  if constexpr (STRIDE >= 1) {
    const uint32_t lo = lane_xor<STRIDE>(uint32_t(w));
    const uint32_t hi = lane_xor<STRIDE>(uint32_t(w >> 32));
    const uint64_t p = (uint64_t(hi) << 32) | lo;
    const bool keep_larger = ((pos & STRIDE) == 0) == ((pos & SIZE) == 0);
    w = ((p > w) == keep_larger) ? p : w;
    bitonic_word_stage<SIZE, STRIDE / 2>(w, pos);
  }
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP lane shifts:
// four shifts within each row of 16 lanes, then the row totals carried
// forward with row broadcasts (lane 15 -> row 1 and 3, lane 31 -> rows 2, 3).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = int(v);
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return uint32_t(x);
}

// Sum over the wave, the same in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

// Publishes the M (<= 64) best of 64 elements held one per lane (key 0 =
// empty slot): the wave sorts them in rank order with a bitonic network on
// lane exchanges, and lane m < M writes the m-th rank word to dst[m].
__device__ __forceinline__ void publish_group_tops(uint32_t key, uint32_t id, int M,
                                                   uint64_t *dst) {
  const int lane = threadIdx.x & 63;
  uint32_t nid = ~id;  // larger ~id = lower id = earlier in rank order
  auto first = [](uint32_t ka, uint32_t ia, uint32_t kb, uint32_t ib) {
    return (ka > kb) | ((ka == kb) & (ia > ib));
  };
  bitonic_lane_stage<2, 1>(key, nid, lane, first);
  bitonic_lane_stage<4, 2>(key, nid, lane, first);
  bitonic_lane_stage<8, 4>(key, nid, lane, first);
  bitonic_lane_stage<16, 8>(key, nid, lane, first);
  bitonic_lane_stage<32, 16>(key, nid, lane, first);
  bitonic_lane_stage<64, 32>(key, nid, lane, first);
  if (lane < M) dst[lane] = key ? (uint64_t(key) << 32) | nid : 0ull;
}

}  // namespace qsa
