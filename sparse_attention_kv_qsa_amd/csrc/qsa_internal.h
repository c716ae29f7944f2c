// Internal launch interface between the C ABI (qsa_api.hip) and the kernels.
// All launchers enqueue on `stream` and return hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Threads of one top-k workgroup (one query row per workgroup).
constexpr int kTopkThreads = 1024;
// Largest k the top-k kernels sort in LDS.
constexpr int kTopkMaxK = 4096;
// Queries at or below this count take the per-block dot-product scorer.
constexpr int kGemvMaxQueries = 8;

// Scores of nq queries against active_blocks summaries, K = heads*dim fp32
// elements each.  Chooses the bandwidth-bound dot-product kernel for small nq
// and the MFMA tile kernel otherwise.
hipError_t launch_block_scores(const float *q, const float *kblk, int nq, int K,
                               int active_blocks, float *scores, hipStream_t stream);

// Top-k ids per row of scores[nq][active_blocks]; k in [1, kTopkMaxK].
hipError_t launch_block_topk(const float *scores, int nq, int active_blocks, int k,
                             int *ids, hipStream_t stream);

}  // namespace qsa
