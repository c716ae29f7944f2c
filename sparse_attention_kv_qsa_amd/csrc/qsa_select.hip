// Scores and top-k in one call: the dispatch of qsa_block_select.
#include <hip/hip_runtime.h>

#include "qsa_internal.h"

namespace qsa {

hipError_t launch_block_select(const float *q, const float *kblk, int nq, int K, int A, int k,
                               float *scores, int *ids, hipStream_t stream, ScratchFn scratch) {
  if (nq <= kWideMaxRows && A > 0 && A <= kWideMaxBlocksFused && gemv_fits(nq, K)) {
    const int ngroups = (A + 63) / 64;
    const int M = wide_words_per_group(ngroups, k);
    void *ws = nullptr;
    hipError_t e = scratch(stream, size_t(nq) * ngroups * M * sizeof(uint64_t), &ws);
    if (e != hipSuccess) return e;
    uint64_t *tops = static_cast<uint64_t *>(ws);
    e = launch_gemv_tops(q, kblk, nq, K, A, scores, tops, M, stream);
    if (e != hipSuccess) return e;
    return launch_wide_rank(scores, nq, A, k, ids, tops, M, stream);
  }
  hipError_t e = launch_block_scores(q, kblk, nq, K, A, scores, kScoresAuto, stream);
  if (e != hipSuccess) return e;
  return launch_block_topk(scores, nq, A, k, ids, stream, scratch);
}

}  // namespace qsa
