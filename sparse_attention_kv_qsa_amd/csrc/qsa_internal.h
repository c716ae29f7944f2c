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
// Rows at or below this count take the whole-GPU top-k (two launches, the
// row spread over many workgroups) instead of one workgroup per row.
constexpr int kWideMaxRows = 16;
// Queries at or below this count take the per-block dot-product scorer.
constexpr int kGemvMaxQueries = 8;
// Precision modes (the QSA_SCORES_* values of qsa.h).
constexpr int kScoresAuto = 0;
constexpr int kScoresFp32 = 1;
constexpr int kScoresBf16x3 = 2;
constexpr int kScoresF16x2 = 3;

// Scores of nq queries against active_blocks summaries, K = heads*dim fp32
// elements each, with the given precision mode (QSA_SCORES_* of qsa.h).
hipError_t launch_block_scores(const float *q, const float *kblk, int nq, int K,
                               int active_blocks, float *scores, int mode, hipStream_t stream);

// The same scores on bf16 matrix cores with the exact three-way split of each
// fp32 operand (six slice products; any nq).
hipError_t launch_block_scores_bf16x3(const float *q, const float *kblk, int nq, int K,
                                      int active_blocks, float *scores, hipStream_t stream);

// The same scores on fp16 matrix cores with a scaled two-piece split of each
// fp32 operand (three piece products; any nq).
hipError_t launch_block_scores_f16x2(const float *q, const float *kblk, int nq, int K,
                                     int active_blocks, float *scores, hipStream_t stream);

// fp32 scores: the dot-product kernel for nq <= kGemvMaxQueries (and K that
// fits its registers), else fp32 MFMA tiles.
hipError_t launch_block_scores_fp32(const float *q, const float *kblk, int nq, int K,
                                    int active_blocks, float *scores, hipStream_t stream);

// The device a stream belongs to (the null stream: the current device).
hipError_t stream_device(hipStream_t stream, int *dev);

// A source of device scratch: at least `bytes` bytes on the stream's device
// for work enqueued on `stream`.
typedef hipError_t (*ScratchFn)(hipStream_t stream, size_t bytes, void **ptr);

// The library's allocating source (qsa_workspace.hip): one growing buffer per
// (device, stream), so consecutive calls on one stream reuse it in stream
// order.
hipError_t workspace(hipStream_t stream, size_t bytes, void **ptr);

// The allocation-free source (qsa_noalloc.hip): one fixed static device array
// per GPU, shared by every call on that GPU; fails with hipErrorInvalidValue
// past kNoAllocScratchBytes.
hipError_t static_scratch(hipStream_t stream, size_t bytes, void **ptr);

// Top-k ids per row of scores[nq][active_blocks]; k in [1, kTopkMaxK].
hipError_t launch_block_topk(const float *scores, int nq, int active_blocks, int k,
                             int *ids, hipStream_t stream, ScratchFn scratch = workspace);

// Scores and top-k ids in one call (k >= 1).  For few queries whose scores
// take the dot-product kernel, the scorer also publishes each 64-block
// group's best rank words, so the selection needs one more launch instead
// of two; otherwise the two steps run as in separate calls.
hipError_t launch_block_select(const float *q, const float *kblk, int nq, int K,
                               int active_blocks, int k, float *scores, int *ids,
                               hipStream_t stream, ScratchFn scratch = workspace);

// Scratch bytes launch_block_select takes from its source for this call (0
// when none: many rows, k == 0 or no active block).
size_t select_scratch_bytes(int nq, int K, int active_blocks, int k);

// The few-row top-k publishes at most this many 8-byte words per row, so a
// select call needs at most kWideMaxRows * kWideMaxWordsPerRow * 8 bytes.
constexpr int kWideMaxWordsPerRow = 16384;
constexpr size_t kNoAllocScratchBytes = size_t(kWideMaxRows) * kWideMaxWordsPerRow * 8;

// Pieces of the fused path.  The whole-GPU top-k groups rows into 64-element
// groups that publish M rank words each (tops[nq][ngroups][M]).
constexpr int kWideMaxBlocksFused = 2048 * 64;  // groups of 64: ngroups <= 2048
bool gemv_fits(int nq, int K);
int wide_words_per_group(int ngroups, int k);
hipError_t launch_gemv_tops(const float *q, const float *kblk, int nq, int K, int A,
                            float *scores, uint64_t *tops, int M, hipStream_t stream);
hipError_t launch_wide_rank(const float *scores, int nq, int A, int k, int *ids,
                            const uint64_t *tops, int M, hipStream_t stream);

// Block-sparse decode attention (qsa_attn.hip): out[nq][heads][dim] from the
// cells of the blocks ids[nq][k] (-1 skipped) in kc/vc[cells][heads][dim],
// cells c < n_cells only.  dim in [4, kAttnMaxDim], a multiple of 4.
constexpr int kAttnMaxDim = 128;
bool attn_dim_ok(int dim);
hipError_t launch_sparse_decode_attention(const float *q, const float *kc, const float *vc,
                                          const int *ids, int nq, int heads, int dim, int k,
                                          int n_cells, float scale, float *out,
                                          hipStream_t stream);
// The same over an int8 pool: codes kq/vq[cells][heads][dim] int8, one
// binary16 scale per (cell, head) in ks/vs[cells][heads]; an element stands
// for code * scale.  dim in [16, kAttnMaxDim], a multiple of 16.
bool attn_i8_dim_ok(int dim);
hipError_t launch_sparse_decode_attention_i8(const float *q, const int8_t *kq,
                                             const uint16_t *ks, const int8_t *vq,
                                             const uint16_t *vs, const int *ids, int nq,
                                             int heads, int dim, int k, int n_cells,
                                             float scale, float *out, hipStream_t stream);

}  // namespace qsa
