// C ABI of libqsa.so (declared in include/qsa.h): argument checks, then the
// launches.  Every check happens before anything is enqueued, so a rejected
// call has no effect on the stream.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "qsa.h"
#include "qsa_internal.h"

static_assert(QSA_TOPK_MAX_K == qsa::kTopkMaxK, "header and kernels disagree on the top-k limit");
static_assert(QSA_ATTN_MAX_DIM == qsa::kAttnMaxDim, "header and kernels disagree on the attention dim");
static_assert(QSA_TOPK_FEW_ROWS == qsa::kWideMaxRows, "header and kernels disagree on the few-row path");
static_assert(QSA_NOALLOC_SCRATCH_BYTES == qsa::kNoAllocScratchBytes,
              "header and kernels disagree on the static scratch size");
static_assert(QSA_SCORES_AUTO == qsa::kScoresAuto && QSA_SCORES_FP32 == qsa::kScoresFp32 &&
                  QSA_SCORES_BF16X3 == qsa::kScoresBf16x3 && QSA_SCORES_F16X2 == qsa::kScoresF16x2,
              "header and kernels disagree on the precision modes");

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int launch_status(hipError_t e) {
  if (e == hipSuccess) return QSA_OK;
  return e == hipErrorOutOfMemory ? QSA_ERR_NOMEM : QSA_ERR_LAUNCH;
}

}  // namespace

extern "C" int qsa_block_scores_ex(const float *q, const float *kblk, int nq, int heads, int dim,
                                   int active_blocks, float *scores, int mode, void *stream) {
  if (nq < 0 || heads < 0 || dim < 0 || active_blocks < 0) return QSA_ERR_SHAPE;
  if (active_blocks > QSA_MAX_ACTIVE_BLOCKS) return QSA_ERR_SHAPE;
  const int64_t K = int64_t(heads) * dim;
  if (K < 4 || K % 4 != 0 || K > QSA_MAX_HEAD_DIM) return QSA_ERR_SHAPE;
  if (mode != QSA_SCORES_AUTO && mode != QSA_SCORES_FP32 && mode != QSA_SCORES_BF16X3 &&
      mode != QSA_SCORES_F16X2)
    return QSA_ERR_MODE;
  if (nq == 0 || active_blocks == 0) return QSA_OK;
  if (!q || !kblk || !scores) return QSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kblk, 16) || !aligned(scores, 4)) return QSA_ERR_ALIGN;
  (void)hipGetLastError();  // start from a clean launch status
  return launch_status(qsa::launch_block_scores(q, kblk, nq, int(K), active_blocks, scores, mode,
                                                static_cast<hipStream_t>(stream)));
}

extern "C" int qsa_block_scores(const float *q, const float *kblk, int nq, int heads, int dim,
                                int active_blocks, float *scores, void *stream) {
  return qsa_block_scores_ex(q, kblk, nq, heads, dim, active_blocks, scores, QSA_SCORES_AUTO,
                             stream);
}

extern "C" int qsa_block_topk(const float *scores, int nq, int active_blocks, int k, int *ids,
                              void *stream) {
  if (nq < 0 || active_blocks < 0 || active_blocks > QSA_MAX_ACTIVE_BLOCKS) return QSA_ERR_SHAPE;
  if (k < 0 || k > QSA_TOPK_MAX_K) return QSA_ERR_K;
  if (nq == 0 || k == 0) return QSA_OK;
  if (!ids || (active_blocks > 0 && !scores)) return QSA_ERR_NULL;
  if (!aligned(ids, 4) || !aligned(scores, 4)) return QSA_ERR_ALIGN;
  (void)hipGetLastError();
  return launch_status(qsa::launch_block_topk(scores, nq, active_blocks, k, ids,
                                              static_cast<hipStream_t>(stream)));
}

namespace {

// The argument checks of qsa_block_select (and its allocation-free variant).
// Returns QSA_OK with *done set when the call is a no-op.
int check_select(const float *q, const float *kblk, int nq, int heads, int dim, int active_blocks,
                 int k, const float *scores, const int *ids, bool *done) {
  *done = false;
  if (nq < 0 || heads < 0 || dim < 0 || active_blocks < 0) return QSA_ERR_SHAPE;
  if (active_blocks > QSA_MAX_ACTIVE_BLOCKS) return QSA_ERR_SHAPE;
  const int64_t K = int64_t(heads) * dim;
  if (K < 4 || K % 4 != 0 || K > QSA_MAX_HEAD_DIM) return QSA_ERR_SHAPE;
  if (k < 0 || k > QSA_TOPK_MAX_K) return QSA_ERR_K;
  if (nq == 0 || (k == 0 && active_blocks == 0)) {
    *done = true;
    return QSA_OK;
  }
  if (active_blocks > 0 && (!q || !kblk || !scores)) return QSA_ERR_NULL;
  if (k > 0 && !ids) return QSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kblk, 16) || !aligned(scores, 4) || !aligned(ids, 4))
    return QSA_ERR_ALIGN;
  return QSA_OK;
}

int run_select(const float *q, const float *kblk, int nq, int heads, int dim, int active_blocks,
               int k, float *scores, int *ids, void *stream, qsa::ScratchFn scratch) {
  (void)hipGetLastError();  // start from a clean launch status
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int K = heads * dim;
  if (k == 0)
    return launch_status(
        qsa::launch_block_scores(q, kblk, nq, K, active_blocks, scores, qsa::kScoresAuto, s));
  if (active_blocks == 0)
    return launch_status(qsa::launch_block_topk(scores, nq, 0, k, ids, s, scratch));
  return launch_status(
      qsa::launch_block_select(q, kblk, nq, K, active_blocks, k, scores, ids, s, scratch));
}

}  // namespace

extern "C" int qsa_block_select(const float *q, const float *kblk, int nq, int heads, int dim,
                                int active_blocks, int k, float *scores, int *ids, void *stream) {
  bool done = false;
  const int st = check_select(q, kblk, nq, heads, dim, active_blocks, k, scores, ids, &done);
  if (st != QSA_OK || done) return st;
  return run_select(q, kblk, nq, heads, dim, active_blocks, k, scores, ids, stream,
                    qsa::workspace);
}

extern "C" int qsa_block_select_noalloc(const float *q, const float *kblk, int nq, int heads,
                                        int dim, int active_blocks, int k, float *scores, int *ids,
                                        void *stream) {
  bool done = false;
  const int st = check_select(q, kblk, nq, heads, dim, active_blocks, k, scores, ids, &done);
  if (st != QSA_OK || done) return st;
  if (qsa::select_scratch_bytes(nq, heads * dim, active_blocks, k) > QSA_NOALLOC_SCRATCH_BYTES)
    return QSA_ERR_SCRATCH;
  return run_select(q, kblk, nq, heads, dim, active_blocks, k, scores, ids, stream,
                    qsa::static_scratch);
}

extern "C" int qsa_sparse_decode_attention(const float *q, const float *kcache, const float *vcache,
                                           const int *ids, int nq, int heads, int dim, int k,
                                           int n_cells, float scale, float *out, void *stream) {
  if (nq < 0 || heads < 0 || dim < 0 || n_cells < 0) return QSA_ERR_SHAPE;
  if (!qsa::attn_dim_ok(dim) || int64_t(heads) * dim > QSA_MAX_HEAD_DIM) return QSA_ERR_SHAPE;
  if (nq > 65535) return QSA_ERR_SHAPE;  // one grid dimension per query
  if (k < 0 || k > QSA_TOPK_MAX_K) return QSA_ERR_K;
  if (nq == 0 || heads == 0) return QSA_OK;
  if (!q || !out || (k > 0 && !ids) || (n_cells > 0 && (!kcache || !vcache))) return QSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kcache, 16) || !aligned(vcache, 16) || !aligned(ids, 4) ||
      !aligned(out, 4))
    return QSA_ERR_ALIGN;
  (void)hipGetLastError();
  return launch_status(qsa::launch_sparse_decode_attention(q, kcache, vcache, ids, nq, heads, dim,
                                                           k, n_cells, scale, out,
                                                           static_cast<hipStream_t>(stream)));
}

extern "C" int qsa_sparse_decode_attention_i8(const float *q, const int8_t *kcode,
                                              const uint16_t *kscale, const int8_t *vcode,
                                              const uint16_t *vscale, const int *ids, int nq,
                                              int heads, int dim, int k, int n_cells, float scale,
                                              float *out, void *stream) {
  if (nq < 0 || heads < 0 || dim < 0 || n_cells < 0) return QSA_ERR_SHAPE;
  if (!qsa::attn_i8_dim_ok(dim) || int64_t(heads) * dim > QSA_MAX_HEAD_DIM) return QSA_ERR_SHAPE;
  if (nq > 65535) return QSA_ERR_SHAPE;
  if (k < 0 || k > QSA_TOPK_MAX_K) return QSA_ERR_K;
  if (nq == 0 || heads == 0) return QSA_OK;
  if (!q || !out || (k > 0 && !ids) ||
      (n_cells > 0 && (!kcode || !kscale || !vcode || !vscale)))
    return QSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kcode, 16) || !aligned(vcode, 16) || !aligned(kscale, 2) ||
      !aligned(vscale, 2) || !aligned(ids, 4) || !aligned(out, 4))
    return QSA_ERR_ALIGN;
  (void)hipGetLastError();
  return launch_status(qsa::launch_sparse_decode_attention_i8(
      q, kcode, kscale, vcode, vscale, ids, nq, heads, dim, k, n_cells, scale, out,
      static_cast<hipStream_t>(stream)));
}

extern "C" const char *qsa_strerror(int status) {
  switch (status) {
    case QSA_OK:
      return "success";
    case QSA_ERR_NULL:
      return "a required pointer is NULL";
    case QSA_ERR_SHAPE:
      return "bad shape: a size is negative, heads*dim is not a multiple of 4 in [4, 4096], "
             "or an attention dim is not a multiple of 4 (int8 pool: 16) in [4 (16), 128]";
    case QSA_ERR_K:
      return "bad k: k < 0 or k > 4096";
    case QSA_ERR_ALIGN:
      return "misaligned pointer: q/kblk need 16 bytes, scores/ids 4 bytes";
    case QSA_ERR_LAUNCH:
      return "the HIP runtime rejected a kernel launch";
    case QSA_ERR_MODE:
      return "unknown precision mode";
    case QSA_ERR_NOMEM:
      return "the library could not allocate its device scratch";
    case QSA_ERR_SCRATCH:
      return "the call needs more device scratch than the allocation-free entry point holds";
    default:
      return "unknown status";
  }
}
