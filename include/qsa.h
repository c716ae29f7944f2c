/*
 * qsa.h -- C ABI of libqsa.so: QSA block selection on AMD Instinct MI355X
 * (gfx950, CDNA4, wave64).
 *
 * QSA keeps the KV cache in blocks of 4 cells, each with a key summary of the
 * same shape as a query ([heads][dim] fp32).  Selection has two steps:
 *
 *   1. block scoring: for every query i and every ACTIVE block b,
 *        score[i][b] = sum_{h<heads} sum_{d<dim} q[i][h][d] * kblk[b][h][d]
 *      i.e. per-head dot products summed over the heads (page "#3108
 *      perf(hip): optimize exact QSA block scoring and top-k selection on
 *      gfx12", Summary item 1: the per-head reductions that make up a 4-head
 *      block score);
 *   2. per-query top-k of the active blocks by score, ties to the lower block
 *      id (same page, Summary item 2: radix top-k with 256-bin digits; page
 *      "#337 hip: gfx12 (RDNA4) QSA select - WMMA block scorer, prompt-aware
 *      top-k dispatch", What item 1: selection work follows the active block
 *      count, never the capacity).
 *
 * Conventions for every entry point:
 *   - Every data pointer is a DEVICE pointer on the device of `stream`, owned
 *     by the caller.
 *   - Device scratch.  Some launches need device memory beyond the caller's
 *     buffers: the published group words of the few-row top-k and of the
 *     fused decode select (at most 128 KB per query row), and the chunk
 *     partials of the decode attention (nq * heads * ceil(k/4) * (dim + 4)
 *     floats at most).  The library keeps one scratch buffer per (device,
 *     stream handle), allocated with hipMalloc on first need, grown when a
 *     call needs more and never freed before the process ends.  Work on one
 *     stream runs in order, so calls on the same stream share it safely;
 *     calls on different streams use different buffers.
 *       May allocate (the first call of a given size on a stream):
 *         qsa_block_topk             when 1 <= nq <= QSA_TOPK_FEW_ROWS, k >= 1 and active_blocks >= 1;
 *         qsa_block_select           under the same condition;
 *         qsa_sparse_decode_attention, qsa_sparse_decode_attention_i8
 *                                    whenever nq >= 1 and heads >= 1.
 *       Never allocate: qsa_block_scores, qsa_block_scores_ex,
 *         qsa_block_select_noalloc (a static array instead, see there), and
 *         qsa_block_topk / qsa_block_select with nq > QSA_TOPK_FEW_ROWS.
 *     Consequences: make one call of each size on a stream before capturing
 *     that stream into a HIP graph (an allocation during capture fails with
 *     QSA_ERR_NOMEM or QSA_ERR_LAUNCH); and synchronise a stream before
 *     destroying it, because the buffer is keyed on the stream handle: if
 *     the runtime hands the handle of a destroyed stream to a new one while
 *     work that uses the buffer is still queued, the two would share it.
 *     The library may be called from several host threads at once.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL = the default stream).  The call returns once the work is
 *     enqueued; results are valid after the stream is synchronised.
 *   - Invalid arguments are rejected before anything is enqueued, and the
 *     status is returned synchronously.  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - Layouts are dense and row-major, without padding.  Sizes are ints;
 *     index arithmetic inside is 64-bit.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     scores and ids on every call (no atomics take part in score arithmetic,
 *     and the selection order is a strict total order).
 */
#ifndef QSA_H
#define QSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define QSA_OK 0
#define QSA_ERR_NULL 1   /* a required pointer is NULL                              */
#define QSA_ERR_SHAPE 2  /* a size < 0, heads*dim not a multiple of 4 in [4, QSA_MAX_HEAD_DIM], active_blocks > QSA_MAX_ACTIVE_BLOCKS, or a bad attention dim */
#define QSA_ERR_K 3      /* k < 0 or k > QSA_TOPK_MAX_K                             */
#define QSA_ERR_ALIGN 4  /* q or kblk not 16-byte aligned, scores/ids not 4-byte aligned */
#define QSA_ERR_LAUNCH 5 /* the HIP runtime rejected a launch (hipGetLastError)     */
#define QSA_ERR_MODE 6   /* unknown precision mode                                  */
#define QSA_ERR_NOMEM 7  /* the library's device scratch could not be allocated     */
#define QSA_ERR_SCRATCH 8 /* qsa_block_select_noalloc: the call needs more than its static scratch */

/* Largest heads*dim (elements of one query or one block summary). */
#define QSA_MAX_HEAD_DIM 4096
/* Largest k accepted by qsa_block_topk. */
#define QSA_TOPK_MAX_K 4096
/* Largest active_blocks of the scoring and top-k calls (2^28 blocks = 2^30
 * cells): a row of scores then stays below the 2^32 bytes one hardware
 * buffer descriptor can address. */
#define QSA_MAX_ACTIVE_BLOCKS 268435456
/* qsa_block_topk spreads each row over the whole GPU when nq is at most this
 * (decode); larger batches select one row per workgroup.  Either way the
 * result is the same. */
#define QSA_TOPK_FEW_ROWS 16

/*
 * qsa_block_scores -- exact block scores (step 1 above).
 *
 *   q       [nq][heads][dim] fp32, 16-byte aligned.
 *   kblk    [>= active_blocks][heads][dim] fp32, 16-byte aligned.  Only rows
 *           [0, active_blocks) are read; rows past them (the rest of the
 *           capacity) are never touched and may hold anything.
 *   scores  out: [nq][active_blocks] fp32, row stride active_blocks.
 *
 * Arithmetic follows a fixed order that does not depend on a block's
 * position, so blocks with identical summaries get bitwise-identical scores
 * within a call.  Small nq (<= 8) uses a bandwidth-bound fp32 per-block dot
 * product; larger nq uses matrix-core tiles (QSA_SCORES_AUTO of
 * qsa_block_scores_ex below).  The error against an exact (FP64) evaluation
 * stays well inside 1e-6 * max|score| for N(0,1) inputs.
 *
 * nq == 0 or active_blocks == 0 is a successful no-op.  Non-finite inputs give
 * non-finite scores.
 */
int qsa_block_scores(const float *q, const float *kblk, int nq, int heads, int dim,
                     int active_blocks, float *scores, void *stream);

/*
 * qsa_block_topk -- per-query top-k of the active blocks (step 2 above).
 *
 *   scores  [nq][active_blocks] fp32 (row stride active_blocks), e.g. the
 *           output of qsa_block_scores.  May be NULL when active_blocks == 0.
 *   ids     out: [nq][k] int32.  Row i lists the k best block ids of query i
 *           in rank order: score descending, equal scores by ascending id.
 *           -0.0 and +0.0 are equal.  When k > active_blocks, slots
 *           [active_blocks, k) hold -1 (so active_blocks == 0 gives all -1).
 *
 * The result is exact on the given scores: it equals a full sort of each row
 * by (score desc, id asc) cut to k.  Scores must not be NaN (a NaN makes the
 * row's result unspecified, though still a set of valid ids).  The kernel's
 * work and dispatch depend on active_blocks only.
 *
 * nq == 0 or k == 0 is a successful no-op.
 */
int qsa_block_topk(const float *scores, int nq, int active_blocks, int k, int *ids,
                   void *stream);

/*
 * qsa_block_scores_ex -- qsa_block_scores with an explicit precision mode.
 *
 *   QSA_SCORES_AUTO    the library's choice (what qsa_block_scores does):
 *                      nq <= 8 -> fp32 per-block dot products (bandwidth-bound);
 *                      larger nq -> QSA_SCORES_F16X2.
 *   QSA_SCORES_FP32    fp32 arithmetic throughout: the dot-product kernel for
 *                      nq <= 8, fp32 matrix-core (MFMA) tiles otherwise.
 *   QSA_SCORES_BF16X3  bf16 matrix cores on an exact three-way split of every
 *                      fp32 operand into bf16 slices hi + mid + lo, summing the
 *                      six slice products of order <= 2 with the hi*hi products
 *                      in their own fp32 accumulator (page "#337 hip: gfx12
 *                      (RDNA4) QSA select - WMMA block scorer, prompt-aware top-k
 *                      dispatch", What item 2).  The dropped products are below
 *                      2^-24 of each term, so the error against FP64 is of the
 *                      same order as fp32 arithmetic's.
 *   QSA_SCORES_F16X2   fp16 matrix cores on a two-piece split: every row (a
 *                      query or a block summary) is scaled by a power of two
 *                      fixed by its first 32 elements (their largest magnitude
 *                      lands in [2^8, 2^9)), each scaled element is cut into
 *                      binary16 hi + lo (both rounded to nearest; 22
 *                      significant bits), and a product sums hi*hi (own fp32
 *                      accumulator) and hi*lo + lo*hi, scaled back exactly.
 *                      The same split principle as QSA_SCORES_BF16X3 with
 *                      wider pieces: three matrix products instead of six,
 *                      error of the same order.  A score whose scaled pieces
 *                      would leave binary16's range (an element more than 2^7
 *                      times its row's first-step maximum) is computed again
 *                      from its two rows in FP64; so is any score of a
 *                      non-finite input.
 *
 * Every mode keeps each score's arithmetic independent of the block's
 * position.  Other arguments, layouts and errors as qsa_block_scores; an
 * unknown mode returns QSA_ERR_MODE.
 */
#define QSA_SCORES_AUTO 0
#define QSA_SCORES_FP32 1
#define QSA_SCORES_BF16X3 2
#define QSA_SCORES_F16X2 3
int qsa_block_scores_ex(const float *q, const float *kblk, int nq, int heads, int dim,
                        int active_blocks, float *scores, int mode, void *stream);

/*
 * qsa_block_select -- both steps in one call: the scores of
 * qsa_block_scores (precision mode QSA_SCORES_AUTO) into `scores`, and the
 * top-k ids of qsa_block_topk on exactly those scores into `ids`.
 *
 * Results are identical to the two separate calls.  For few queries (nq <=
 * 8, the decode regime, with active_blocks <= 131072) the scoring kernel
 * also publishes, for every group of 64 consecutive blocks, the group's best
 * (score, id) pairs, which the top-k would otherwise read back in a launch
 * of its own -- one launch fewer on the latency-bound decode path (page
 * "#3108 perf(hip): optimize exact QSA block scoring and top-k selection on
 * gfx12", decode table: the selection, not the scoring, dominated decode).
 *
 * Arguments, layouts, alignment and errors as for the two calls.  k == 0
 * computes the scores only; active_blocks == 0 writes ids of -1 only;
 * nq == 0 is a successful no-op.
 */
int qsa_block_select(const float *q, const float *kblk, int nq, int heads, int dim,
                     int active_blocks, int k, float *scores, int *ids, void *stream);

/*
 * qsa_block_select_noalloc -- qsa_block_select for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, checks and results
 * (bitwise) as qsa_block_select; the caller still passes every input and
 * output.
 *
 * It never calls hipMalloc, hipFree or any allocating routine.  Its scratch
 * is one static device array of QSA_NOALLOC_SCRATCH_BYTES per GPU, created
 * with the library's code object and held until the process ends; the first
 * call on a device looks up the array's address (hipGetSymbolAddress).  That
 * size covers every call qsa_block_select accepts (at most QSA_TOPK_FEW_ROWS
 * rows of 16,384 eight-byte words; larger batches need none), and a call
 * that would need more returns QSA_ERR_SCRATCH before enqueuing anything.
 *
 * Every call on one GPU shares that GPU's array, whatever its stream: calls
 * that overlap on one GPU (on different streams, or from several host
 * threads without ordering) race and give undefined results.  Calls on one
 * stream are ordered and safe.  Nothing in the array has to start at zero.
 */
#define QSA_NOALLOC_SCRATCH_BYTES 2097152
int qsa_block_select_noalloc(const float *q, const float *kblk, int nq, int heads, int dim,
                             int active_blocks, int k, float *scores, int *ids, void *stream);

/*
 * qsa_sparse_decode_attention -- attention of each query over the KV cells of
 * its selected blocks (the consumer of qsa_block_topk's ids; page "#3102
 * perf(hip): enable wave32 QSA decode attention and MMVQ row reuse on gfx12",
 * Summary item 1: decode attention over the selected blocks' cells, computed
 * in chunks whose partials are merged in sequential chunk order).
 *
 *   q        [nq][heads][dim] fp32, 16-byte aligned.
 *   kcache   [>= n_cells][heads][dim] fp32 keys, one row per cell, 16-byte
 *   vcache   aligned; the same for values.  Cell c belongs to block c / 4.
 *            Only cells [0, n_cells) are read.
 *   ids      [nq][k] int32 block ids, e.g. the output of qsa_block_topk.
 *            Negative entries (the -1 padding) are skipped, and so are the
 *            cells at or past n_cells of a listed block.  A block listed
 *            twice is attended twice.
 *   scale    multiplies every dot product (e.g. 1/sqrt(dim)).
 *   out      out: [nq][heads][dim] fp32, 4-byte aligned:
 *              s_c = scale * q[i][h] . kcache[c][h]
 *              out[i][h] = sum_c exp(s_c - max s) vcache[c][h] / sum_c exp(s_c - max s)
 *            over the attended cells c of query i; all zeros when query i
 *            attends no cell.
 *
 * dim must be a multiple of 4 in [4, QSA_ATTN_MAX_DIM], heads*dim at most
 * QSA_MAX_HEAD_DIM and nq at most 65535 (else QSA_ERR_SHAPE); k in [0, QSA_TOPK_MAX_K] (else
 * QSA_ERR_K).  The cells are processed in chunks of 4, 8 or 16 listed blocks
 * (fixed by k, nq * heads and dim) and merged in chunk order, so results
 * are deterministic for given sizes (a query's output may differ in its
 * last bits between calls with different nq * heads, within the bound
 * below).  Against an FP64 evaluation the error of out[i][h][d] stays within
 *   max|v| * (T + 2 n_s 2^-24 |scale| max_c sum_d |q[i][h][d] k[c][h][d]|)
 * over the attended cells c, where n_s = 5 + log2(LPC) roundings per score
 * (LPC = dim/4 rounded up to a power of two) and T is a first-order bound
 * over the kernels' own summation sequences: in units of 2^-24,
 *   T = 2 (R + log2(64/LPC)) + min(n, 32) + 2 ceil(n/32) + 6 + 2 (8 + ln 4k)
 * for chunks of CB listed blocks (CB = 4 up to k = 1024, else 8 or 16;
 * R = 4 CB LPC / 64 cell rows per lane, n = ceil(k / CB) chunks), which
 * assumes expf within 2 ulp.  At dim 128 T runs from 2.7e-6 (k = 1) to
 * 8.3e-6 (k = 4096).
 * nq == 0 or heads == 0 is a successful no-op.
 */
#define QSA_ATTN_MAX_DIM 128
int qsa_sparse_decode_attention(const float *q, const float *kcache, const float *vcache,
                                const int *ids, int nq, int heads, int dim, int k, int n_cells,
                                float scale, float *out, void *stream);

/*
 * qsa_sparse_decode_attention_i8 -- the same attention over an int8 key/value
 * pool (the int8 pool of the decode-attention table on the page above; page
 * "#3224 [Engine] perf(hip): tune RDNA4 QSA prompt WMMA path
 * (STRATA_HIP_WMMA stays opt-in)", Summary item 2: int8 keys and values with
 * FP16 scales).  A key element stands for kcode[c][h][d] * kscale[c][h], a
 * value element for vcode[c][h][d] * vscale[c][h]:
 *
 *   kcode    [>= n_cells][heads][dim] int8 codes, 16-byte aligned; vcode the
 *   vcode    same for values.
 *   kscale   [>= n_cells][heads] IEEE binary16 scales (bit patterns), 2-byte
 *   vscale   aligned.
 *   q, ids, n_cells, scale, out, stream: as for qsa_sparse_decode_attention,
 *            whose formula this computes on the dequantised rows.
 *
 * dim must be a multiple of 16 in [16, QSA_ATTN_MAX_DIM] (else
 * QSA_ERR_SHAPE); other limits and errors as above.  The kernel forms
 * scale * (kscale * sum_d q_d kcode_d) and sums (w * vscale) * vcode in fp32;
 * against an FP64 evaluation on the dequantised rows the error stays within
 * the bound above with n_s = 18 + log2(LPC), LPC = dim/16 rounded up to a
 * power of two, and one more rounding per value term (w * vscale).
 * A cell costs 2 * (dim + 2) bytes per head to read instead of 8 * dim.
 */
int qsa_sparse_decode_attention_i8(const float *q, const int8_t *kcode, const uint16_t *kscale,
                                   const int8_t *vcode, const uint16_t *vscale, const int *ids,
                                   int nq, int heads, int dim, int k, int n_cells, float scale,
                                   float *out, void *stream);

/* Human-readable text of a status code (a static string; never NULL). */
const char *qsa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
