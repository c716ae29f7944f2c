/*
 * CPU oracle for QSA block selection (exact block scoring + per-query top-k).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or constant with the HIP library, and the HIP library
 * never calls it.
 *
 * Built with plain gcc (-O2, no -ffast-math, no FTZ); see oracle/__init__.py.
 *
 * Sources (web pages on the selection path of a closed inference engine):
 *   [P3] "#3102 perf(hip): enable wave32 QSA decode attention and MMVQ row
 *        reuse on gfx12", Summary item 1 (decode attention over the cells of
 *        the selected blocks, computed in chunks whose partial results are
 *        merged in sequential chunk order) and the decode-attention
 *        microbenchmark table (attended widths, one or four queries).
 *   [P2] "#3224 [Engine] perf(hip): tune RDNA4 QSA prompt WMMA path
 *        (STRATA_HIP_WMMA stays opt-in)", Summary item 2 (an int8 key/value
 *        pool carries FP16 scales for its keys and values).
 *   [P1] "#3108 perf(hip): optimize exact QSA block scoring and top-k selection
 *        on gfx12", Summary item 1 (a block score is the sum over the query's
 *        heads of per-head dot products against the block's key summary) and
 *        item 2 (radix top-k selection of blocks per query).
 *   [P4] "#337 hip: gfx12 (RDNA4) QSA select - WMMA block scorer, prompt-aware
 *        top-k dispatch", What item 1 (top-k runs over the active blocks, not
 *        the capacity) and item 2 (scores are checked against an FP64
 *        reference; top-k ids must equal the reference selection on the same
 *        scores).
 *
 * Readings where the pages are silent (listed in the design notes too):
 *   - layouts are dense row-major: q[nq][heads][dim], kblk[blocks][heads][dim],
 *     scores[nq][active_blocks], ids[nq][k];
 *   - heads are combined by a sum, with no 1/sqrt(d) or other scale;
 *   - ties in score go to the lower block id; -0.0 and +0.0 are equal;
 *   - ids come out in rank order (score descending, id ascending), and slots
 *     past active_blocks (k > active_blocks) hold -1;
 *   - scores must be finite (NaN is reported as an error);
 *   - decode attention ([P3]): per query and head, scaled dot-product
 *     attention over the cells of the listed blocks (block b holds cells
 *     4b .. 4b+3; cells at or past n_cells and ids of -1 are skipped), with a
 *     caller-given scale; no attended cell gives a zero output;
 *   - an int8 key/value pool ([P3] microbenchmark table, "int8" pool; [P2]
 *     Summary item 2: int8 keys and values with FP16 key and value scales)
 *     holds one signed 8-bit code per (cell, head, d) and one IEEE binary16
 *     scale per (cell, head); the value it stands for is code * scale.
 *
 * Pins (what this oracle is checked against, not itself): a hand-worked
 * 3-block example, exact integer inputs vs numpy int64 matmul, exact rationals
 * (fractions.Fraction) on tiny inputs, numpy float64 matmul, brute-force rank
 * on tiny rows with heavy ties, numpy lexsort, and invariants; see
 * tests/test_oracle.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* Status codes of this oracle (independent of the HIP library's codes). */
#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NAN 2
#define ORACLE_ERR_NOMEM 3

/*
 * Block scores in FP64 ([P1] Summary item 1; [P4] What item 2):
 *   out[i][b] = sum_{h<heads} sum_{d<dim} q[i][h][d] * kblk[b][h][d]
 * for 0 <= i < nq and 0 <= b < active_blocks.
 *
 * Every product of two fp32 numbers is exact in FP64 (24+24 <= 53 significand
 * bits), so the only rounding is in the heads*dim-1 sequential additions.
 * Rows b >= active_blocks of kblk are never read.
 */
int oracle_block_scores_f64(const float *q, const float *kblk, int64_t nq,
                            int64_t heads, int64_t dim, int64_t active_blocks,
                            double *out) {
  if (nq < 0 || heads < 0 || dim < 0 || active_blocks < 0) return ORACLE_ERR_ARG;
  if (nq == 0 || active_blocks == 0) return ORACLE_OK;
  if (!q || !kblk || !out) return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < nq; ++i) {
    for (int64_t b = 0; b < active_blocks; ++b) {
      double s = 0.0;
      for (int64_t h = 0; h < heads; ++h) {
        for (int64_t d = 0; d < dim; ++d) {
          const double qv = (double)q[(i * heads + h) * dim + d];
          const double kv = (double)kblk[(b * heads + h) * dim + d];
          s += qv * kv;
        }
      }
      out[i * active_blocks + b] = s;
    }
  }
  return ORACLE_OK;
}

/* One candidate of a row: its score and its block id. */
typedef struct {
  double score;
  int64_t id;
} cand_t;

/*
 * The selection order: a comes before b when its score is larger, or the
 * scores are equal and its id is smaller.  IEEE comparison, so -0.0 == +0.0.
 * This is a strict total order on a row of finite scores, so the sorted row,
 * and hence the top-k, is unique.
 */
static int cand_cmp(const void *pa, const void *pb) {
  const cand_t *a = (const cand_t *)pa;
  const cand_t *b = (const cand_t *)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  if (a->id < b->id) return -1;
  if (a->id > b->id) return 1;
  return 0;
}

/* Sort-based top-k of one row whose scores have already been widened. */
static void topk_row(cand_t *c, int64_t active_blocks, int64_t k, int32_t *ids) {
  qsort(c, (size_t)active_blocks, sizeof(cand_t), cand_cmp);
  for (int64_t r = 0; r < k; ++r) ids[r] = (r < active_blocks) ? (int32_t)c[r].id : -1;
}

/*
 * Top-k of fp32 scores ([P1] Summary item 2; [P4] What item 1, "top-k ids
 * equal the reference's" on the same scores): for every row i, sort the block
 * ids b in [0, active_blocks) by (score descending, id ascending) and write
 * the first k of them to ids[i][0..k); slots r >= active_blocks get -1.
 * A NaN score anywhere in the active range returns ORACLE_ERR_NAN.
 */
int oracle_block_topk(const float *scores, int64_t nq, int64_t active_blocks,
                      int64_t k, int32_t *ids) {
  if (nq < 0 || active_blocks < 0 || k < 0) return ORACLE_ERR_ARG;
  if (nq == 0 || k == 0) return ORACLE_OK;
  if (!ids || (active_blocks > 0 && !scores)) return ORACLE_ERR_ARG;
  cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(active_blocks > 0 ? active_blocks : 1));
  if (!c) return ORACLE_ERR_NOMEM;
  for (int64_t i = 0; i < nq; ++i) {
    for (int64_t b = 0; b < active_blocks; ++b) {
      const float s = scores[i * active_blocks + b];
      if (isnan(s)) {
        free(c);
        return ORACLE_ERR_NAN;
      }
      c[b].score = (double)s; /* widening is exact and keeps the order */
      c[b].id = b;
    }
    topk_row(c, active_blocks, k, ids + i * k);
  }
  free(c);
  return ORACLE_OK;
}

/*
 * The same top-k on FP64 scores.  Used only as a diagnostic (how often a
 * selection on the rounded fp32 scores equals the selection on the FP64
 * ones), never as a gate.
 */
int oracle_block_topk_f64(const double *scores, int64_t nq, int64_t active_blocks,
                          int64_t k, int32_t *ids) {
  if (nq < 0 || active_blocks < 0 || k < 0) return ORACLE_ERR_ARG;
  if (nq == 0 || k == 0) return ORACLE_OK;
  if (!ids || (active_blocks > 0 && !scores)) return ORACLE_ERR_ARG;
  cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(active_blocks > 0 ? active_blocks : 1));
  if (!c) return ORACLE_ERR_NOMEM;
  for (int64_t i = 0; i < nq; ++i) {
    for (int64_t b = 0; b < active_blocks; ++b) {
      const double s = scores[i * active_blocks + b];
      if (isnan(s)) {
        free(c);
        return ORACLE_ERR_NAN;
      }
      c[b].score = s;
      c[b].id = b;
    }
    topk_row(c, active_blocks, k, ids + i * k);
  }
  free(c);
  return ORACLE_OK;
}

/*
 * Block-sparse decode attention in FP64 ([P3] Summary item 1): for query i
 * and head h, over the attended cells c (the cells 4b .. 4b+3 of every listed
 * block b = ids[i][j] >= 0, j < k, with c < n_cells; a block listed twice
 * counts twice),
 *   s_c = scale * sum_{d<dim} q[i][h][d] * kc[c][h][d]
 *   w_c = exp(s_c - max_c s_c)
 *   out[i][h][d] = sum_c w_c * vc[c][h][d] / sum_c w_c
 * and out = 0 when no cell is attended.  Layouts: q[nq][heads][dim],
 * kc and vc [cells][heads][dim], ids[nq][k], out[nq][heads][dim].
 * The cells are visited in list order, the four cells of a block in order.
 */
int oracle_sparse_decode_attn_f64(const float *q, const float *kc, const float *vc,
                                  const int32_t *ids, int64_t nq, int64_t heads,
                                  int64_t dim, int64_t k, int64_t n_cells, double scale,
                                  double *out) {
  if (nq < 0 || heads < 0 || dim < 0 || k < 0 || n_cells < 0) return ORACLE_ERR_ARG;
  if (nq == 0 || heads == 0 || dim == 0) return ORACLE_OK;
  if (!q || !out || (k > 0 && (!ids || !kc || !vc))) return ORACLE_ERR_ARG;
  double *s = (double *)malloc(sizeof(double) * (size_t)(4 * k > 0 ? 4 * k : 1));
  int64_t *cell = (int64_t *)malloc(sizeof(int64_t) * (size_t)(4 * k > 0 ? 4 * k : 1));
  if (!s || !cell) {
    free(s);
    free(cell);
    return ORACLE_ERR_NOMEM;
  }
  for (int64_t i = 0; i < nq; ++i) {
    /* the attended cells of this query, in list order */
    int64_t n = 0;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t b = ids[i * k + j];
      if (b < 0) continue;
      for (int64_t e = 0; e < 4; ++e)
        if (4 * b + e < n_cells) cell[n++] = 4 * b + e;
    }
    for (int64_t h = 0; h < heads; ++h) {
      double *o = out + (i * heads + h) * dim;
      for (int64_t d = 0; d < dim; ++d) o[d] = 0.0;
      if (n == 0) continue;
      double m = -INFINITY;
      for (int64_t c = 0; c < n; ++c) {
        double dot = 0.0;
        for (int64_t d = 0; d < dim; ++d)
          dot += (double)q[(i * heads + h) * dim + d] * (double)kc[(cell[c] * heads + h) * dim + d];
        s[c] = scale * dot;
        if (s[c] > m) m = s[c];
      }
      double l = 0.0;
      for (int64_t c = 0; c < n; ++c) {
        const double w = exp(s[c] - m);
        l += w;
        for (int64_t d = 0; d < dim; ++d) o[d] += w * (double)vc[(cell[c] * heads + h) * dim + d];
      }
      for (int64_t d = 0; d < dim; ++d) o[d] /= l;
    }
  }
  free(s);
  free(cell);
  return ORACLE_OK;
}

/*
 * IEEE 754 binary16 to double, from the format: one sign bit, five exponent
 * bits with bias 15 and ten fraction bits; exponent 0 holds zero and the
 * subnormals (fraction * 2^-24), exponent 31 infinity (fraction 0) and NaN.
 */
double oracle_half_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 31;
  const int f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f == 0 ? INFINITY : NAN;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/*
 * The same attention over an int8 pool ([P3] microbenchmark table, int8 pool;
 * [P2] Summary item 2): key element (c, h, d) is kcode[c][h][d] *
 * half(kscale[c][h]), value element vcode[c][h][d] * half(vscale[c][h]); each
 * is formed in FP64 and the attention is then the one above.  Layouts:
 * kcode, vcode [cells][heads][dim] int8; kscale, vscale [cells][heads]
 * binary16 bit patterns.
 */
int oracle_sparse_decode_attn_i8_f64(const float *q, const int8_t *kcode, const uint16_t *kscale,
                                     const int8_t *vcode, const uint16_t *vscale,
                                     const int32_t *ids, int64_t nq, int64_t heads, int64_t dim,
                                     int64_t k, int64_t n_cells, double scale, double *out) {
  if (nq < 0 || heads < 0 || dim < 0 || k < 0 || n_cells < 0) return ORACLE_ERR_ARG;
  if (nq == 0 || heads == 0 || dim == 0) return ORACLE_OK;
  if (!q || !out || (k > 0 && (!ids || !kcode || !kscale || !vcode || !vscale)))
    return ORACLE_ERR_ARG;
  double *s = (double *)malloc(sizeof(double) * (size_t)(4 * k > 0 ? 4 * k : 1));
  int64_t *cell = (int64_t *)malloc(sizeof(int64_t) * (size_t)(4 * k > 0 ? 4 * k : 1));
  if (!s || !cell) {
    free(s);
    free(cell);
    return ORACLE_ERR_NOMEM;
  }
  for (int64_t i = 0; i < nq; ++i) {
    int64_t n = 0;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t b = ids[i * k + j];
      if (b < 0) continue;
      for (int64_t e = 0; e < 4; ++e)
        if (4 * b + e < n_cells) cell[n++] = 4 * b + e;
    }
    for (int64_t h = 0; h < heads; ++h) {
      double *o = out + (i * heads + h) * dim;
      for (int64_t d = 0; d < dim; ++d) o[d] = 0.0;
      if (n == 0) continue;
      double m = -INFINITY;
      for (int64_t c = 0; c < n; ++c) {
        const int64_t r = cell[c] * heads + h;
        const double ks = oracle_half_to_double(kscale[r]);
        double dot = 0.0;
        for (int64_t d = 0; d < dim; ++d)
          dot += (double)q[(i * heads + h) * dim + d] * ((double)kcode[r * dim + d] * ks);
        s[c] = scale * dot;
        if (s[c] > m) m = s[c];
      }
      double l = 0.0;
      for (int64_t c = 0; c < n; ++c) {
        const int64_t r = cell[c] * heads + h;
        const double vs = oracle_half_to_double(vscale[r]);
        const double w = exp(s[c] - m);
        l += w;
        for (int64_t d = 0; d < dim; ++d) o[d] += w * ((double)vcode[r * dim + d] * vs);
      }
      for (int64_t d = 0; d < dim; ++d) o[d] /= l;
    }
  }
  free(s);
  free(cell);
  return ORACLE_OK;
}
