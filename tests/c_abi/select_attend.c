/*
 * The decode layer through the C ABI alone: a plain C program that includes
 * only include/qsa.h and the HIP runtime's C API, moves its inputs to the
 * device, calls qsa_block_select and qsa_sparse_decode_attention on one
 * stream, and writes the results back to files.  tests/test_c_abi.py builds
 * it (CPU) and runs it against the CPU oracle (GPU).
 *
 *   select_attend DIR NQ HEADS DIM ACTIVE CAPACITY K
 *
 * reads DIR/q.bin   [NQ][HEADS][DIM] float32
 *       DIR/kblk.bin [CAPACITY][HEADS][DIM] float32
 *       DIR/kc.bin, DIR/vc.bin [4 CAPACITY][HEADS][DIM] float32
 * writes DIR/scores.bin [NQ][ACTIVE] float32, DIR/ids.bin [NQ][K] int32,
 *        DIR/out.bin [NQ][HEADS][DIM] float32.
 * Exit status 0 on success; anything else prints the failing call.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "qsa.h"

static int fail_hip(const char *what, hipError_t e) {
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 2;
}

static void *read_file(const char *dir, const char *name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return NULL;
  void *buf = malloc(bytes ? bytes : 1);
  size_t got = buf ? fread(buf, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char *dir, const char *name, const void *buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f) return 0;
  size_t put = fwrite(buf, 1, bytes, f);
  fclose(f);
  return put == bytes;
}

int main(int argc, char **argv) {
  if (argc != 8) {
    fprintf(stderr, "usage: %s DIR NQ HEADS DIM ACTIVE CAPACITY K\n", argv[0]);
    return 1;
  }
  const char *dir = argv[1];
  const int nq = atoi(argv[2]), heads = atoi(argv[3]), dim = atoi(argv[4]);
  const int active = atoi(argv[5]), capacity = atoi(argv[6]), k = atoi(argv[7]);
  const size_t K = (size_t)heads * dim;
  const size_t qb = nq * K * 4, kbb = capacity * K * 4, cb = 4 * (size_t)capacity * K * 4;
  const size_t sb = (size_t)nq * active * 4, ib = (size_t)nq * k * 4, ob = qb;

  float *q = read_file(dir, "q.bin", qb), *kblk = read_file(dir, "kblk.bin", kbb);
  float *kc = read_file(dir, "kc.bin", cb), *vc = read_file(dir, "vc.bin", cb);
  if (!q || !kblk || !kc || !vc) {
    fprintf(stderr, "could not read the inputs in %s\n", dir);
    return 1;
  }

  hipError_t e;
  hipStream_t stream;
  if ((e = hipStreamCreate(&stream)) != hipSuccess) return fail_hip("hipStreamCreate", e);
  void *dq, *dkb, *dkc, *dvc, *ds, *di, *dout;
  if ((e = hipMalloc(&dq, qb)) != hipSuccess) return fail_hip("hipMalloc q", e);
  if ((e = hipMalloc(&dkb, kbb)) != hipSuccess) return fail_hip("hipMalloc kblk", e);
  if ((e = hipMalloc(&dkc, cb)) != hipSuccess) return fail_hip("hipMalloc kc", e);
  if ((e = hipMalloc(&dvc, cb)) != hipSuccess) return fail_hip("hipMalloc vc", e);
  if ((e = hipMalloc(&ds, sb ? sb : 4)) != hipSuccess) return fail_hip("hipMalloc scores", e);
  if ((e = hipMalloc(&di, ib ? ib : 4)) != hipSuccess) return fail_hip("hipMalloc ids", e);
  if ((e = hipMalloc(&dout, ob)) != hipSuccess) return fail_hip("hipMalloc out", e);
  if ((e = hipMemcpy(dq, q, qb, hipMemcpyHostToDevice)) != hipSuccess) return fail_hip("copy q", e);
  if ((e = hipMemcpy(dkb, kblk, kbb, hipMemcpyHostToDevice)) != hipSuccess) return fail_hip("copy kblk", e);
  if ((e = hipMemcpy(dkc, kc, cb, hipMemcpyHostToDevice)) != hipSuccess) return fail_hip("copy kc", e);
  if ((e = hipMemcpy(dvc, vc, cb, hipMemcpyHostToDevice)) != hipSuccess) return fail_hip("copy vc", e);

  int st = qsa_block_select(dq, dkb, nq, heads, dim, active, k, ds, di, stream);
  if (st != QSA_OK) {
    fprintf(stderr, "qsa_block_select: %s\n", qsa_strerror(st));
    return 3;
  }
  st = qsa_sparse_decode_attention(dq, dkc, dvc, di, nq, heads, dim, k, 4 * active,
                                   (float)(1.0 / sqrt((double)dim)), dout, stream);
  if (st != QSA_OK) {
    fprintf(stderr, "qsa_sparse_decode_attention: %s\n", qsa_strerror(st));
    return 3;
  }
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return fail_hip("hipStreamSynchronize", e);

  float *s = malloc(sb ? sb : 4), *out = malloc(ob);
  int32_t *ids = malloc(ib ? ib : 4);
  if (!s || !out || !ids) return 1;
  if ((e = hipMemcpy(s, ds, sb, hipMemcpyDeviceToHost)) != hipSuccess) return fail_hip("copy scores", e);
  if ((e = hipMemcpy(ids, di, ib, hipMemcpyDeviceToHost)) != hipSuccess) return fail_hip("copy ids", e);
  if ((e = hipMemcpy(out, dout, ob, hipMemcpyDeviceToHost)) != hipSuccess) return fail_hip("copy out", e);
  if (!write_file(dir, "scores.bin", s, sb) || !write_file(dir, "ids.bin", ids, ib) ||
      !write_file(dir, "out.bin", out, ob)) {
    fprintf(stderr, "could not write the outputs in %s\n", dir);
    return 1;
  }
  hipFree(dq);
  hipFree(dkb);
  hipFree(dkc);
  hipFree(dvc);
  hipFree(ds);
  hipFree(di);
  hipFree(dout);
  hipStreamDestroy(stream);
  free(q);
  free(kblk);
  free(kc);
  free(vc);
  free(s);
  free(out);
  free(ids);
  printf("select_attend ok: nq=%d heads=%d dim=%d active=%d k=%d\n", nq, heads, dim, active, k);
  return 0;
}
