// Block-sparse decode attention over the selected blocks (gfx950, wave64).
//
// Page "#3102 perf(hip): enable wave32 QSA decode attention and MMVQ row
// reuse on gfx12", Summary item 1: after selection, each decode query attends
// only to the KV cells of its selected blocks; the cells are processed in
// chunks whose partial results are merged in sequential chunk order.  For
// query i and head h, over the attended cells c (cells 4b .. 4b+3 of every
// listed block b = ids[i][j] >= 0, c < n_cells):
//   s_c = scale * q[i][h] . k[c][h],   w_c = exp(s_c - max s),
//   out[i][h] = sum_c w_c v[c][h] / sum_c w_c        (0 if no cell).
//
// Two launches:
//   1. attn_chunk_kernel: one wave per (query, head, chunk of CB listed
//      blocks = up to 4 * CB cells; CB = 4, 8 or 16, see chunk_blocks).
//      A cell row of `dim` fp32 is spread over LPC lanes (a float4 each;
//      LPC = dim/4 rounded up to a power of two, dim <= 128), so one load
//      instruction covers 64/LPC cells.  The wave first
//      issues every key and value load of its chunk, then forms the dot
//      products (4 FMAs per lane and an LPC-lane butterfly: a fixed tree),
//      the chunk maximum m, the weights exp(s - m), their sum l and the
//      weighted value sum acc, and writes (m, l, acc[dim]).
//   2. attn_merge_kernel: one workgroup per (query, head, 64 dims) folds
//      the chunk partials: M = max m_j, L = sum l_j e^(m_j - M),
//      out = sum acc_j e^(m_j - M) / L, in a fixed order (each wave sums 32
//      consecutive chunks, then the waves' sums are added in order).
//      A fused variant (the last chunk wave of a (query, head) merging, found
//      by an atomic count) is slower on this GPU: the device-scope release
//      every wave needs writes back its XCD's L2, and even with write-through
//      partials and no fences the count's atomics serialise on one address
//      (k = 4096: 512 waves per (query, head)).
// Bound: HBM (the gathered key and value rows); the fixed chunking and merge
// order make the result deterministic.
//
// An int8 pool (the int8 rows of that page's decode-attention table; page
// "#3224 [Engine] perf(hip): tune RDNA4 QSA prompt WMMA path (STRATA_HIP_WMMA
// stays opt-in)", Summary item 2: int8 keys and values carry FP16 scales)
// holds one signed code per (cell, head, d) and one binary16 scale per
// (cell, head).  attn_chunk_i8_kernel gathers 16 codes per lane (a row of dim
// codes over dim/16 lanes), forms the dot product of q with the codes and
// multiplies by the key scale once per cell, and accumulates (w * value scale)
// * code; the partials and the merge are those of the fp32 pool.  A cell then
// costs 2 * (dim + 2) bytes per head instead of 8 * dim.
#include <hip/hip_runtime.h>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

// Sum over the LPC lanes of a cell (lane bits below log2 LPC), the same tree in
// every lane.
template <int LPC>
__device__ __forceinline__ float cell_sum(float v) {
  if constexpr (LPC >= 2) v += __uint_as_float(lane_xor<1>(__float_as_uint(v)));
  if constexpr (LPC >= 4) v += __uint_as_float(lane_xor<2>(__float_as_uint(v)));
  if constexpr (LPC >= 8) v += __uint_as_float(lane_xor<4>(__float_as_uint(v)));
  if constexpr (LPC >= 16) v += __uint_as_float(lane_xor<8>(__float_as_uint(v)));
  if constexpr (LPC >= 32) v += __uint_as_float(lane_xor<16>(__float_as_uint(v)));
  if constexpr (LPC >= 64) v += __uint_as_float(lane_xor<32>(__float_as_uint(v)));
  return v;
}

// Combine across the 64/LPC cell groups of the wave (lane bits from log2 LPC up).
template <int LPC, class Op>
__device__ __forceinline__ float group_all(float v, Op op) {
  if constexpr (LPC <= 1) v = op(v, __uint_as_float(lane_xor<1>(__float_as_uint(v))));
  if constexpr (LPC <= 2) v = op(v, __uint_as_float(lane_xor<2>(__float_as_uint(v))));
  if constexpr (LPC <= 4) v = op(v, __uint_as_float(lane_xor<4>(__float_as_uint(v))));
  if constexpr (LPC <= 8) v = op(v, __uint_as_float(lane_xor<8>(__float_as_uint(v))));
  if constexpr (LPC <= 16) v = op(v, __uint_as_float(lane_xor<16>(__float_as_uint(v))));
  if constexpr (LPC <= 32) v = op(v, __uint_as_float(lane_xor<32>(__float_as_uint(v))));
  return v;
}

constexpr int kMergeMaxChunks = 512;  // QSA_TOPK_MAX_K / 8: chunk_blocks keeps nchunks within it

template <int LPC, int CB>
__global__ __launch_bounds__(64) void attn_chunk_kernel(const float *__restrict__ q,
                                                        const float *__restrict__ kc,
                                                        const float *__restrict__ vc,
                                                        const int *__restrict__ ids, int heads,
                                                        int dim, int k, int n_cells, float scale,
                                                        float *__restrict__ part, int nchunks) {
  constexpr int CPI = 64 / LPC;                                    // cells per load instruction
  constexpr int ROUNDS = 4 * CB / CPI > 0 ? 4 * CB / CPI : 1;  // loads per chunk
  const int lane = threadIdx.x;
  const int chunk = blockIdx.x;
  const int h = blockIdx.y;
  const int i = blockIdx.z;
  const int sub = lane & (LPC - 1);             // float4 slot within the row
  const int grp = lane / LPC;                   // cell group of this lane
  const bool live = 4 * sub < dim;              // lanes past the row hold zeros

  // The chunk's listed blocks, one per lane (lanes 0 .. CB-1).
  const int j0 = chunk * CB;
  int my_id = -1;
  if (lane < CB && j0 + lane < k) my_id = ids[int64_t(i) * k + j0 + lane];

  const int64_t row = int64_t(heads) * dim;     // floats per cell
  const int64_t col = int64_t(h) * dim + 4 * sub;

  // Cell of round r for this lane: slot r*CPI + grp of the chunk's cells.
  int64_t cell[ROUNDS];
  bool ok[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int slot = r * CPI + grp;
    const int b = __shfl(my_id, (slot >> 2) & 63, 64);  // -1 past the chunk's blocks
    const int64_t c = int64_t(b) * 4 + (slot & 3);
    ok[r] = slot < 4 * CB && b >= 0 && c < n_cells;
    cell[r] = c;
  }
  // Every load of the chunk in flight at once (keys, then values); masked
  // lanes load nothing.
  f4 kv[ROUNDS], vv[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    kv[r] = f4{0.f, 0.f, 0.f, 0.f};
    if (ok[r] && live) kv[r] = *reinterpret_cast<const f4 *>(kc + cell[r] * row + col);
  }
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    vv[r] = f4{0.f, 0.f, 0.f, 0.f};
    if (ok[r] && live) vv[r] = *reinterpret_cast<const f4 *>(vc + cell[r] * row + col);
  }
  f4 qv = {0.f, 0.f, 0.f, 0.f};
  if (live) qv = *reinterpret_cast<const f4 *>(q + (int64_t(i) * heads + h) * dim + 4 * sub);

  // Scores of this lane's cells (the same value in all LPC lanes of a cell).
  float s[ROUNDS];
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    float p = qv.x * kv[r].x;
    p = __builtin_fmaf(qv.y, kv[r].y, p);
    p = __builtin_fmaf(qv.z, kv[r].z, p);
    p = __builtin_fmaf(qv.w, kv[r].w, p);
    s[r] = ok[r] ? scale * cell_sum<LPC>(p) : -INFINITY;
    m = fmaxf(m, s[r]);
  }
  m = group_all<LPC>(m, [](float a, float b) { return fmaxf(a, b); });

  float l = 0.f;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  if (m > -INFINITY) {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const float w = ok[r] ? expf(s[r] - m) : 0.f;
      l += w;
      acc.x = __builtin_fmaf(w, vv[r].x, acc.x);
      acc.y = __builtin_fmaf(w, vv[r].y, acc.y);
      acc.z = __builtin_fmaf(w, vv[r].z, acc.z);
      acc.w = __builtin_fmaf(w, vv[r].w, acc.w);
    }
  }
  auto add = [](float a, float b) { return a + b; };
  l = group_all<LPC>(l, add);
  acc.x = group_all<LPC>(acc.x, add);
  acc.y = group_all<LPC>(acc.y, add);
  acc.z = group_all<LPC>(acc.z, add);
  acc.w = group_all<LPC>(acc.w, add);

  // part[(i * heads + h) * nchunks + chunk] = {m, l, acc[dim]} (dim + 2 floats,
  // padded to dim + 4 so the float4 stores stay aligned).
  float *dst = part + ((int64_t(i) * heads + h) * nchunks + chunk) * (dim + 4);
  if (lane == 0) {
    dst[0] = m;
    dst[1] = l;
  }
  if (grp == 0 && live) *reinterpret_cast<f4 *>(dst + 4 + 4 * sub) = acc;
}

// The int8 pool.  LPC lanes hold one cell's row of dim codes, 16 each (LPC =
// dim/16 rounded up to a power of two, dim <= 128), so one load instruction
// covers 64/LPC cells; the scales are one 2-byte load per cell (all LPC lanes
// of a cell read the same address).
template <int LPC, int CB>
__global__ __launch_bounds__(64) void attn_chunk_i8_kernel(
    const float *__restrict__ q, const int8_t *__restrict__ kq, const uint16_t *__restrict__ ks,
    const int8_t *__restrict__ vq, const uint16_t *__restrict__ vs, const int *__restrict__ ids,
    int heads, int dim, int k, int n_cells, float scale, float *__restrict__ part, int nchunks) {
  constexpr int CPI = 64 / LPC;
  constexpr int ROUNDS = 4 * CB / CPI > 0 ? 4 * CB / CPI : 1;
  const int lane = threadIdx.x;
  const int chunk = blockIdx.x;
  const int h = blockIdx.y;
  const int i = blockIdx.z;
  const int sub = lane & (LPC - 1);
  const int grp = lane / LPC;
  const bool live = 16 * sub < dim;

  const int j0 = chunk * CB;
  int my_id = -1;
  if (lane < CB && j0 + lane < k) my_id = ids[int64_t(i) * k + j0 + lane];

  const int64_t row = int64_t(heads) * dim;  // codes per cell
  const int64_t col = int64_t(h) * dim + 16 * sub;

  int64_t cell[ROUNDS];
  bool ok[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int slot = r * CPI + grp;
    const int b = __shfl(my_id, (slot >> 2) & 63, 64);
    const int64_t c = int64_t(b) * 4 + (slot & 3);
    ok[r] = slot < 4 * CB && b >= 0 && c < n_cells;
    cell[r] = c;
  }
  uint4 kv[ROUNDS], vv[ROUNDS];
  uint16_t ksc[ROUNDS], vsc[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    kv[r] = uint4{0u, 0u, 0u, 0u};
    ksc[r] = 0;
    if (ok[r]) {
      if (live) kv[r] = *reinterpret_cast<const uint4 *>(kq + cell[r] * row + col);
      ksc[r] = ks[cell[r] * heads + h];
    }
  }
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    vv[r] = uint4{0u, 0u, 0u, 0u};
    vsc[r] = 0;
    if (ok[r]) {
      if (live) vv[r] = *reinterpret_cast<const uint4 *>(vq + cell[r] * row + col);
      vsc[r] = vs[cell[r] * heads + h];
    }
  }
  float qv[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) qv[e] = 0.f;
  if (live) {
    const f4 *qp = reinterpret_cast<const f4 *>(q + (int64_t(i) * heads + h) * dim + 16 * sub);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f4 t = qp[e];
      qv[4 * e] = t.x;
      qv[4 * e + 1] = t.y;
      qv[4 * e + 2] = t.z;
      qv[4 * e + 3] = t.w;
    }
  }

  // Signed byte e of a row of 16 codes, as a float.
  auto code = [](const uint4 &u, int e) {
    const uint32_t wv = e < 4 ? u.x : e < 8 ? u.y : e < 12 ? u.z : u.w;
    return float(int(int8_t(uint8_t(wv >> (8 * (e & 3))))));
  };

  float s[ROUNDS];
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    float p = qv[0] * code(kv[r], 0);
#pragma unroll
    for (int e = 1; e < 16; ++e) p = __builtin_fmaf(qv[e], code(kv[r], e), p);
    const float kscale = float(__builtin_bit_cast(_Float16, ksc[r]));
    s[r] = ok[r] ? scale * (cell_sum<LPC>(p) * kscale) : -INFINITY;
    m = fmaxf(m, s[r]);
  }
  m = group_all<LPC>(m, [](float a, float b) { return fmaxf(a, b); });

  float l = 0.f;
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  if (m > -INFINITY) {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const float w = ok[r] ? expf(s[r] - m) : 0.f;
      l += w;
      const float wv = w * float(__builtin_bit_cast(_Float16, vsc[r]));
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = __builtin_fmaf(wv, code(vv[r], e), acc[e]);
    }
  }
  auto add = [](float a, float b) { return a + b; };
  l = group_all<LPC>(l, add);
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = group_all<LPC>(acc[e], add);

  float *dst = part + ((int64_t(i) * heads + h) * nchunks + chunk) * (dim + 4);
  if (lane == 0) {
    dst[0] = m;
    dst[1] = l;
  }
  if (grp == 0 && live) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      *reinterpret_cast<f4 *>(dst + 4 + 16 * sub + 4 * e) =
          f4{acc[4 * e], acc[4 * e + 1], acc[4 * e + 2], acc[4 * e + 3]};
  }
}

// One workgroup per (query, head, 64 dims of the row) folds the chunk
// partials, one wave per 32 chunks (nw = ceil(nchunks / 32) waves, at most
// 16), so every wave issues all of its loads at once and the fold costs one
// round trip to memory at any k; a row of 128 dims is split over two
// workgroups, which halves the bytes each CU loads.  M = max m_j over all
// chunks, e_j = exp(m_j - M); wave w forms sum_j e_j l_j and sum_j e_j
// acc_j[d] over its chunks in chunk order, and wave 0 adds the waves' sums in
// wave order and divides.  (Both workgroups of a row form M, e_j and the l
// sums identically.)
constexpr int kMergeChunksPerWave = 32;
constexpr int kMergeMaxWaves = kMergeMaxChunks / kMergeChunksPerWave;

__global__ __launch_bounds__(64 * kMergeMaxWaves) void attn_merge_kernel(
    const float *__restrict__ part, int heads, int dim, int nchunks, float *__restrict__ out) {
  __shared__ float red[kMergeMaxWaves][2 + 64];  // per wave: L, unused, acc[64 dims]
  __shared__ float ew[kMergeMaxChunks];          // e_j of every chunk
  __shared__ float wmax[kMergeMaxWaves];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int nw = blockDim.x >> 6;
  const int h = blockIdx.x;
  const int i = blockIdx.y;
  const int d = 64 * int(blockIdx.z) + lane;  // this lane's dim
  const int stride = dim + 4;
  const float *src = part + (int64_t(i) * heads + h) * nchunks * stride;
  float *o = out + (int64_t(i) * heads + h) * dim;
  const int j0 = w * kMergeChunksPerWave;
  const int nj = min(kMergeChunksPerWave, nchunks - j0);  // >= 1: nw = ceil(nchunks / 32)

  // Every load of this wave first: lane u < nj holds chunk j0 + u's maximum
  // and sum; a0 holds dim d of the value sums of all its chunks.
  const bool live = d < dim;
  float mj = -INFINITY, lj = 0.f;
  if (lane < nj) {
    mj = src[int64_t(j0 + lane) * stride];
    lj = src[int64_t(j0 + lane) * stride + 1];
  }
  float a0[kMergeChunksPerWave];
#pragma unroll
  for (int u = 0; u < kMergeChunksPerWave; ++u)
    a0[u] = (u < nj && live) ? src[int64_t(j0 + u) * stride + 4 + d] : 0.f;
  const float m = group_all<1>(mj, [](float x, float y) { return fmaxf(x, y); });
  if (lane == 0) wmax[w] = m;
  __syncthreads();
  float M = wmax[0];
  for (int u = 1; u < nw; ++u) M = fmaxf(M, wmax[u]);
  if (M == -INFINITY) {  // no attended cell
    if (w == 0 && live) o[d] = 0.f;
    return;  // uniform across the workgroup
  }
  const float e = mj == -INFINITY ? 0.f : expf(mj - M);  // empty chunks weigh 0
  if (lane < nj) ew[j0 + lane] = e;
  const float L = group_all<1>(lj * e, [](float x, float y) { return x + y; });
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's weights are in LDS
  __builtin_amdgcn_wave_barrier();

  // Value sums over this wave's chunks, in chunk order.
  float acc0 = 0.f;
#pragma unroll
  for (int u = 0; u < kMergeChunksPerWave; ++u) {
    const float eu = u < nj ? ew[j0 + u] : 0.f;
    acc0 = __builtin_fmaf(a0[u], eu, acc0);
  }
  if (lane == 0) red[w][0] = L;
  red[w][2 + lane] = acc0;
  __syncthreads();
  if (w == 0) {
    float Lt = red[0][0], s0 = red[0][2 + lane];
    for (int u = 1; u < nw; ++u) {
      Lt += red[u][0];
      s0 += red[u][2 + lane];
    }
    if (live) o[d] = s0 / Lt;
  }
}

template <int LPC, int CB>
hipError_t launch_chunks(const float *q, const float *kc, const float *vc, const int *ids, int nq,
                         int heads, int dim, int k, int n_cells, float scale, float *part,
                         int nchunks, hipStream_t stream) {
  if constexpr (4 * CB / (64 / LPC) > 16) {
    return hipErrorInvalidValue;  // more rows than registers: never chosen
  } else {
    attn_chunk_kernel<LPC, CB><<<dim3(nchunks, heads, nq), 64, 0, stream>>>(
        q, kc, vc, ids, heads, dim, k, n_cells, scale, part, nchunks);
    return hipGetLastError();
  }
}

template <int CB>
hipError_t chunks_f32(int lpc, const float *q, const float *kc, const float *vc, const int *ids,
                      int nq, int heads, int dim, int k, int n_cells, float scale, float *part,
                      int nchunks, hipStream_t stream) {
  switch (lpc) {
    case 1: return launch_chunks<1, CB>(q, kc, vc, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream);
    case 2: return launch_chunks<2, CB>(q, kc, vc, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream);
    case 4: return launch_chunks<4, CB>(q, kc, vc, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream);
    case 8: return launch_chunks<8, CB>(q, kc, vc, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream);
    case 16: return launch_chunks<16, CB>(q, kc, vc, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream);
    default: return launch_chunks<32, CB>(q, kc, vc, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream);
  }
}

template <int LPC, int CB>
hipError_t launch_chunks_i8(const float *q, const int8_t *kq, const uint16_t *ks,
                            const int8_t *vq, const uint16_t *vs, const int *ids, int nq,
                            int heads, int dim, int k, int n_cells, float scale, float *part,
                            int nchunks, hipStream_t stream) {
  if constexpr (4 * CB / (64 / LPC) > 16) {
    return hipErrorInvalidValue;  // more rows than registers: never chosen
  } else {
    attn_chunk_i8_kernel<LPC, CB><<<dim3(nchunks, heads, nq), 64, 0, stream>>>(
        q, kq, ks, vq, vs, ids, heads, dim, k, n_cells, scale, part, nchunks);
    return hipGetLastError();
  }
}

template <int CB>
hipError_t chunks_i8(int lpc, const float *q, const int8_t *kq, const uint16_t *ks,
                     const int8_t *vq, const uint16_t *vs, const int *ids, int nq, int heads,
                     int dim, int k, int n_cells, float scale, float *part, int nchunks,
                     hipStream_t stream) {
  switch (lpc) {
    case 1: return launch_chunks_i8<1, CB>(q, kq, ks, vq, vs, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream);
    case 2: return launch_chunks_i8<2, CB>(q, kq, ks, vq, vs, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream);
    case 4: return launch_chunks_i8<4, CB>(q, kq, ks, vq, vs, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream);
    default: return launch_chunks_i8<8, CB>(q, kq, ks, vq, vs, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream);
  }
}

// Listed blocks per chunk wave: 4 up to k = 1024 (at most 256 chunks per
// (query, head)); above, 8, or 16 when 8 would give more than 4096 chunk
// waves in all and 16 blocks' rows fit 128 VGPRs of loads in flight (4 * 16
// cells over 64 / lpc cells per load, at most 16 loads of keys and 16 of
// values).  Measured with the two-workgroup merge (attention call, graph
// replay, 4 heads): 4 blocks at k = 512 (-1.0 us fp32, -1.0 us int8 against
// 8); at k = 2048, 8 (4 is 1 us slower for one query, 1.3-3 us for four);
// at k = 4096 with int8 codes, 8 for one query (15.0 against 15.9 us) and 16
// for four (23.7 against 26.0 us).  Every choice keeps nchunks within
// kMergeMaxChunks for k <= 4096.
int chunk_blocks(int nq, int heads, int k, int lpc) {
  if (k <= 1024) return 4;
  const int64_t waves8 = int64_t(nq) * heads * ((k + 7) / 8);
  if (waves8 > 4096 && 4 * 16 * lpc / 64 <= 16) return 16;
  return 8;
}

// Chunk partials of nq * heads * nchunks chunks from the stream's scratch.
hipError_t chunk_partials(hipStream_t stream, int nq, int heads, int dim, int k, int cb,
                          int *nchunks, float **part) {
  *nchunks = k > 0 ? (k + cb - 1) / cb : 1;
  if (*nchunks > kMergeMaxChunks) return hipErrorInvalidValue;  // never chosen
  void *ws = nullptr;
  hipError_t e =
      workspace(stream, size_t(nq) * heads * *nchunks * (dim + 4) * sizeof(float), &ws);
  *part = static_cast<float *>(ws);
  return e;
}

hipError_t launch_merge(const float *part, int nq, int heads, int dim, int nchunks, float *out,
                        hipStream_t stream) {
  const int nw = (nchunks + kMergeChunksPerWave - 1) / kMergeChunksPerWave;
  attn_merge_kernel<<<dim3(heads, nq, (dim + 63) / 64), 64 * nw, 0, stream>>>(part, heads, dim,
                                                                             nchunks, out);
  return hipGetLastError();
}

}  // namespace

bool attn_dim_ok(int dim) { return dim >= 4 && dim % 4 == 0 && dim <= kAttnMaxDim; }
bool attn_i8_dim_ok(int dim) { return dim >= 16 && dim % 16 == 0 && dim <= kAttnMaxDim; }

hipError_t launch_sparse_decode_attention(const float *q, const float *kc, const float *vc,
                                          const int *ids, int nq, int heads, int dim, int k,
                                          int n_cells, float scale, float *out,
                                          hipStream_t stream) {
  const int lpc = dim <= 4 ? 1 : dim <= 8 ? 2 : dim <= 16 ? 4 : dim <= 32 ? 8 : dim <= 64 ? 16 : 32;
  const int cb = chunk_blocks(nq, heads, k, lpc);
  int nchunks = 0;
  float *part = nullptr;
  hipError_t e = chunk_partials(stream, nq, heads, dim, k, cb, &nchunks, &part);
  if (e != hipSuccess) return e;
  switch (cb) {
    case 4: e = chunks_f32<4>(lpc, q, kc, vc, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream); break;
    case 16: e = chunks_f32<16>(lpc, q, kc, vc, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream); break;
    default: e = chunks_f32<8>(lpc, q, kc, vc, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream); break;
  }
  if (e != hipSuccess) return e;
  return launch_merge(part, nq, heads, dim, nchunks, out, stream);
}

hipError_t launch_sparse_decode_attention_i8(const float *q, const int8_t *kq,
                                             const uint16_t *ks, const int8_t *vq,
                                             const uint16_t *vs, const int *ids, int nq,
                                             int heads, int dim, int k, int n_cells,
                                             float scale, float *out, hipStream_t stream) {
  const int lpc = dim <= 16 ? 1 : dim <= 32 ? 2 : dim <= 64 ? 4 : 8;
  const int cb = chunk_blocks(nq, heads, k, lpc);
  int nchunks = 0;
  float *part = nullptr;
  hipError_t e = chunk_partials(stream, nq, heads, dim, k, cb, &nchunks, &part);
  if (e != hipSuccess) return e;
  switch (cb) {
    case 4: e = chunks_i8<4>(lpc, q, kq, ks, vq, vs, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream); break;
    case 16: e = chunks_i8<16>(lpc, q, kq, ks, vq, vs, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream); break;
    default: e = chunks_i8<8>(lpc, q, kq, ks, vq, vs, ids, nq, heads, dim, k, n_cells, scale, part, nchunks, stream); break;
  }
  if (e != hipSuccess) return e;
  return launch_merge(part, nq, heads, dim, nchunks, out, stream);
}

}  // namespace qsa
