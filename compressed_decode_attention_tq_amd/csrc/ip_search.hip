// Approximate inner-product nearest-neighbour search over a quantized database ([tq-80]
// §技术背景与学术渊源: the quantizer also serves approximate nearest-neighbour search, its
// codebook being data-independent, so indexing is just quantizing).  The score of database
// vector t for query j is q_j . x_hat_t = n16_t * (R q_j) . c[idx_t]: the decode score of
// the packed keys without the softmax ([google], the scoring kernel).
//
// Three launches:
//   ip_score_kernel   the scores of up to 8 queries (one workgroup column of blockIdx.y per
//                     group of 8) against the database, on matrix cores: queries are the
//                     rows of v_mfma_f32_16x16x32_f16 (fp16 value and remainder rows, as in
//                     the decode kernel), 16 database vectors its columns; written to HBM.
//   topk_chunk_kernel per (query, chunk of kChunkScores scores): the chunk's k best, found
//                     by a radix select in LDS, written in index order.
//   topk_merge_kernel per query: the same selection over the chunks' candidates, then the
//                     k results ranked by descending score, ties by ascending index.
#include "tq_common.h"
#include "tq_launch.h"
#include "lanes.h"

namespace tq {
namespace {

typedef _Float16 half8s __attribute__((ext_vector_type(8)));
typedef float floatx4s __attribute__((ext_vector_type(4)));

constexpr int kScoreWaves = 8;
constexpr int kChunkScores = 8192;  // scores per top-k block
constexpr int kTopkThreads = 256;

__device__ __forceinline__ uint16_t h16s(float x) { return __half_as_ushort(__float2half_rn(x)); }
__device__ __forceinline__ float f16s(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Table entry e of two codes a = e mod L, b = e div L (L = 2^BK): {hi(c_a) | hi(c_b) << 16,
// lo(c_a) | lo(c_b) << 16}, hi = the fp16 value of the centroid and lo = the fp16 remainder.
// A byte of 4-bit codes (a 6-bit field of 3-bit codes) is one entry: coordinates 2j, 2j+1.
template <int BK>
__global__ __launch_bounds__(64 * kScoreWaves) void ip_score_kernel(CacheView db, const void *__restrict__ q,
                                                                   int q_dtype, int n_q, int n, float *scores,
                                                                   int tiles_per_block) {
  constexpr int L = 1 << BK, KROW = 16 * BK;
  __shared__ uint2 tab[L * L];
  __shared__ float qrot[8][kD];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q0 = blockIdx.y * 8;                 // first query of this group
  const int nq = min(8, n_q - q0);

  for (int e = threadIdx.x; e < L * L; e += blockDim.x) {
    const float ca = db.centroids[e % L], cb = db.centroids[e / L];
    const uint16_t ha = h16s(ca), hb = h16s(cb);
    tab[e] = make_uint2((uint32_t)ha | ((uint32_t)hb << 16),
                        (uint32_t)h16s(ca - f16s(ha)) | ((uint32_t)h16s(cb - f16s(hb)) << 16));
  }
  if (wave < nq) {  // wave h rotates query q0 + h: R q = H (s . q) / sqrt(d)
    const size_t qi = (size_t)(q0 + wave) * kD + 2 * lane;
    float x0 = load_elem(q, qi, q_dtype), x1 = load_elem(q, qi + 1, q_dtype);
    if (db.signs[2 * lane] < 0) x0 = -x0;
    if (db.signs[2 * lane + 1] < 0) x1 = -x1;
    float u0 = x0 + x1, u1 = x0 - x1;
    wave_fwht_upper(u0, u1, lane);
    qrot[wave][2 * lane] = u0 * 0.08838834764831845f;
    qrot[wave][2 * lane + 1] = u1 * 0.08838834764831845f;
  }
  __syncthreads();

  // A operands: lane row r = lane % 16 is query r / 2, its fp16 part (r even) or remainder;
  // product m covers coordinates 32 quarter + 4m .. + 3 in the pattern (a, b, a, b, c, d, c, d)
  // that meets the table's {hi a, hi b, lo a, lo b, hi c, hi d, lo c, lo d}.
  const int row = lane & 15, quarter = lane >> 4, h = row >> 1;
  half8s aop[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    _Float16 p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = h < nq ? qrot[h][32 * quarter + 4 * m + j] : 0.f;
      const _Float16 hi = (_Float16)v;
      p[j] = (row & 1) ? (_Float16)(v - (float)hi) : hi;
    }
    aop[m] = half8s{p[0], p[1], p[0], p[1], p[2], p[3], p[2], p[3]};
  }

  const uint8_t *plane = db.plane(0, 0);
  const uint16_t *norms = db.norm_plane(0, 0);
  const int n_sub = (n + 15) / 16;
  const int s_begin = blockIdx.x * tiles_per_block, s_end = min(s_begin + tiles_per_block, n_sub);
  for (int sub = s_begin + wave; sub < s_end; sub += kScoreWaves) {
    const int t = sub * 16 + row;                 // this lane's database vector (column)
    const bool live = t < n;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    float nrm = 0.f;
    if (live) {
      const uint8_t *src = plane + (size_t)t * KROW + quarter * (4 * BK);
      if (BK == 4) {
        const uint4 v = *reinterpret_cast<const uint4 *>(src);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      } else {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(src);
        w[0] = p[0]; w[1] = p[1]; w[2] = p[2];
      }
      nrm = f16s(norms[t]);
    }
    floatx4s acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint32_t e0, e1;  // the entries of coordinates (4m, 4m+1) and (4m+2, 4m+3) of the quarter
      if (BK == 4) {
        e0 = (w[m >> 1] >> (16 * (m & 1))) & 0xffu;
        e1 = (w[m >> 1] >> (16 * (m & 1) + 8)) & 0xffu;
      } else {
        const int b0 = 12 * m, b1 = 12 * m + 6;
        e0 = (b0 & 31) <= 26 ? (w[b0 >> 5] >> (b0 & 31)) & 63u
                             : ((w[b0 >> 5] >> (b0 & 31)) | (w[(b0 >> 5) + 1] << (32 - (b0 & 31)))) & 63u;
        e1 = (b1 & 31) <= 26 ? (w[b1 >> 5] >> (b1 & 31)) & 63u
                             : ((w[b1 >> 5] >> (b1 & 31)) | (w[(b1 >> 5) + 1] << (32 - (b1 & 31)))) & 63u;
      }
      const uint2 x = tab[e0], y = tab[e1];
      const uint32_t bw[4] = {x.x, x.y, y.x, y.y};
      half8s bop;
      __builtin_memcpy(&bop, bw, 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[m], bop, acc, 0, 0, 0);
    }
    // output rows 4 quarter .. + 3 of column `row`: queries 2 quarter (fp16 + remainder rows)
    // and 2 quarter + 1, for the database vector of this lane
    const int ha = 2 * quarter, hb = ha + 1;
    if (live) {
      if (ha < nq) scores[(size_t)(q0 + ha) * n + t] = (acc[0] + acc[1]) * nrm;
      if (hb < nq) scores[(size_t)(q0 + hb) * n + t] = (acc[2] + acc[3]) * nrm;
    }
  }
}

// Order-preserving unsigned key of a float: a larger float has a larger key.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Block prefix sum (exclusive) of one count per thread; returns the thread's offset and
// leaves the total in *total.
__device__ int block_exclusive_scan(int v, int *tmp, int *total) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int off = 1; off < kTopkThreads; off <<= 1) {
    const int add = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  const int incl = tmp[tid];
  *total = tmp[kTopkThreads - 1];
  __syncthreads();
  return incl - v;
}

// Selects the k best of cnt (score, index) pairs staged in index order in LDS and writes them
// in that order to out_s / out_i (k entries; missing ones as -inf / -1).  Radix select of the
// k-th largest key, 8 bits at a time from the top; among keys equal to it the lowest staged
// positions are taken.  Each thread owns a contiguous run of staged entries.
__device__ void block_topk(const float *sc, const int32_t *ix, int cnt, int k, float *out_s, int32_t *out_i,
                           int *hist, int *tmp) {
  const int tid = threadIdx.x;
  const int per = (cnt + kTopkThreads - 1) / kTopkThreads;
  const int lo = min(tid * per, cnt), hi = min(lo + per, cnt);
  const int kk = min(k, cnt);
  uint32_t prefix = 0u, mask = 0u;
  int remaining = kk;  // how many still to take at or below the current prefix
  for (int digit = 3; digit >= 0 && kk > 0; --digit) {
    for (int b = tid; b < 256; b += kTopkThreads) hist[b] = 0;
    __syncthreads();
    for (int i = lo; i < hi; ++i) {
      const uint32_t key = order_key(sc[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> (8 * digit)) & 0xffu], 1);
    }
    __syncthreads();
    if (tid == 0) {  // the digit holding the remaining-th largest
      int above = 0, b = 255;
      for (; b > 0; --b) {
        if (above + hist[b] >= remaining) break;
        above += hist[b];
      }
      tmp[kTopkThreads] = b;
      tmp[kTopkThreads + 1] = remaining - above;
    }
    __syncthreads();
    prefix |= (uint32_t)tmp[kTopkThreads] << (8 * digit);
    mask |= 0xffu << (8 * digit);
    remaining = tmp[kTopkThreads + 1];
    __syncthreads();
  }
  // keys above the k-th are all taken; of the keys equal to it, the first `remaining`
  int n_eq = 0;
  for (int i = lo; i < hi; ++i) n_eq += (kk > 0 && order_key(sc[i]) == prefix) ? 1 : 0;
  int tot_eq;
  int eq_rank = block_exclusive_scan(n_eq, tmp, &tot_eq);
  int n_take = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = order_key(sc[i]);
    if (kk > 0 && (key > prefix || (key == prefix && eq_rank++ < remaining))) ++n_take;
  }
  int tot_take;
  int pos = block_exclusive_scan(n_take, tmp, &tot_take);
  eq_rank = block_exclusive_scan(n_eq, tmp, &tot_eq);
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = order_key(sc[i]);
    if (kk > 0 && (key > prefix || (key == prefix && eq_rank++ < remaining))) {
      out_s[pos] = sc[i];
      out_i[pos] = ix[i];
      ++pos;
    }
  }
  for (int i = tot_take + tid; i < k; i += kTopkThreads) {
    out_s[i] = -INFINITY;
    out_i[i] = -1;
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_chunk_kernel(const float *__restrict__ scores, int n, int k,
                                                                 float *cand_s, int32_t *cand_i, int n_chunks) {
  __shared__ float sc[kChunkScores];
  __shared__ int32_t ix[kChunkScores];
  __shared__ int hist[256];
  __shared__ int tmp[kTopkThreads + 2];
  const int chunk = blockIdx.x, j = blockIdx.y;
  const int base = chunk * kChunkScores, cnt = min(kChunkScores, n - base);
  for (int i = threadIdx.x; i < cnt; i += kTopkThreads) {
    sc[i] = scores[(size_t)j * n + base + i];
    ix[i] = base + i;
  }
  __syncthreads();
  const size_t o = ((size_t)j * n_chunks + chunk) * k;
  block_topk(sc, ix, cnt, k, cand_s + o, cand_i + o, hist, tmp);
}

__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(const float *__restrict__ cand_s,
                                                                 const int32_t *__restrict__ cand_i, int n_cand, int k,
                                                                 int32_t *out_idx, float *out_score) {
  __shared__ float sc[kChunkScores];
  __shared__ int32_t ix[kChunkScores];
  __shared__ float bs[64];
  __shared__ int32_t bi[64];
  __shared__ int hist[256];
  __shared__ int tmp[kTopkThreads + 2];
  const int j = blockIdx.x;
  // chunks' candidates in chunk order: every chunk's list is in index order, so the staging
  // is in index order (the empty slots, -inf with index -1, sort last)
  for (int i = threadIdx.x; i < n_cand; i += kTopkThreads) {
    sc[i] = cand_s[(size_t)j * n_cand + i];
    ix[i] = cand_i[(size_t)j * n_cand + i];
  }
  __syncthreads();
  block_topk(sc, ix, n_cand, k, bs, bi, hist, tmp);
  __syncthreads();
  // rank the k results: descending score, ascending index on ties (no index -1 is ever
  // ahead of a real one, since its score is -inf)
  for (int a = threadIdx.x; a < k; a += kTopkThreads) {
    const float s = bs[a];
    const int32_t id = bi[a];
    int rank = 0;
    for (int b = 0; b < k; ++b) {
      const float t = bs[b];
      const int32_t tb = bi[b];
      const bool ahead = t > s || (t == s && ((tb >= 0 && (id < 0 || tb < id)) || (tb == id && b < a)));
      rank += ahead ? 1 : 0;
    }
    out_idx[(size_t)j * k + rank] = id;
    out_score[(size_t)j * k + rank] = s;
  }
}

}  // namespace

hipError_t launch_ip_search(const CacheView &db, const void *q, int q_dtype, int n_q, int n, int k, int32_t *out_idx,
                            float *out_score, float *scores, float *cand_s, int32_t *cand_i, hipStream_t stream) {
  const int n_sub = (n + 15) / 16;
  const int n_cu = compute_units();
  const int blocks = min(n_sub, max(1, 2 * n_cu));
  const int tiles_per_block = (n_sub + blocks - 1) / blocks;
  const dim3 g1((n_sub + tiles_per_block - 1) / tiles_per_block, (n_q + 7) / 8);
  if (db.bits == 4) ip_score_kernel<4><<<g1, 64 * kScoreWaves, 0, stream>>>(db, q, q_dtype, n_q, n, scores, tiles_per_block);
  else ip_score_kernel<3><<<g1, 64 * kScoreWaves, 0, stream>>>(db, q, q_dtype, n_q, n, scores, tiles_per_block);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_chunks = (n + kChunkScores - 1) / kChunkScores;
  topk_chunk_kernel<<<dim3(n_chunks, n_q), kTopkThreads, 0, stream>>>(scores, n, k, cand_s, cand_i, n_chunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  topk_merge_kernel<<<n_q, kTopkThreads, 0, stream>>>(cand_s, cand_i, n_chunks * k, k, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace tq
