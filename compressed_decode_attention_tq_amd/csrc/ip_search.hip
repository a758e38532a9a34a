// Approximate inner-product nearest-neighbour search over a quantized database ([tq-80]
// §技术背景与学术渊源: the quantizer also serves approximate nearest-neighbour search, its
// codebook being data-independent, so indexing is just quantizing).  The score of database
// vector t for query j is q_j . x_hat_t = n16_t * (R q_j) . c[idx_t]: the decode score of
// the packed keys without the softmax ([google], the scoring kernel).
//
// Launches:
//   ip_score_kernel   the scores of up to 8 queries (one workgroup row of blockIdx.y per
//                     group of 8) against kBlockTokens database vectors per workgroup, on
//                     matrix cores: queries are the rows of v_mfma_f32_16x16x32_f16 (fp16
//                     value and remainder rows, as in the decode kernel), 16 vectors its
//                     columns.  The scores stay in LDS; wave h then takes query h's k best,
//                     highest score first, equal scores by lowest index, by taking the best
//                     k times (wave-wide max of the key, then min index).
//   topk_merge_kernel per query, kChunkScores candidates per block to k, repeated until one
//                     block holds them all (two levels for 2^20 vectors at k = 10).  Small
//                     slices keep each lane's share short: a round's cost is one lane
//                     re-scanning its entries.
#include "tq_common.h"
#include "tq_launch.h"
#include "lanes.h"

#include <utility>

namespace tq {
namespace {

typedef _Float16 half8s __attribute__((ext_vector_type(8)));
typedef float floatx4s __attribute__((ext_vector_type(4)));

constexpr int kScoreWaves = 8;
constexpr int kChunkScores = 1024;  // candidates per merge block
constexpr int kBlockTokens = kSearchBlock;  // database vectors per score workgroup (scores kept in LDS)
constexpr int kTopkThreads = 256;

__device__ __forceinline__ uint16_t h16s(float x) { return __half_as_ushort(__float2half_rn(x)); }
__device__ __forceinline__ float f16s(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Order-preserving unsigned key of a float: a larger float has a larger key, and every
// finite score has a key above 0, which marks an empty or taken slot.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Wave-wide integer max / min with the lane exchanges of lanes.h: DPP quad permutes and row
// rotations within 16 lanes, then the permlane swaps of rows and halves.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_int(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : (uint32_t)min((int)a, (int)b); };
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor2, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppRowRor4, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppRowRor8, 0xF, 0xF, false));
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r32[0], r32[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_reduce_int<true>(v); }
__device__ __forceinline__ int wave_min_i32(int v) { return (int)wave_reduce_int<false>((uint32_t)v); }

// The k best of the entries a wave holds (kPer per lane: key, index), best first: highest
// key, then lowest index.  Each round the wave's best is found from the lanes' own bests;
// only the lane that gave it up looks at its entries again.  Results go to out_k / out_i
// (k slots; 0 / -1 once the entries run out).
template <int kPer>
__device__ void wave_select(uint32_t (&key)[kPer], int (&idx)[kPer], int k, int lane, uint32_t *out_k, int *out_i) {
  uint32_t bk = 0u;
  int bi = 0x7fffffff;
  auto lane_best = [&]() {
    bk = 0u;
    bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (key[j] > bk || (key[j] == bk && key[j] != 0u && idx[j] < bi)) {
        bk = key[j];
        bi = idx[j];
      }
  };
  lane_best();
  for (int r = 0; r < k; ++r) {
    const uint32_t mk = wave_max_u32(bk);
    const int mi = wave_min_i32(bk == mk ? bi : 0x7fffffff);
    if (lane == 0) {
      out_k[r] = mk;
      out_i[r] = mk == 0u ? -1 : mi;
    }
    if (mk == 0u) continue;
    if (bk == mk && bi == mi) {  // the one lane that held it
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (key[j] == mk && idx[j] == mi) key[j] = 0u;
      lane_best();
    }
  }
}

// The k best of kPer entries per lane, as wave_select, with a prefilter: the k-th largest of
// the 64 lane maxima is a lower bound of the k-th largest entry (k lanes hold an entry at
// least that large), so only entries at or above it can be among the k best.  When at most
// 64 pass, they are compacted through `scratch` (64 keys + 64 indices of LDS) to one per lane
// and the rounds no longer re-scan kPer entries; otherwise the plain selection runs.
template <int kPer>
__device__ void wave_select_pruned(uint32_t (&key)[kPer], int (&idx)[kPer], int k, int lane, uint32_t *scratch,
                                   uint32_t *out_k, int *out_i) {
  uint32_t lm = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) lm = max(lm, key[j]);
  uint32_t v = lm, theta = 0u;
  for (int r = 0; r < k && r < 64; ++r) {  // the k-th largest lane maximum
    theta = wave_max_u32(v);
    const uint64_t at = __ballot(v == theta);
    if (lane == __ffsll((unsigned long long)at) - 1) v = 0u;
  }
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) cnt += (key[j] != 0u && key[j] >= theta) ? 1 : 0;
  // exclusive prefix of the counts over the lanes
  int incl = cnt;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m);
    if (lane >= m) incl += o;
  }
  const int total = __shfl(incl, 63);
  if (total > 64) {  // many entries tie with the bound: select over all of them
    wave_select<kPer>(key, idx, k, lane, out_k, out_i);
    return;
  }
  int pos = incl - cnt;
  uint32_t *sk = scratch;
  int *si = reinterpret_cast<int *>(scratch + 64);
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (key[j] != 0u && key[j] >= theta) {
      sk[pos] = key[j];
      si[pos] = idx[j];
      ++pos;
    }
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
  uint32_t k1[1] = {lane < total ? sk[lane] : 0u};
  int i1[1] = {lane < total ? si[lane] : 0x7fffffff};
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
  wave_select<1>(k1, i1, k, lane, out_k, out_i);
}

constexpr int kSelWaves = kTopkThreads / 64;
constexpr int kSelPer = kChunkScores / kTopkThreads;  // entries per lane

// Block top-k of n (key, index) entries read by `get` (i -> {key, index}), best first, into
// out_k / out_i (k slots): every wave selects from its slice, then wave 0 from the waves' k
// bests each.
template <typename Get>
__device__ void block_select(int n, int k, Get get, uint32_t *wk, int *wi, uint32_t *out_k, int *out_i) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  {
    uint32_t key[kSelPer];
    int idx[kSelPer];
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      const int i = (wave * kSelPer + j) * 64 + lane;  // coalesced: lanes take neighbours
      key[j] = 0u;
      idx[j] = 0x7fffffff;
      if (i < n) get(i, key[j], idx[j]);
    }
    wave_select<kSelPer>(key, idx, k, lane, wk + wave * kSearchMaxK, wi + wave * kSearchMaxK);
  }
  __syncthreads();
  if (wave == 0) {
    constexpr int kPer2 = kSelWaves * kSearchMaxK / 64;
    uint32_t key[kPer2];
    int idx[kPer2];
#pragma unroll
    for (int j = 0; j < kPer2; ++j) {
      const int e = j * 64 + lane, w = e / kSearchMaxK, r = e % kSearchMaxK;
      key[j] = r < k ? wk[w * kSearchMaxK + r] : 0u;
      idx[j] = r < k ? wi[w * kSearchMaxK + r] : 0x7fffffff;
      if (key[j] == 0u) idx[j] = 0x7fffffff;
    }
    wave_select<kPer2>(key, idx, k, lane, out_k, out_i);
  }
}

// Table entry e of two codes a = e mod L, b = e div L (L = 2^BK): {hi(c_a) | hi(c_b) << 16,
// lo(c_a) | lo(c_b) << 16}, hi = the fp16 value of the centroid and lo = the fp16 remainder.
// A byte of 4-bit codes (a 6-bit field of 3-bit codes) is one entry: coordinates 2j, 2j+1.
template <int BK>
// Workgroup x of query group y scores vectors [x kBlockTokens, (x + 1) kBlockTokens) into LDS,
// then wave h takes the k best of query h's scores (best first) as the block's candidates
// cand_s / cand_i [query][block][k].
__global__ __launch_bounds__(64 * kScoreWaves) void ip_score_kernel(CacheView db, const void *__restrict__ q,
                                                                   int q_dtype, int n_q, int n, int k, float *cand_s,
                                                                   int32_t *cand_i) {
  constexpr int L = 1 << BK, KROW = 16 * BK;
  constexpr int kTilesPerBlock = kBlockTokens / 16;
  __shared__ uint2 tab[L * L];
  __shared__ float qrot[8][kD];
  __shared__ float sc[8][kBlockTokens];
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
  const int s_begin = blockIdx.x * kTilesPerBlock, s_end = min(s_begin + kTilesPerBlock, n_sub);
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
    const int ha = 2 * quarter, hb = ha + 1, c = (sub - s_begin) * 16 + row;
    sc[ha][c] = (acc[0] + acc[1]) * nrm;
    sc[hb][c] = (acc[2] + acc[3]) * nrm;
  }
  __syncthreads();
  if (wave < nq) {  // the block's k best for query q0 + wave; vectors past n hold no entry
    constexpr int kPer = kBlockTokens / 64;
    const int t0 = blockIdx.x * kBlockTokens;
    uint32_t key[kPer];
    int idx[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = j * 64 + lane;
      const bool live = t0 + c < n;
      key[j] = live ? order_key(sc[wave][c]) : 0u;
      idx[j] = live ? t0 + c : 0x7fffffff;
    }
    uint32_t *ok = reinterpret_cast<uint32_t *>(&sc[wave][0]);  // this wave's row is free now
    int *oi = reinterpret_cast<int *>(&sc[wave][kSearchMaxK]);
    wave_select_pruned<kPer>(key, idx, k, lane, reinterpret_cast<uint32_t *>(&sc[wave][2 * kSearchMaxK]), ok, oi);
    const size_t o = ((size_t)(q0 + wave) * gridDim.x + blockIdx.x) * k;
    for (int r = lane; r < k; r += 64) {
      cand_s[o + r] = ok[r] == 0u ? -INFINITY : key_value(ok[r]);
      cand_i[o + r] = oi[r];
    }
  }
}


// Block (x, query j) takes candidates [x kChunkScores, ...) of the query's n_cand and writes
// their k best, best first, to out_s / out_i [query][gridDim.x][k].
__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(const float *__restrict__ cand_s,
                                                                 const int32_t *__restrict__ cand_i, int n_cand, int k,
                                                                 int32_t *out_idx, float *out_score) {
  __shared__ uint32_t wk[kSelWaves * kSearchMaxK];
  __shared__ int wi[kSelWaves * kSearchMaxK];
  __shared__ uint32_t ok[kSearchMaxK];
  __shared__ int oi[kSearchMaxK];
  const int j = blockIdx.y;
  const int base = blockIdx.x * kChunkScores;
  const float *cs = cand_s + (size_t)j * n_cand + base;
  const int32_t *ci = cand_i + (size_t)j * n_cand + base;
  block_select(min(kChunkScores, n_cand - base), k,
               [&](int i, uint32_t &key, int &idx) {
                 idx = ci[i];
                 key = idx < 0 ? 0u : order_key(cs[i]);  // an empty candidate slot
                 if (idx < 0) idx = 0x7fffffff;
               },
               wk, wi, ok, oi);
  __syncthreads();
  const size_t o = ((size_t)j * gridDim.x + blockIdx.x) * k;
  for (int r = threadIdx.x; r < k; r += kTopkThreads) {  // already best first
    out_idx[o + r] = oi[r];
    out_score[o + r] = ok[r] == 0u ? -INFINITY : key_value(ok[r]);
  }
}

}  // namespace

hipError_t launch_ip_search(const CacheView &db, const void *q, int q_dtype, int n_q, int n, int k, int32_t *out_idx,
                            float *out_score, float *cand_s0, int32_t *cand_i0, float *cand_s1, int32_t *cand_i1,
                            hipStream_t stream) {
  const int blocks = (n + kBlockTokens - 1) / kBlockTokens;
  const dim3 g1(blocks, (n_q + 7) / 8);
  if (db.bits == 4) ip_score_kernel<4><<<g1, 64 * kScoreWaves, 0, stream>>>(db, q, q_dtype, n_q, n, k, cand_s0, cand_i0);
  else ip_score_kernel<3><<<g1, 64 * kScoreWaves, 0, stream>>>(db, q, q_dtype, n_q, n, k, cand_s0, cand_i0);
  hipError_t e = hipGetLastError();
  // merge levels: each block reduces kChunkScores candidates to k, until one block is left
  long n_cand = (long)blocks * k;
  float *src_s = cand_s0, *dst_s = cand_s1;
  int32_t *src_i = cand_i0, *dst_i = cand_i1;
  while (e == hipSuccess) {
    const int groups = (int)((n_cand + kChunkScores - 1) / kChunkScores);
    const bool last = groups == 1;
    topk_merge_kernel<<<dim3(groups, n_q), kTopkThreads, 0, stream>>>(src_s, src_i, (int)n_cand, k,
                                                                     last ? out_idx : dst_i, last ? out_score : dst_s);
    e = hipGetLastError();
    if (last) break;
    n_cand = (long)groups * k;
    std::swap(src_s, dst_s);
    std::swap(src_i, dst_i);
  }
  return e;
}

}  // namespace tq
