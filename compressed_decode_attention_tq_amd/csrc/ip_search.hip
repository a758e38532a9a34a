// Approximate inner-product nearest-neighbour search over a quantized database ([tq-80]
// §技术背景与学术渊源: the quantizer also serves approximate nearest-neighbour search, its
// codebook being data-independent, so indexing is just quantizing).  The score of database
// vector t for query j is q_j . x_hat_t = n16_t * (R q_j) . c[idx_t]: the decode score of
// the packed keys without the softmax ([google], the scoring kernel).
//
// Launches:
//   ip_score_kernel    workgroup x of query group y (up to 8 queries) scores kBlockTokens
//                      database vectors on matrix cores: the queries are the rows of
//                      v_mfma_f32_16x16x32_f16 (fp16 value and remainder rows, as in the
//                      decode kernel), 16 vectors its columns.  The scores stay in LDS; wave h
//                      then ranks query h's: the k-th largest of its 64 lane maxima bounds the
//                      block's k-th best from below, the (normally few) scores reaching it are
//                      sorted across the lanes, and the first k are the block's candidates.
//   topk_final_kernel  one workgroup per query.  Two keys that k scores reach bound the
//                      query's k-th best from below: the largest block k-th best, and the k-th
//                      largest of the lanes' maxima over block bests.  Only candidates reaching
//                      the larger bound are ranked; normally at most 64, sorted at once.
// Ranking order everywhere: higher score first, equal scores by lower index, as one 64-bit
// unsigned comparison of key << 32 | ~index, sorted across a wave's lanes by a bitonic network
// of lane exchanges; longer lists are kept to their best 64 by merging sorted runs.
#include "tq_common.h"
#include "tq_launch.h"
#include "lanes.h"

namespace tq {
namespace {

typedef _Float16 half8s __attribute__((ext_vector_type(8)));
typedef float floatx4s __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kScoreWaves = 8;
constexpr int kBlockTokens = kSearchBlock;  // database vectors per score workgroup (scores kept in LDS)
constexpr int kFinalWaves = 16;  // waves of the final workgroup
constexpr int kFinalRows = 12;   // candidate rows of 64 in flight per wave
constexpr int kBoundLoads = 16;  // block bounds in flight per lane

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

// Wave-wide unsigned max with the lane exchanges of lanes.h: DPP quad permutes and row
// rotations within 16 lanes, then the permlane swaps of rows and halves.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppQuadXor2, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppRowRor4, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppRowRor8, 0xF, 0xF, false));
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(r32[0], r32[1]);
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Ranking across the 64 lanes of a wave, one entry per lane as the 64-bit value
// key << 32 | ~index: entry a comes before b when its key is larger, or the keys are equal and
// its index smaller, which is a > b as unsigned integers.  0 is an empty entry (key 0 marks no
// vector), after every other.
__device__ __forceinline__ uint64_t rank_entry(uint32_t key, int idx) {
  return ((uint64_t)key << 32) | (uint32_t)~idx;
}
__device__ __forceinline__ int entry_index(uint64_t e) { return (int)~(uint32_t)e; }
__device__ __forceinline__ uint32_t entry_key(uint64_t e) { return (uint32_t)(e >> 32); }

// the value of lane (lane xor M), for 32- and 64-bit entries
template <int M, typename T>
__device__ __forceinline__ T lane_xor_t(T v, int lane) {
  if constexpr (sizeof(T) == 4) {
    return __float_as_uint(lane_xor<M>(__uint_as_float(v), lane));
  } else {
    const uint32_t lo = __float_as_uint(lane_xor<M>(__uint_as_float((uint32_t)v), lane));
    const uint32_t hi = __float_as_uint(lane_xor<M>(__uint_as_float((uint32_t)(v >> 32)), lane));
    return ((uint64_t)hi << 32) | lo;
  }
}
// One compare-exchange stage of a bitonic network: blocks of SIZE lanes, partner lane
// (lane xor M).  The lower lane of a pair keeps the larger value in blocks that run in rank
// order (lane 0 first, largest first), the smaller in the others; REV reverses the network's
// final order.
template <int SIZE, int M, bool REV, typename T>
__device__ __forceinline__ void bitonic_step(T &v, int lane) {
  const T p = lane_xor_t<M>(v, lane);
  const bool up = ((lane & SIZE) == 0) != REV;  // SIZE = 64: every lane in one block
  const bool larger = ((lane & M) == 0) == up;
  v = ((p > v) == larger) ? p : v;
}
// Bitonic merge of a bitonic sequence of 64 values into rank order (REV: reversed).
template <bool REV, typename T>
__device__ __forceinline__ void bitonic_merge64(T &v, int lane) {
  bitonic_step<64, 32, REV>(v, lane);
  bitonic_step<64, 16, REV>(v, lane);
  bitonic_step<64, 8, REV>(v, lane);
  bitonic_step<64, 4, REV>(v, lane);
  bitonic_step<64, 2, REV>(v, lane);
  bitonic_step<64, 1, REV>(v, lane);
}
// Sort 64 values into rank order (REV: reversed), 21 compare-exchange stages.
template <bool REV, typename T>
__device__ __forceinline__ void bitonic_sort64(T &v, int lane) {
  bitonic_step<2, 1, REV>(v, lane);
  bitonic_step<4, 2, REV>(v, lane);
  bitonic_step<4, 1, REV>(v, lane);
  bitonic_step<8, 4, REV>(v, lane);
  bitonic_step<8, 2, REV>(v, lane);
  bitonic_step<8, 1, REV>(v, lane);
  bitonic_step<16, 8, REV>(v, lane);
  bitonic_step<16, 4, REV>(v, lane);
  bitonic_step<16, 2, REV>(v, lane);
  bitonic_step<16, 1, REV>(v, lane);
  bitonic_step<32, 16, REV>(v, lane);
  bitonic_step<32, 8, REV>(v, lane);
  bitonic_step<32, 4, REV>(v, lane);
  bitonic_step<32, 2, REV>(v, lane);
  bitonic_step<32, 1, REV>(v, lane);
  bitonic_merge64<REV>(v, lane);
}
// The best 64 of two ranked lists, ranked: v in rank order, r in reversed order.  Lane l's
// larger of (a_l, b_63-l) leaves the best 64 as a bitonic sequence.
__device__ __forceinline__ void merge_best64(uint64_t &v, uint64_t r, int lane) {
  v = r > v ? r : v;
  bitonic_merge64<false, uint64_t>(v, lane);
}

// Workgroup x of query group y scores vectors [x kBlockTokens, (x + 1) kBlockTokens) into LDS,
// then wave h takes the k best of query h's scores (best first) as the block's candidates:
// cand [query][block][k] rank entries (0: no vector), bnd [query][block] the keys of the k-th
// and the best.
// Table entry e of two codes a = e mod L, b = e div L (L = 2^BK): {hi(c_a) | hi(c_b) << 16,
// lo(c_a) | lo(c_b) << 16}, hi = the fp16 value of the centroid and lo = the fp16 remainder.
// A byte of 4-bit codes (a 6-bit field of 3-bit codes) is one entry: coordinates 2j, 2j+1.
template <int BK>
__global__ __launch_bounds__(64 * kScoreWaves) void ip_score_kernel(CacheView db, const void *__restrict__ q,
                                                                   int q_dtype, int n_q, int n, int k,
                                                                   uint64_t *cand, uint2 *bnd) {
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
        // each code word is read once: streaming (nt) loads, 1% faster on a 1M-vector scan
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
      } else {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(src);
        w[0] = __builtin_nontemporal_load(p);
        w[1] = __builtin_nontemporal_load(p + 1);
        w[2] = __builtin_nontemporal_load(p + 2);
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
    uint32_t key[kPer];  // entry j of a lane is vector t0 + 64 j + lane
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = j * 64 + lane;
      key[j] = t0 + c < n ? order_key(sc[wave][c]) : 0u;
    }
    const size_t o = (size_t)(q0 + wave) * gridDim.x + blockIdx.x;
    // The k-th largest lane maximum is reached by k entries (one per lane), so no entry below
    // it is among the k best; normally at most 64 reach it, and one sort ranks them.
    uint32_t lm = 0u;
#pragma unroll
    for (int j = 0; j < kPer; ++j) lm = max(lm, key[j]);
    bitonic_sort64<false>(lm, lane);
    const uint32_t theta = max((uint32_t)__builtin_amdgcn_readlane((int)lm, k - 1), 1u);
    float mine = 0.f;  // entries of this lane that reach the bound (a per-lane count keeps the
                       // ballot masks of the compaction below out of scalar registers)
#pragma unroll
    for (int j = 0; j < kPer; ++j) mine += key[j] >= theta ? 1.f : 0.f;
    const int n_pass = (int)wave_reduce<false>(mine);  // exact: at most 1024
    uint64_t *slot = reinterpret_cast<uint64_t *>(&sc[wave][0]);  // this wave's row is free now
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
    uint64_t v;  // the block's ranked entries, one per lane; lane r < k holds the r-th best
    if (n_pass <= 64) {
      int at = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const bool pass = key[j] >= theta;
        const uint64_t m = __ballot(pass);
        if (pass) slot[at + lanes_below(m)] = rank_entry(key[j], t0 + j * 64 + lane);
        at += __popcll(m);
      }
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");
      v = lane < n_pass ? slot[lane] : 0ull;
      bitonic_sort64<false>(v, lane);
    } else {  // many entries tie with the bound: rank the scores 64 at a time, keep the best 64
      v = 0ull;
#pragma unroll 1
      for (int j = 0; j < kPer; ++j) {
        const int c = j * 64 + lane;
        const uint32_t kc = t0 + c < n ? order_key(sc[wave][c]) : 0u;
        uint64_t r = kc >= theta ? rank_entry(kc, t0 + c) : 0ull;
        bitonic_sort64<true>(r, lane);
        merge_best64(v, r, lane);
      }
    }
    if (lane < k) cand[o * k + lane] = v;  // 0 past the last vector
    const uint32_t vk = entry_key(v);
    if (lane == 0)
      bnd[o] = make_uint2((uint32_t)__builtin_amdgcn_readlane((int)vk, k - 1),
                          (uint32_t)__builtin_amdgcn_readlane((int)vk, 0));
  }
}

// Workgroup j ranks query j's candidates (`blocks` blocks of k) into out_idx / out_score [j][k].
__global__ __launch_bounds__(64 * kFinalWaves) void topk_final_kernel(const uint64_t *__restrict__ cand,
                                                                     const uint2 *__restrict__ bnd, int blocks,
                                                                     int k, int32_t *out_idx, float *out_score) {
  __shared__ int passed[kFinalWaves];
  __shared__ uint64_t stage[kFinalWaves][kFinalRows * 64];  // a wave's passing entries of one batch
  __shared__ uint64_t lists[kFinalWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = blockIdx.x;

  // wave w ranks candidate rows w, w + kFinalWaves, ... (64 entries each); the first rows'
  // loads go out before those of the bound
  const uint64_t *c = cand + (size_t)j * blocks * k;
  const int total = blocks * k;
  uint64_t e[kFinalRows];
  auto load_rows = [&](int r0) {
#pragma unroll
    for (int t = 0; t < kFinalRows; ++t) {
      const int i = (r0 + t * kFinalWaves) * 64 + lane;
      e[t] = i < total ? c[i] : 0ull;
    }
  };
  load_rows(wave);

  // The bound, in every wave alike (no exchange between waves): a key that k scores of the
  // query reach bounds its k-th best from below, and only entries at or above it (and not
  // empty) can be among the k best.  Two such keys: the largest block k-th best, and the k-th
  // largest of the lanes' maxima over block bests (each lane's maximum is the best of a block
  // of its own, so k blocks reach it).
  uint32_t mk = 0u, mb = 0u;
  for (int b0 = 0; b0 < blocks; b0 += 64 * kBoundLoads) {  // lane l takes blocks l, l + 64, ...
    uint2 v[kBoundLoads];
#pragma unroll
    for (int t = 0; t < kBoundLoads; ++t) {
      const int b = b0 + t * 64 + lane;
      v[t] = b < blocks ? bnd[(size_t)j * blocks + b] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int t = 0; t < kBoundLoads; ++t) {
      mk = max(mk, v[t].x);
      mb = max(mb, v[t].y);
    }
  }
  mk = wave_max_u32(mk);
  bitonic_sort64<false>(mb, lane);
  const uint32_t lim = max(max(mk, 1u), (uint32_t)__builtin_amdgcn_readlane((int)mb, k - 1));
  const uint64_t floor = (uint64_t)lim << 32;

  if (total <= kFinalWaves * kFinalRows * 64) {  // every candidate is loaded: count those passing
    int cnt = 0;
#pragma unroll
    for (int t = 0; t < kFinalRows; ++t) cnt += __popcll(__ballot(e[t] >= floor));
    if (lane == 0) passed[wave] = cnt;
    __syncthreads();
    int n_pass = 0, at = 0;
#pragma unroll
    for (int w = 0; w < kFinalWaves; ++w) {
      at += w < wave ? passed[w] : 0;
      n_pass += passed[w];
    }
    if (n_pass <= 64) {  // the usual case: one sort of all of them
      uint64_t *slots = &stage[0][0];
#pragma unroll
      for (int t = 0; t < kFinalRows; ++t) {
        const bool pass = e[t] >= floor;
        const uint64_t bm = __ballot(pass);
        if (pass) slots[at + lanes_below(bm)] = e[t];
        at += __popcll(bm);
      }
      __syncthreads();
      if (wave == 0) {
        uint64_t v = lane < n_pass ? slots[lane] : 0ull;
        bitonic_sort64<false>(v, lane);
        if (lane < k) {
          out_idx[(size_t)j * k + lane] = v == 0ull ? -1 : entry_index(v);
          out_score[(size_t)j * k + lane] = v == 0ull ? -INFINITY : key_value(entry_key(v));
        }
      }
      return;
    }
  }

  // a wave's running best 64, in rank order: each batch's passing entries are compacted into
  // the wave's LDS stage, then ranked 64 at a time (one copy of the sort code, in a loop) and
  // merged in
  uint64_t best = 0ull;
  uint64_t *st = stage[wave];
  for (int r0 = wave; r0 * 64 < total; r0 += kFinalWaves * kFinalRows) {
    if (r0 != wave) load_rows(r0);
    int n_st = 0;
#pragma unroll
    for (int t = 0; t < kFinalRows; ++t) {
      const bool pass = e[t] >= floor;
      const uint64_t bm = __ballot(pass);
      if (pass) st[n_st + lanes_below(bm)] = e[t];
      n_st += __popcll(bm);
    }
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
#pragma unroll 1
    for (int c0 = 0; c0 < n_st; c0 += 64) {
      uint64_t v = c0 + lane < n_st ? st[c0 + lane] : 0ull;
      bitonic_sort64<true>(v, lane);
      merge_best64(best, v, lane);
    }
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
  }

  // merge the waves' lists pairwise: wave w takes wave w + s's list, reversed
  lists[wave][lane] = best;
#pragma unroll 1
  for (int s = 1; s < kFinalWaves; s <<= 1) {
    __syncthreads();
    if ((wave & (2 * s - 1)) == 0) {
      merge_best64(best, lists[wave + s][63 - lane], lane);
      lists[wave][lane] = best;
    }
  }
  if (wave == 0 && lane < k) {
    out_idx[(size_t)j * k + lane] = best == 0ull ? -1 : entry_index(best);
    out_score[(size_t)j * k + lane] = best == 0ull ? -INFINITY : key_value(entry_key(best));
  }
}

}  // namespace

hipError_t launch_ip_search(const CacheView &db, const void *q, int q_dtype, int n_q, int n, int k, int32_t *out_idx,
                            float *out_score, const SearchState &st, hipStream_t stream) {
  const int blocks = (n + kBlockTokens - 1) / kBlockTokens;
  const dim3 grid(blocks, (n_q + 7) / 8);
  if (db.bits == 4)
    ip_score_kernel<4><<<grid, 64 * kScoreWaves, 0, stream>>>(db, q, q_dtype, n_q, n, k, st.cand, st.bnd);
  else
    ip_score_kernel<3><<<grid, 64 * kScoreWaves, 0, stream>>>(db, q, q_dtype, n_q, n, k, st.cand, st.bnd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  topk_final_kernel<<<n_q, 64 * kFinalWaves, 0, stream>>>(st.cand, st.bnd, blocks, k, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace tq
