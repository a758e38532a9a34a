// Generic decode attention over the packed cache (any code width, any GQA group <= 16).
//
// Scoring in the rotated domain ([google] "Google 最新極限壓縮算法…": scores computed
// directly against quantized keys; weighted V sums kept in the rotated domain and rotated
// back once), online softmax per split of the context, an LSE merge of the splits, and the
// exact Sparse-V rule of [inferrs] "inferrs & TurboQuant：本地 LLM 推理的内存革命", §Sparse V
// (rows whose final softmax weight is below tau are not decoded).
//
// Sparse V is exact although the final log-sum-exp is only known at the end: pass 1 keeps a
// row as a candidate unless its score is below (running LSE of the split) + ln tau; the
// running LSE never exceeds the final one, so no row the exact rule keeps is dropped.
// Pass 2 applies the exact rule to the candidates with the merged LSE and reads only the
// V codes of kept rows.
#include "tq_common.h"
#include "tq_launch.h"

namespace tq {
namespace {

constexpr float kInvSqrtD = 0.08838834764831845f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ int seq_len_of(const DecodeArgs &a, int b) {
  if (a.seq_lens == nullptr) return a.ctx_len;
  return min(max(a.seq_lens[b], 0), a.ctx_len);
}

// Rotated, scaled queries of the g heads of one kv head: qt[j] = scale * R q_{kvh*g+j}.
__device__ void load_rotated_queries(const DecodeArgs &a, int b, int kvh, float (*qt)[kD]) {
  const int g = a.group;
  for (int e = threadIdx.x; e < g * kD; e += blockDim.x) {
    const int j = e / kD, i = e % kD;
    const float x = load_elem(a.q, ((size_t)b * a.n_q_heads + kvh * g + j) * kD + i, a.q_dtype);
    qt[j][i] = a.k.signs[i] < 0 ? -x : x;
  }
  block_fwht128(&qt[0][0], g);
  const float qs = a.scale * kInvSqrtD;
  for (int e = threadIdx.x; e < g * kD; e += blockDim.x) qt[e / kD][e % kD] *= qs;
  __syncthreads();
}

__global__ __launch_bounds__(256) void decode_split_generic(DecodeArgs a) {
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int g = a.group, S = a.plan.n_splits;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool sparse = a.sparse != 0;

  __shared__ float qt[16][kD];
  __shared__ float pq[16][kD];  // QJL keys: S qt[j], the sketch of each scaled rotated query
  __shared__ float lutK[256], lutV[256];
  __shared__ float pbuf[16][256];
  __shared__ float nvs[256];
  __shared__ float stat_s[16];
  __shared__ int wave_cnt[4];

  const int T = seq_len_of(a, b);
  const int t_begin = s * a.plan.split_len;
  const int t_end = min(t_begin + a.plan.split_len, T);
  const int bk = a.k.bits, bv = a.v.bits;
  for (int i = tid; i < (1 << bk); i += blockDim.x) lutK[i] = a.k.centroids[i];
  for (int i = tid; i < (1 << bv); i += blockDim.x) lutV[i] = a.v.centroids[i];
  load_rotated_queries(a, b, kvh, qt);
  const bool qjl = a.qjl_m > 0;
  if (qjl) {  // ([google] §第二步：QJL) pq[j][r] = sum_i S[r][i] qt[j][i]
    for (int e = tid; e < g * kD; e += blockDim.x) {
      const int j = e / kD, r = e % kD;
      const float *row = a.qjl_proj + (size_t)r * kD;
      float acc = 0.f;
      for (int i = 0; i < kD; ++i) acc = fmaf(row[i], qt[j][i], acc);
      pq[j][r] = acc;
    }
    __syncthreads();
  }
  // sqrt(pi / 2) / m: the sign sketch's estimate of the residual's inner product is unbiased
  const float qjl_kappa = qjl ? 1.2533141373155003f / (float)a.qjl_m : 0.f;

  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.f; }
  const int ci = tid & (kD - 1), jj = tid >> 7;
  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.f;

  const uint8_t *kplane = a.k.plane(b, kvh);
  const uint16_t *knorm = a.k.norm_plane(b, kvh);
  const uint8_t *vplane = a.v.plane(b, kvh);
  const uint16_t *vnorm = a.v.norm_plane(b, kvh);
  float *cand_base = nullptr;
  if (sparse)
    cand_base = a.cand + (((size_t)b * a.n_kv_heads + kvh) * S + s) * (size_t)a.plan.split_len * (1 + g);
  int cand_written = 0;

  for (int t0 = t_begin; t0 < t_end; t0 += 256) {
    const int t = t0 + tid;
    const bool valid = t < t_end;
    float d[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) d[j] = 0.f;
    if (valid) {
      const uint8_t *row = kplane + (size_t)t * 16 * bk;
      for (int i0 = 0; i0 < kD; i0 += 8) {
        float cv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) cv[e] = lutK[read_field(row, (uint64_t)(i0 + e) * bk, bk)];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j < g) {
#pragma unroll
            for (int e = 0; e < 8; ++e) d[j] = fmaf(qt[j][i0 + e], cv[e], d[j]);
          }
        }
      }
      const float nk = half_bits_to_float(knorm[t]);
#pragma unroll
      for (int j = 0; j < 16; ++j) d[j] *= nk;
      if (qjl) {
        // QJL correction: kappa ||r|| sum_r (S qt[j])_r (2 bit_r - 1), the unbiased estimate of
        // the residual's share of the score ([google] _prod_score_kernel: the score against
        // the codes plus the sign-sketch term)
        const size_t unit = (size_t)b * a.n_kv_heads + kvh;
        const uint4 sb = *reinterpret_cast<const uint4 *>(a.qjl_bits + (unit * a.k.capacity + t) * (kD / 8));
        const uint32_t wv[4] = {sb.x, sb.y, sb.z, sb.w};
        float e[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) e[j] = 0.f;
        for (int r = 0; r < kD; ++r) {
          const bool on = (wv[r >> 5] >> (r & 31)) & 1u;
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (j < g) e[j] += on ? pq[j][r] : -pq[j][r];
        }
        const float rk = qjl_kappa * half_bits_to_float(a.qjl_rnorm[unit * a.k.capacity + t]);
#pragma unroll
        for (int j = 0; j < 16; ++j) d[j] = fmaf(rk, e[j], d[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < g) pbuf[j][tid] = valid ? d[j] : -INFINITY;
    if (a.scores != nullptr && valid) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j < g) a.scores[((size_t)b * a.n_q_heads + kvh * g + j) * a.ctx_len + t] = d[j];
    }
    nvs[tid] = valid ? half_bits_to_float(vnorm[t]) : 0.f;
    __syncthreads();

#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = wave + 4 * r;
      if (j < g) {
        float x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = pbuf[j][lane + 64 * k];
        const float cm = wave_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const float m_new = fmaxf(m_run[r], cm);
        float alpha = 1.f, psum = 0.f;
        if (m_new != -INFINITY) {
          alpha = m_run[r] == -INFINITY ? 0.f : __expf(m_run[r] - m_new);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            x[k] = x[k] == -INFINITY ? 0.f : __expf(x[k] - m_new);
            psum += x[k];
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) x[k] = 0.f;
        }
        psum = wave_sum(psum);
        l_run[r] = l_run[r] * alpha + psum;
        m_run[r] = m_new;
        if (!sparse) {
#pragma unroll
          for (int k = 0; k < 4; ++k) pbuf[j][lane + 64 * k] = x[k];
          if (lane == 0) stat_s[j] = alpha;
        } else if (lane == 0) {
          stat_s[j] = m_new == -INFINITY ? INFINITY : m_new + __logf(l_run[r]);
        }
      }
    }
    __syncthreads();

    if (!sparse) {
      const int nvalid = min(256, t_end - t0);
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (jj + 2 * r < g) acc[r] *= stat_s[jj + 2 * r];
      const uint64_t fmask = (1ull << bv) - 1ull;
      for (int gi = 0; gi < (nvalid + 7) / 8; ++gi) {
        const uint8_t *chunk = vplane + (size_t)((t0 >> 3) + gi) * kD * bv + (size_t)ci * bv;
        uint64_t w = 0;
        for (int by = 0; by < bv; ++by) w |= (uint64_t)chunk[by] << (8 * by);
        for (int rr = 0; rr < 8; ++rr) {
          const int tt = 8 * gi + rr;
          if (tt >= nvalid) break;
          const float val = lutV[(w >> (rr * bv)) & fmask] * nvs[tt];
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (jj + 2 * r < g) acc[r] = fmaf(pbuf[jj + 2 * r][tt], val, acc[r]);
        }
      }
    } else {
      bool flag = false;
      if (valid) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (j < g && pbuf[j][tid] >= stat_s[j] + a.ln_tau) flag = true;
      }
      const uint64_t bal = __ballot(flag);
      const int rank = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wave_cnt[wave] = __popcll(bal);
      __syncthreads();
      int off = cand_written;
      for (int w = 0; w < wave; ++w) off += wave_cnt[w];
      if (flag) {
        float *rec = cand_base + (size_t)(off + rank) * (1 + g);
        rec[0] = __int_as_float(t);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (j < g) rec[1 + j] = pbuf[j][tid];
      }
      cand_written += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    }
    __syncthreads();
  }

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = wave + 4 * r;
    if (j < g && lane == 0)
      a.part_ml[((size_t)b * a.n_q_heads + kvh * g + j) * S + s] = make_float2(m_run[r], l_run[r]);
  }
  if (!sparse) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int j = jj + 2 * r;
      if (j < g) a.part_o[(((size_t)b * a.n_q_heads + kvh * g + j) * S + s) * kD + ci] = acc[r];
    }
  } else if (tid == 0) {
    a.cand_count[((size_t)b * a.n_kv_heads + kvh) * S + s] = cand_written;
  }
}

// Sparse V, second pass, one block per split.  The exact weights p = exp(s - LSE) of the
// candidate rows (zero where p < tau), times the row's value norm, go to an LDS table
// w[split_len][GP] (GP = the group size padded to 4, 8 or 16; padding heads stay 0); then
// the block reads only the split's 8-token value groups that hold a kept row.  A group is
// 128 coordinates of BV contiguous bytes, so one wave reads a whole group with lane l
// taking coordinates 2l and 2l+1 (2*BV bytes, one coalesced access), and adds
// w[t][j] * c_V[code] for every head j; the four waves take every fourth group, a batch of
// groups in flight at a time, and are summed through LDS at the end.
template <int BV>
__device__ __forceinline__ void load_coord_pair(const uint8_t *src, uint64_t &lo, uint64_t &hi) {
  if constexpr (BV == 2) {
    const uint32_t x = *reinterpret_cast<const uint32_t *>(src);
    lo = x & 0xFFFFu;
    hi = x >> 16;
  } else if constexpr (BV == 3) {
    const uint16_t *h = reinterpret_cast<const uint16_t *>(src);
    const uint32_t u0 = h[0], u1 = h[1], u2 = h[2];
    lo = u0 | (uint64_t)(u1 & 0xFFu) << 16;
    hi = (u1 >> 8) | (uint64_t)u2 << 8;
  } else if constexpr (BV == 4) {
    const uint2 x = *reinterpret_cast<const uint2 *>(src);
    lo = x.x;
    hi = x.y;
  } else {
    const uint4 x = *reinterpret_cast<const uint4 *>(src);
    lo = x.x | (uint64_t)x.y << 32;
    hi = x.z | (uint64_t)x.w << 32;
  }
}

template <int GP, int BV>
__global__ __launch_bounds__(256) void decode_sparse_v(DecodeArgs a) {
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int g = a.group, S = a.plan.n_splits, L = a.plan.split_len;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float lse_s[16];
  __shared__ float lutV[1 << BV];
  __shared__ __align__(16) float w[kSparseWeights];  // [token in split][GP]; then [wave][GP][kD]
  __shared__ int gflag[kSparseWeights / 32];         // 8-token groups holding a kept row
  __shared__ uint16_t nvs[kSparseWeights / 4];       // fp16 value norms of the split
  static_assert(4 * GP * kD <= kSparseWeights, "wave sums fit the weight table");

  const int t_begin = s * L;
  {  // the split's value norms go to LDS with the other set-up loads
    const uint16_t *vnorm = a.v.norm_plane(b, kvh) + t_begin;
    const int n_valid = min(L, seq_len_of(a, b) - t_begin);
    for (int i = tid; i < L; i += blockDim.x) nvs[i] = i < n_valid ? vnorm[i] : (uint16_t)0;
  }
  for (int i = tid; i < (1 << BV); i += blockDim.x) lutV[i] = a.v.centroids[i];
  for (int i = tid; i < L * GP; i += blockDim.x) w[i] = 0.f;
  for (int i = tid; i < L / 8; i += blockDim.x) gflag[i] = 0;
  for (int j = wave; j < g; j += 4) {
    const int SL = a.lse_splits;
    const float2 *ml = a.lse_ml + ((size_t)b * a.n_q_heads + kvh * g + j) * SL;
    float mx = -INFINITY;
    for (int k = lane; k < SL; k += 64) mx = fmaxf(mx, ml[k].x);
    mx = wave_max(mx);
    float l = 0.f;
    if (mx != -INFINITY)
      for (int k = lane; k < SL; k += 64)
        if (ml[k].x != -INFINITY) l += ml[k].y * __expf(ml[k].x - mx);
    l = wave_sum(l);
    if (lane == 0) lse_s[j] = mx == -INFINITY ? INFINITY : mx + __logf(l);
  }
  __syncthreads();

  const int count = a.cand_count[((size_t)b * a.n_kv_heads + kvh) * S + s];
  const float *base =
      a.cand + (((size_t)b * a.n_kv_heads + kvh) * S + s) * (size_t)L * (1 + g);
  // two records per thread per round, their loads issued together
  for (int r0 = 0; r0 < count; r0 += 2 * 256) {
    float rec[2][1 + GP];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = r0 + k * 256 + tid;
      const float *src = base + (size_t)min(r, count - 1) * (1 + g);
#pragma unroll
      for (int jj = 0; jj <= GP; ++jj) rec[k][jj] = jj <= g ? src[jj] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (r0 + k * 256 + tid >= count) continue;
      const int tl = __float_as_int(rec[k][0]) - t_begin;
      const float nv = half_bits_to_float(nvs[tl]);
      bool any = false;
#pragma unroll
      for (int j = 0; j < GP; ++j) {
        if (j < g) {
          const float z = rec[k][1 + j] - lse_s[j];
          const bool keep = z >= a.ln_tau;
          w[tl * GP + j] = keep ? __expf(z) * nv : 0.f;
          any |= keep;
        }
      }
      if (any) gflag[tl >> 3] = 1;
    }
  }
  __syncthreads();

  const uint8_t *vgroups = a.v.plane(b, kvh) + (size_t)(t_begin >> 3) * kD * BV + 2 * lane * BV;
  float acc_a[GP], acc_b[GP];
#pragma unroll
  for (int j = 0; j < GP; ++j) acc_a[j] = acc_b[j] = 0.f;
  const int n_groups = L / 8;
  constexpr uint32_t kMask = (1u << BV) - 1u;
  constexpr int kBatch = BV == 8 ? 8 : 16;
  for (int g0 = wave; g0 < n_groups; g0 += 4 * kBatch) {
    uint64_t lo[kBatch], hi[kBatch];
    bool on[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int gi = g0 + 4 * u;
      on[u] = gi < n_groups && gflag[gi];
      lo[u] = hi[u] = 0;
      if (on[u]) load_coord_pair<BV>(vgroups + (size_t)gi * kD * BV, lo[u], hi[u]);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (!on[u]) continue;
      const float4 *wr = reinterpret_cast<const float4 *>(w + (size_t)(8 * (g0 + 4 * u)) * GP);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float va = lutV[(uint32_t)(lo[u] >> (r * BV)) & kMask];
        const float vb = lutV[(uint32_t)(hi[u] >> (r * BV)) & kMask];
#pragma unroll
        for (int q = 0; q < GP / 4; ++q) {
          const float4 ww = wr[r * (GP / 4) + q];
          acc_a[4 * q + 0] = fmaf(ww.x, va, acc_a[4 * q + 0]);
          acc_a[4 * q + 1] = fmaf(ww.y, va, acc_a[4 * q + 1]);
          acc_a[4 * q + 2] = fmaf(ww.z, va, acc_a[4 * q + 2]);
          acc_a[4 * q + 3] = fmaf(ww.w, va, acc_a[4 * q + 3]);
          acc_b[4 * q + 0] = fmaf(ww.x, vb, acc_b[4 * q + 0]);
          acc_b[4 * q + 1] = fmaf(ww.y, vb, acc_b[4 * q + 1]);
          acc_b[4 * q + 2] = fmaf(ww.z, vb, acc_b[4 * q + 2]);
          acc_b[4 * q + 3] = fmaf(ww.w, vb, acc_b[4 * q + 3]);
        }
      }
    }
  }
  __syncthreads();  // weights no longer read: the table now holds the wave sums
  float2 *red = reinterpret_cast<float2 *>(w);
#pragma unroll
  for (int j = 0; j < GP; ++j) red[(wave * GP + j) * (kD / 2) + lane] = make_float2(acc_a[j], acc_b[j]);
  __syncthreads();
  for (int e = tid; e < g * kD; e += blockDim.x) {
    const int j = e / kD, c = e % kD;
    float o = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) o += w[(wv * GP + j) * kD + c];
    a.part_o[(((size_t)b * a.n_q_heads + kvh * g + j) * S + s) * kD + c] = o;
  }
}

template <int GP>
void launch_sparse_v(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
  switch (a.v.bits) {
    case 2: decode_sparse_v<GP, 2><<<grid, 256, 0, stream>>>(a); break;
    case 3: decode_sparse_v<GP, 3><<<grid, 256, 0, stream>>>(a); break;
    case 4: decode_sparse_v<GP, 4><<<grid, 256, 0, stream>>>(a); break;
    default: decode_sparse_v<GP, 8><<<grid, 256, 0, stream>>>(a); break;
  }
}

// LSE merge of the split partials, normalisation and the inverse rotation R^T.
// Block (query head, batch) of 512 threads: 4 groups of 128 (one coordinate per thread)
// take every 4th split, with independent loads unrolled so the latency overlaps.
constexpr int kMergeGroups = 4;

__global__ __launch_bounds__(128 * kMergeGroups) void decode_merge(DecodeArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y;
  const int i = threadIdx.x & (kD - 1), grp = threadIdx.x >> 7;
  const int S = a.plan.n_splits;
  const float2 *ml = a.part_ml + ((size_t)b * a.n_q_heads + hq) * S;
  const float *po = a.part_o + ((size_t)b * a.n_q_heads + hq) * S * kD;
  __shared__ float red_m[kMergeGroups * 2];
  __shared__ float red_l[kMergeGroups];
  __shared__ float red_o[kMergeGroups][kD];
  __shared__ float buf[kD];

  // Sparse V: the LSE comes from the first pass's partials, and the second pass's partials
  // are already normalised, so they are plain sums
  const int SL = a.sparse ? a.lse_splits : S;
  const float2 *lml = a.sparse ? a.lse_ml + ((size_t)b * a.n_q_heads + hq) * SL : ml;
  float mx = -INFINITY;
  for (int k = threadIdx.x; k < SL; k += blockDim.x) mx = fmaxf(mx, lml[k].x);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
  if ((threadIdx.x & 63) == 0) red_m[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = red_m[0];
#pragma unroll
  for (int w = 1; w < kMergeGroups * 2; ++w) mx = fmaxf(mx, red_m[w]);

  float o = 0.f, l = 0.f;
  if (mx != -INFINITY && !a.sparse) {
    int k = grp;
    for (; k + 3 * kMergeGroups < S; k += 4 * kMergeGroups) {
      float2 p[4];
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        p[u] = ml[k + u * kMergeGroups];
        v[u] = po[(size_t)(k + u * kMergeGroups) * kD + i];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = p[u].x == -INFINITY ? 0.f : __expf(p[u].x - mx);
        l += p[u].y * w;
        o += v[u] * w;
      }
    }
    for (; k < S; k += kMergeGroups) {
      const float2 p = ml[k];
      const float w = p.x == -INFINITY ? 0.f : __expf(p.x - mx);
      l += p.y * w;
      o += po[(size_t)k * kD + i] * w;
    }
  } else if (mx != -INFINITY) {
    for (int k = grp; k < SL; k += kMergeGroups) {
      const float2 p = lml[k];
      if (p.x != -INFINITY) l += p.y * __expf(p.x - mx);
    }
    int k = grp;
    for (; k + 15 * kMergeGroups < S; k += 16 * kMergeGroups) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = po[(size_t)(k + u * kMergeGroups) * kD + i];
#pragma unroll
      for (int u = 0; u < 16; ++u) o += v[u];
    }
    for (; k < S; k += kMergeGroups) o += po[(size_t)k * kD + i];
  }
  red_o[grp][i] = o;
  if (i == 0) red_l[grp] = l;
  __syncthreads();
  if (grp == 0) {
    float ot = red_o[0][i], lt = red_l[0];
#pragma unroll
    for (int q = 1; q < kMergeGroups; ++q) {
      ot += red_o[q][i];
      lt += red_l[q];
    }
    if (mx != -INFINITY && !a.sparse) ot /= lt;
    if (mx == -INFINITY) ot = 0.f;
    buf[i] = ot;
    if (i == 0 && a.lse != nullptr)
      a.lse[(size_t)b * a.n_q_heads + hq] = mx == -INFINITY ? -INFINITY : mx + __logf(lt);
  }
  if (a.scores != nullptr) {  // positions past the sequence length read -inf
    const int T = seq_len_of(a, b);
    float *row = a.scores + ((size_t)b * a.n_q_heads + hq) * a.ctx_len;
    for (int t = T + (int)threadIdx.x; t < a.ctx_len; t += blockDim.x) row[t] = -INFINITY;
  }
  block_fwht128(buf, 1);
  if (grp == 0) {
    const float r = buf[i] * kInvSqrtD;
    a.out[((size_t)b * a.n_q_heads + hq) * kD + i] = a.k.signs[i] < 0 ? -r : r;
  }
}

}  // namespace

int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// After a split pass: the Sparse-V second pass (if a.sparse), then the LSE merge of the splits.
static hipError_t finish_split_decode(const DecodeArgs &a, dim3 grid_split, hipStream_t stream) {
  if (a.sparse) {
    if (a.group <= 4) launch_sparse_v<4>(a, grid_split, stream);
    else if (a.group <= 8) launch_sparse_v<8>(a, grid_split, stream);
    else launch_sparse_v<16>(a, grid_split, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  decode_merge<<<dim3(a.n_q_heads, a.batch), 128 * kMergeGroups, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_sparse_two_pass(const DecodeArgs &a, hipStream_t stream) {
  // Sparse V on matrix cores, two launches: the key pass (no candidate records) for each
  // row's LSE, then the dense kernel with the rows under the final-weight threshold masked
  // out of the value product; it merges its splits itself.  (Values of 2 bits.)  With a.xk
  // set, the key pass first writes the decode step's new key and value.
  DecodeArgs v2 = a;
  v2.sparse = 0;
  v2.xk = v2.xv = nullptr;
  v2.lse_ml = a.fpart_ml;
  v2.lse_splits = a.fplan.n_splits;
  v2.fplan = plan_fused_vmask(a.batch, a.n_kv_heads, a.ctx_len);  // at most 64 tiles per split
  v2.fpart_ml = a.vpart_ml;
  v2.fpart_o = a.vpart_o;
  if (!(a.sparse && decode_fused_sparse_supported(a) && a.vpart_ml != nullptr && a.tile_max != nullptr &&
        decode_fused_supported(v2)))
    return hipErrorNotSupported;
  DecodeArgs k1 = a;
  k1.cand = nullptr;
  k1.cand_count = nullptr;
  const hipError_t e = launch_decode_fused_sparse(k1, stream);
  if (e != hipSuccess) return e;
  return launch_decode_fused_vmask(v2, stream);
}

hipError_t launch_decode(const DecodeArgs &args, hipStream_t stream) {
  if (decode_fused_supported(args)) return launch_decode_fused(args, compute_units(), stream);
  DecodeArgs a = args;
  dim3 grid_split(a.plan.n_splits, a.n_kv_heads, a.batch);
  hipError_t e;
  if (a.sparse) {
    e = launch_sparse_two_pass(a, stream);
    if (e != hipErrorNotSupported) return e;
  }
  if (decode_fused_sparse_supported(a)) {  // key-only fused first pass
    a.lse_ml = a.fpart_ml;
    a.lse_splits = a.fplan.n_splits;
    e = launch_decode_fused_sparse(a, stream);
  } else {
    a.lse_ml = a.part_ml;
    a.lse_splits = a.plan.n_splits;
    if (decode_mfma_supported(a)) {
      e = launch_decode_mfma(a, compute_units(), stream);
    } else {
      return launch_decode_generic(a, stream);
    }
  }
  if (e != hipSuccess) return e;
  return finish_split_decode(a, grid_split, stream);
}

hipError_t launch_decode_generic(const DecodeArgs &args, hipStream_t stream) {
  DecodeArgs a = args;
  a.lse_ml = a.part_ml;
  a.lse_splits = a.plan.n_splits;
  const dim3 grid_split(a.plan.n_splits, a.n_kv_heads, a.batch);
  decode_split_generic<<<grid_split, 256, 0, stream>>>(a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return finish_split_decode(a, grid_split, stream);
}

}  // namespace tq
