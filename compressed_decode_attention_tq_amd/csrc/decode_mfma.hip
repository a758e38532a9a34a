// Decode attention on matrix cores (gfx950 v_mfma_f32_16x16x32_f16) for the common code
// widths: keys 3 or 4 bits (TQ_LAYOUT_ROWS), values 2 bits (TQ_LAYOUT_GROUP8), query group
// up to 8 heads per kv head.
//
// What is computed is the same as the generic kernels ([google] "Google 最新極限壓縮算法…":
// scores taken directly against the quantized keys, values summed in the rotated domain);
// only the schedule differs:
//   * Codes become fp16 operands through lookup tables in LDS.  A key byte (two 4-bit codes,
//     or a 6-bit pair of 3-bit codes) gives {hi(c_a), hi(c_b), lo(c_a), lo(c_b)}, the two
//     centroids split into an fp16 hi part and the fp16 remainder; a value byte (four 2-bit
//     codes of one coordinate, four consecutive tokens) gives four fp16 centroids.  Tables
//     are replicated 32 times so the 32 lanes of one LDS pass never share a bank; one
//     v_perm builds a lookup address; two lookups form one 8-half operand as loaded.
//   * Scores, about 22 significant bits: the query rows of the score product hold the
//     rotated query's fp16 hi part (rows 0..G-1) and its remainder (rows G..2G-1), each
//     repeated to match the {hi, hi, lo, lo} key operand, so one product gives
//     (q_hi + q_lo) . (c_hi + c_lo) for 16 coordinates; the two row halves are summed when
//     the scores are compacted through LDS to one token per lane.
//   * Values: O[row][coord] += P'[row][token] V[token][coord] with P' = p * ||v|| split the
//     same way into rows 0..G-1 (fp16 hi) and G..2G-1 (remainder); the GROUP8 layout gives
//     each lane 8 consecutive tokens of 8 coordinates in 16 bytes.
//   * Online softmax with a stale reference: p = exp(s - m_ref); m_ref only moves when a
//     tile would push p * ||v|| past the fp16 range, so the accumulator is rarely rescaled.
//   * Persistent workgroups, one per CU (160 KB of LDS), 8 waves each; a wave owns whole
//     (batch, kv head, split) items and writes (m_ref, l, O) partials that the merge kernel
//     combines, or Sparse-V candidate rows for the second pass.
#include "tq_common.h"
#include "tq_launch.h"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 64;
constexpr float kInvSqrtD = 0.08838834764831845f;
constexpr float kAMax = 30000.f;  // largest p * ||v|| kept in an fp16 operand

// LDS map (bytes):
//   [0, 64K)      K table: entry e at e*256 + copy*8 (copy < 32)
//   [64K, 128K)   V table: entry e at 64K + e*256 + copy*8 (copy < 32)
//   [128K, 160K)  per-wave 4 KB buffer: scores [64 tokens][16 rows] fp32, then P'
//                 [16 rows][64 tokens] fp16; both with XOR-swizzled 16-byte units so the
//                 16 lanes of one LDS pass hit 16 different bank groups
constexpr int kLdsBytes = 160 * 1024;
constexpr uint32_t kVBase = 64 * 1024;
constexpr uint32_t kWBase = 128 * 1024;

__device__ __forceinline__ uint2 lds_u64(const uint8_t *lds, uint32_t addr) {
  return *reinterpret_cast<const uint2 *>(lds + addr);
}
__device__ __forceinline__ uint16_t h16(float x) { return __half_as_ushort(__float2half_rn(x)); }
__device__ __forceinline__ float f16(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// byte offset of score (token, 4-row group) inside the wave buffer
__device__ __forceinline__ uint32_t score_off(int tok, int grp) {
  return (uint32_t)tok * 64u + ((uint32_t)(grp ^ ((tok >> 2) & 3)) << 4);
}
// byte offset of the 16-byte unit (row, unit = tokens 8u .. 8u+7) of the P' staging
__device__ __forceinline__ uint32_t pst_off(int row, int unit) {
  return (uint32_t)row * 128u + ((uint32_t)(unit ^ ((row >> 1) & 7)) << 4);
}

template <int BK>
__device__ void build_tables(uint8_t *lds, const float *kc, const float *vc) {
  for (int idx = threadIdx.x; idx < 256 * 32; idx += blockDim.x) {
    const int e = idx >> 5, copy = idx & 31;
    const float c0 = BK == 4 ? kc[e & 15] : kc[e & 7];
    const float c1 = BK == 4 ? kc[e >> 4] : kc[(e >> 3) & 7];
    const uint16_t h0 = h16(c0), h1 = h16(c1);
    uint2 kv;
    kv.x = (uint32_t)h0 | ((uint32_t)h1 << 16);
    kv.y = (uint32_t)h16(c0 - f16(h0)) | ((uint32_t)h16(c1 - f16(h1)) << 16);
    *reinterpret_cast<uint2 *>(lds + e * 256 + copy * 8) = kv;
    uint2 vv;
    vv.x = (uint32_t)h16(vc[e & 3]) | ((uint32_t)h16(vc[(e >> 2) & 3]) << 16);
    vv.y = (uint32_t)h16(vc[(e >> 4) & 3]) | ((uint32_t)h16(vc[(e >> 6) & 3]) << 16);
    *reinterpret_cast<uint2 *>(lds + kVBase + e * 256 + copy * 8) = vv;
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// NH = query heads per kv head padded to 4 or 8; BK = key bits (3 or 4); value bits 2.
template <int BK, int NH, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(NH == 4 || NH == 8, "two row halves of NH rows must fit 16 rows");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  build_tables<BK>(lds, a.k.centroids, a.v.centroids);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = a.group, S = a.plan.n_splits;
  const int m_row = lane & 15, quarter = lane >> 4;
  const uint32_t kc8 = (uint32_t)(lane & 31) << 3;
  const uint32_t vc8 = ((uint32_t)(lane & 31) << 3) | 0x00010000u;  // + 64K table base
  uint8_t *wbuf = lds + kWBase + wave * 4096;
  // query row this lane feeds: hi part of head m_row, remainder of head m_row - NH, or 0
  const int q_head = m_row < NH ? m_row : m_row - NH;
  const bool q_is_lo = m_row >= NH;
  const bool q_live = m_row < 2 * NH && q_head < g;

  const int n_items = a.batch * a.n_kv_heads * S;
  const int wave_id = blockIdx.x * kWaves + wave, n_waves = gridDim.x * kWaves;

  for (int item = wave_id; item < n_items; item += n_waves) {
    const int split = item % S;
    const int kvh = (item / S) % a.n_kv_heads;
    const int b = item / (S * a.n_kv_heads);
    int T = a.ctx_len;
    if (a.seq_lens != nullptr) T = min(max(a.seq_lens[b], 0), a.ctx_len);
    const int t_begin = split * a.plan.split_len;
    const int t_end = min(t_begin + a.plan.split_len, T);

    // ---- rotated, scaled query (hi or lo part), each value repeated for {hi, hi, lo, lo}
    half8 qop[8];
    {
      float v[32];
      const size_t qbase = ((size_t)b * a.n_q_heads + kvh * g + (q_live ? q_head : 0)) * kD + 32 * quarter;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float x = q_live ? load_elem(a.q, qbase + e, a.q_dtype) : 0.f;
        v[e] = a.k.signs[32 * quarter + e] < 0 ? -x : x;
      }
#pragma unroll
      for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e)
          if ((e & h) == 0) {
            const float x0 = v[e], x1 = v[e + h];
            v[e] = x0 + x1;
            v[e + h] = x0 - x1;
          }
      }
#pragma unroll
      for (int m = 16; m <= 32; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const float o = __shfl_xor(v[e], m);
          v[e] = upper ? (o - v[e]) : (v[e] + o);
        }
      }
      const float qs = a.scale * kInvSqrtD;
      _Float16 part[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float x = v[e] * qs;
        const _Float16 hi = (_Float16)x;
        part[e] = q_is_lo ? (_Float16)(x - (float)hi) : hi;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        qop[m][0] = part[4 * m];     qop[m][1] = part[4 * m + 1];
        qop[m][2] = part[4 * m];     qop[m][3] = part[4 * m + 1];
        qop[m][4] = part[4 * m + 2]; qop[m][5] = part[4 * m + 3];
        qop[m][6] = part[4 * m + 2]; qop[m][7] = part[4 * m + 3];
      }
    }

    float m_ref[NH], l_part[NH];
#pragma unroll
    for (int j = 0; j < NH; ++j) { m_ref[j] = -INFINITY; l_part[j] = 0.f; }
    floatx4 oacc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) oacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};

    const uint8_t *kplane = a.k.plane(b, kvh);
    const uint16_t *knorm = a.k.norm_plane(b, kvh);
    const uint8_t *vplane = a.v.plane(b, kvh);
    const uint16_t *vnorm = a.v.norm_plane(b, kvh);
    float *cand_base = nullptr;
    int cand_written = 0;
    if (SPARSE) cand_base = a.cand + ((size_t)item) * (size_t)a.plan.split_len * (1 + g);

    // ---- tile loads: key quarter rows (token 16s + m_row, coordinates 32q..32q+31) and
    //      key norms are fetched one tile ahead (issued as soon as the score products of
    //      the previous tile have consumed them); value groups and value norms at the top of
    //      the tile they belong to, ahead of the score products
    uint32_t kw[4][4];
    uint16_t nk_h = 0;
    auto load_keys = [&](int t0) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint8_t *src = kplane + (size_t)(t0 + 16 * s + m_row) * (16 * BK) + quarter * (4 * BK);
        if (BK == 4) {
          const uint4 w = *reinterpret_cast<const uint4 *>(src);
          kw[s][0] = w.x; kw[s][1] = w.y; kw[s][2] = w.z; kw[s][3] = w.w;
        } else {
          const uint32_t *pp = reinterpret_cast<const uint32_t *>(src);
          kw[s][0] = pp[0]; kw[s][1] = pp[1]; kw[s][2] = pp[2]; kw[s][3] = 0u;
        }
      }
      nk_h = knorm[t0 + lane];
    };
    if (t_begin < t_end) load_keys(t_begin);
    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
      uint4 vw[2];
      uint16_t nv_h = 0;
      if (!SPARSE) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const size_t grp8 = (size_t)(t0 >> 3) + 4 * c + quarter;
          vw[c] = *reinterpret_cast<const uint4 *>(vplane + grp8 * (kD * 2) + m_row * 16);
        }
        nv_h = vnorm[t0 + lane];
      }
      const bool tv = t0 + lane < t_end;

      // ---- scores: sub-tile s, 16-coordinate chunk m -> key fields 2m, 2m+1 of the quarter
      auto key_operands = [&](int m, half8 (&dst)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uint2 t2[2];
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int f = 2 * m + p;  // field index within the quarter row
            uint32_t addr;
            if (BK == 4) {
              addr = __builtin_amdgcn_perm(kw[s][f >> 2], kc8, 0x0C0C0000u | ((4u + (f & 3)) << 8));
            } else {
              const int bit = 6 * f;
              uint32_t fld;
              if ((bit & 31) <= 26) fld = (kw[s][bit >> 5] >> (bit & 31)) & 63u;
              else fld = ((kw[s][bit >> 5] >> (bit & 31)) | (kw[s][(bit >> 5) + 1] << (32 - (bit & 31)))) & 63u;
              addr = (fld << 8) | kc8;
            }
            t2[p] = lds_u64(lds, addr);
          }
          __builtin_memcpy(&dst[s], t2, 16);
        }
      };
      floatx4 acc[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[s] = floatx4{0.f, 0.f, 0.f, 0.f};
      half8 bop[2][4];
      key_operands(0, bop[0]);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        // lookups of step m+1 go out before the products of step m, so their LDS latency
        // hides behind four matrix instructions; the fence keeps the scheduler to this order
        if (m + 1 < 8) key_operands(m + 1, bop[(m + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qop[m], bop[m & 1][s], acc[s], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      const float nk = half_bits_to_float(nk_h);
      if (t0 + kTile < t_end) load_keys(t0 + kTile);
      const float nv = SPARSE ? 1.f : half_bits_to_float(nv_h);
      // lane holds rows 4q..4q+3 of token 16s + m_row
#pragma unroll
      for (int s = 0; s < 4; ++s)
        *reinterpret_cast<floatx4 *>(wbuf + score_off(16 * s + m_row, quarter)) = acc[s];
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");
      float sc[NH];
#pragma unroll
      for (int k = 0; k < NH / 4; ++k) {
        const floatx4 hi = *reinterpret_cast<const floatx4 *>(wbuf + score_off(lane, k));
        const floatx4 lo = *reinterpret_cast<const floatx4 *>(wbuf + score_off(lane, k + NH / 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[4 * k + j] = hi[j] + lo[j];
      }
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");

      // ---- online softmax with a stale reference (lane = token t0 + lane, all heads)
      float p[NH];
      bool need = false;
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const bool ok = tv && j < g;
        const float s = ok ? sc[j] * nk : -INFINITY;
        sc[j] = s;
        const float pe = ok ? __expf(s - m_ref[j]) : 0.f;
        p[j] = pe;
        if (ok && !(pe * nv <= kAMax)) need = true;
      }
      if (a.scores != nullptr) {
#pragma unroll
        for (int j = 0; j < NH; ++j)
          if (j < g && tv) a.scores[((size_t)b * a.n_q_heads + kvh * g + j) * a.ctx_len + t0 + lane] = sc[j];
      }
      if (__any(need)) {
        // move the reference to the tile's largest s + ln||v|| (per head), rescale
        float alpha[NH];
        const float lnv = __logf(fmaxf(nv, 1e-30f));
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const float z = wave_max(sc[j] == -INFINITY ? -INFINITY : sc[j] + lnv);
          const float m_new = fmaxf(m_ref[j], z);
          alpha[j] = (m_new == m_ref[j]) ? 1.f : (m_ref[j] == -INFINITY ? 0.f : __expf(m_ref[j] - m_new));
          m_ref[j] = m_new;
          l_part[j] *= alpha[j];
          p[j] = sc[j] == -INFINITY ? 0.f : __expf(sc[j] - m_new);
        }
        if (!SPARSE) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float al = (NH == 8 && (quarter & 1)) ? alpha[(4 + jj) % NH] : alpha[jj];
#pragma unroll
            for (int n = 0; n < 8; ++n) oacc[n][jj] *= al;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NH; ++j) l_part[j] += p[j];

      if (!SPARSE) {
        // ---- P' (hi rows 0..NH-1, remainder rows NH..2NH-1) to LDS, read back as operand
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const float pv = p[j] * nv;
          const _Float16 hi = (_Float16)pv;
          const _Float16 lo = (_Float16)(pv - (float)hi);
          *reinterpret_cast<_Float16 *>(wbuf + pst_off(j, lane >> 3) + 2 * (lane & 7)) = hi;
          *reinterpret_cast<_Float16 *>(wbuf + pst_off(NH + j, lane >> 3) + 2 * (lane & 7)) = lo;
        }
        __builtin_amdgcn_wave_barrier();
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          uint4 pa = *reinterpret_cast<const uint4 *>(wbuf + pst_off(m_row, 4 * c + quarter));
          if (m_row >= 2 * NH) pa = make_uint4(0u, 0u, 0u, 0u);
          half8 aop;
          __builtin_memcpy(&aop, &pa, 16);
          const uint32_t vwd[4] = {vw[c].x, vw[c].y, vw[c].z, vw[c].w};
          auto value_operand = [&](int n) {
            const uint32_t w = vwd[n >> 1];
            const uint32_t sel_lo = 0x0C020000u | ((4u + 2u * (n & 1)) << 8);
            const uint32_t sel_hi = 0x0C020000u | ((5u + 2u * (n & 1)) << 8);
            uint2 t2[2];
            t2[0] = lds_u64(lds, __builtin_amdgcn_perm(w, vc8, sel_lo));
            t2[1] = lds_u64(lds, __builtin_amdgcn_perm(w, vc8, sel_hi));
            half8 bo;
            __builtin_memcpy(&bo, t2, 16);
            return bo;
          };
          half8 vb[2];
          vb[0] = value_operand(0);
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            if (n + 1 < 8) vb[(n + 1) & 1] = value_operand(n + 1);
            __builtin_amdgcn_sched_barrier(0);
            oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, vb[n & 1], oacc[n], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_wave_barrier();
        __asm__ volatile("" ::: "memory");
      } else {
        // ---- Sparse V pass 1: candidate rows, kept unless s < running LSE + ln tau
        bool flag = false;
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const float lt = wave_sum(l_part[j]);
          const float lse_run = m_ref[j] == -INFINITY ? INFINITY : m_ref[j] + __logf(lt);
          if (sc[j] >= lse_run + a.ln_tau) flag = true;
        }
        const uint64_t bal = __ballot(flag);
        const int rank = __popcll(bal & ((1ull << lane) - 1ull));
        if (flag) {
          float *rec = cand_base + (size_t)(cand_written + rank) * (1 + g);
          rec[0] = __int_as_float(t0 + lane);
#pragma unroll
          for (int j = 0; j < NH; ++j)
            if (j < g) rec[1 + j] = sc[j];
        }
        cand_written += __popcll(bal);
      }
    }

    // ---- partials of this item
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const float lt = wave_sum(l_part[j]);
      if (lane == 0 && j < g)
        a.part_ml[((size_t)b * a.n_q_heads + kvh * g + j) * S + split] = make_float2(m_ref[j], lt);
    }
    if (!SPARSE) {
      // add the remainder rows onto the hi rows: rows NH.. live 16*NH/4 lanes further on
      constexpr int kLoLanes = NH == 4 ? 16 : 32;
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) oacc[n][jj] += __shfl_xor(oacc[n][jj], kLoLanes);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int head = 4 * quarter + jj;
        if (head < g && quarter < NH / 4) {
          float *dst = a.part_o + (((size_t)b * a.n_q_heads + kvh * g + head) * S + split) * kD + 8 * m_row;
          *reinterpret_cast<float4 *>(dst) = make_float4(oacc[0][jj], oacc[1][jj], oacc[2][jj], oacc[3][jj]);
          *reinterpret_cast<float4 *>(dst + 4) = make_float4(oacc[4][jj], oacc[5][jj], oacc[6][jj], oacc[7][jj]);
        }
      }
    } else if (lane == 0) {
      a.cand_count[item] = cand_written;
    }
  }
}

template <int BK, bool SPARSE>
hipError_t launch_g(const DecodeArgs &a, int grid, hipStream_t stream) {
  if (a.group <= 4) decode_mfma_kernel<BK, 4, SPARSE><<<grid, kThreads, 0, stream>>>(a);
  else decode_mfma_kernel<BK, 8, SPARSE><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs &a) {
  return (a.k.bits == 3 || a.k.bits == 4) && a.v.bits == 2 && a.group <= 8 &&
         a.k.layout == TQ_LAYOUT_ROWS && a.v.layout == TQ_LAYOUT_GROUP8 &&
         a.plan.split_len % kTile == 0;
}

hipError_t launch_decode_mfma(const DecodeArgs &a, int n_cu, hipStream_t stream) {
  const long items = (long)a.batch * a.n_kv_heads * a.plan.n_splits;
  int grid = (int)std::min<long>(n_cu, (items + kWaves - 1) / kWaves);
  if (grid < 1) grid = 1;
  if (a.k.bits == 4) return a.sparse ? launch_g<4, true>(a, grid, stream) : launch_g<4, false>(a, grid, stream);
  return a.sparse ? launch_g<3, true>(a, grid, stream) : launch_g<3, false>(a, grid, stream);
}

}  // namespace tq
