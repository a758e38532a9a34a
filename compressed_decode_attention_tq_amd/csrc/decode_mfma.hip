// Decode attention on matrix cores (gfx950 v_mfma_f32_16x16x32_f16) for the common code
// widths: keys 3 or 4 bits (TQ_LAYOUT_ROWS), values 2 bits (TQ_LAYOUT_GROUP8).
//
// What is computed is the same as the generic kernels ([google] "Google 最新極限壓縮算法…":
// scores taken directly against the quantized keys, values summed in the rotated domain);
// only the schedule differs:
//   * Codes become fp16 operands through lookup tables in LDS.  A key byte (two 4-bit codes,
//     or a 6-bit pair of 3-bit codes) gives the two centroids as fp16 hi parts plus fp16 lo
//     parts; a value byte (four 2-bit codes of one coordinate, four
//     consecutive tokens) gives four fp16 centroids.  Tables are replicated 32 times so the
//     32 lanes of one LDS pass never share a bank; one v_perm builds a lookup address.
//   * Scores: S[head][token] = Qrot . K per 16-token sub-tile with the rotated query and the
//     centroids each split into fp16 hi + lo parts: hi*hi + lo*hi + hi*lo, three matrix-core
//     products into one fp32 accumulator, about 22 significant bits, which keeps large-norm
//     scores accurate enough for the exponentials (the lo parts are often fp16 subnormals,
//     which the matrix cores take as they are).  Scores are then compacted through LDS to
//     one token per lane.
//   * Values: O[head][coord] += P'[head][token] V[token][coord] with P' = p * ||v|| in fp16;
//     the GROUP8 layout gives each lane 8 consecutive tokens of 8 coordinates in 16 bytes.
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
constexpr float kAMax = 30000.f;        // largest p * ||v|| kept in an fp16 operand

// LDS map (bytes):
//   [0, 64K)      K table: entry e at e*256 + copy*8 (copy < 32): {hi pair, lo pair}
//   [64K, 128K)   V table: entry e at 64K + e*256 + copy*8 (copy < 32): 4 fp16
//   [128K, 160K)  per-wave 4 KB buffer: scores [64 tokens][16 heads] fp32, then P'
//                 [16 heads][64 tokens] fp16 (rows of 128 bytes)
constexpr int kLdsBytes = 160 * 1024;
constexpr uint32_t kVBase = 64 * 1024;
constexpr uint32_t kWBase = 128 * 1024;

__device__ __forceinline__ uint2 lds_u64(const uint8_t *lds, uint32_t addr) {
  return *reinterpret_cast<const uint2 *>(lds + addr);
}

__device__ __forceinline__ uint16_t h16(float x) { return __half_as_ushort(__float2half_rn(x)); }
__device__ __forceinline__ float f16(uint16_t h) { return __half2float(__ushort_as_half(h)); }

template <int BK>
__device__ void build_tables(uint8_t *lds, const float *kc, const float *vc) {
  for (int idx = threadIdx.x; idx < 256 * 32; idx += blockDim.x) {
    const int e = idx >> 5, copy = idx & 31;
    const float c0 = BK == 4 ? kc[e & 15] : kc[e & 7];
    const float c1 = BK == 4 ? kc[e >> 4] : kc[(e >> 3) & 7];
    const uint16_t h0 = h16(c0), h1 = h16(c1);
    const uint16_t l0 = h16(c0 - f16(h0)), l1 = h16(c1 - f16(h1));
    uint2 kv;
    kv.x = (uint32_t)h0 | ((uint32_t)h1 << 16);
    kv.y = (uint32_t)l0 | ((uint32_t)l1 << 16);
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

// NH = query heads handled per lane (group padded to 4, 8 or 16); BK = key bits (3 or 4);
// value bits are 2.
template <int BK, int NH, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  build_tables<BK>(lds, a.k.centroids, a.v.centroids);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = a.group, S = a.plan.n_splits;
  const int m_row = lane & 15, quarter = lane >> 4;
  const uint32_t kc8 = (uint32_t)(lane & 31) << 3;
  const uint32_t vc8 = ((uint32_t)(lane & 31) << 3) | 0x00010000u;  // + 64K table base
  uint8_t *wbuf = lds + kWBase + wave * 4096;
  float *sbuf = reinterpret_cast<float *>(wbuf);                     // [64][16] fp32

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

    // ---- rotated, scaled query of head m_row (rows >= g are zero), split hi + lo
    half8 qhi[4], qlo[4];
    {
      float v[32];
      const bool hv = m_row < g;
      const size_t qbase = ((size_t)b * a.n_q_heads + kvh * g + (hv ? m_row : 0)) * kD + 32 * quarter;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float x = hv ? load_elem(a.q, qbase + e, a.q_dtype) : 0.f;
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
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = v[8 * r + e] * qs;
          const _Float16 hi = (_Float16)x;
          qhi[r][e] = hi;
          qlo[r][e] = (_Float16)(x - (float)hi);
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

    // ---- loads of one tile: key quarter rows (token 16s + m_row, coordinates
    //      32q..32q+31), value groups, norms of token `lane`
    uint32_t kw[4][4], kw_n[4][4];
    uint4 vw[2], vw_n[2];
    uint16_t nk_h = 0, nv_h = 0, nk_n = 0, nv_n = 0;
    auto load_tile = [&](int tl, uint32_t (&kd)[4][4], uint4 (&vd)[2], uint16_t &nkh, uint16_t &nvh) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint8_t *src = kplane + (size_t)(tl + 16 * s + m_row) * (16 * BK) + quarter * (4 * BK);
        if (BK == 4) {
          const uint4 w = *reinterpret_cast<const uint4 *>(src);
          kd[s][0] = w.x; kd[s][1] = w.y; kd[s][2] = w.z; kd[s][3] = w.w;
        } else {
          const uint32_t *pp = reinterpret_cast<const uint32_t *>(src);
          kd[s][0] = pp[0]; kd[s][1] = pp[1]; kd[s][2] = pp[2]; kd[s][3] = 0u;
        }
      }
      if (!SPARSE) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const size_t grp8 = (size_t)(tl >> 3) + 4 * c + quarter;
          vd[c] = *reinterpret_cast<const uint4 *>(vplane + grp8 * (kD * 2) + m_row * 16);
        }
        nvh = vnorm[tl + lane];
      }
      nkh = knorm[tl + lane];
    };
    if (t_begin < t_end) load_tile(t_begin, kw, vw, nk_h, nv_h);

    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
      if (t0 + kTile < t_end) load_tile(t0 + kTile, kw_n, vw_n, nk_n, nv_n);
      if (BK == 3) {  // four 24-bit chunks of 8 codes each
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t p0 = kw[s][0], p1 = kw[s][1], p2 = kw[s][2];
          kw[s][0] = p0 & 0xFFFFFFu;
          kw[s][1] = ((p0 >> 24) | (p1 << 8)) & 0xFFFFFFu;
          kw[s][2] = ((p1 >> 16) | (p2 << 16)) & 0xFFFFFFu;
          kw[s][3] = p2 >> 8;
        }
      }
      const bool tv = t0 + lane < t_end;
      const float nk = half_bits_to_float(nk_h);
      const float nv = SPARSE ? 1.f : half_bits_to_float(nv_h);

      // ---- scores on matrix cores: four 16-token sub-tiles as independent accumulator
      //      chains; per 32-coordinate chunk r, all lookups first, then hi*hi, lo*hi, hi*lo
      floatx4 acc[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[s] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        half8 bh[4], bl[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uint2 t4[4];
          const uint32_t w = kw[s][r];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            uint32_t addr;
            if (BK == 4) addr = __builtin_amdgcn_perm(w, kc8, 0x0C0C0000u | ((4u + p) << 8));
            else addr = (((w >> (6 * p)) & 63u) << 8) | kc8;
            t4[p] = lds_u64(lds, addr);
          }
          const uint32_t hv[4] = {t4[0].x, t4[1].x, t4[2].x, t4[3].x};
          const uint32_t lv[4] = {t4[0].y, t4[1].y, t4[2].y, t4[3].y};
          __builtin_memcpy(&bh[s], hv, 16);
          __builtin_memcpy(&bl[s], lv, 16);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qhi[r], bh[s], acc[s], 0, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qlo[r], bh[s], acc[s], 0, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qhi[r], bl[s], acc[s], 0, 0, 0);
      }
      // lane holds heads 4q..4q+3 of token 16s + m_row (rows >= NH are unused padding)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        *reinterpret_cast<floatx4 *>(sbuf + (16 * s + m_row) * 16 + 4 * quarter) = acc[s];
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");
      float sc[NH];
#pragma unroll
      for (int k = 0; k < NH / 4; ++k) {
        const float4 d = *reinterpret_cast<const float4 *>(sbuf + lane * 16 + 4 * k);
        sc[4 * k] = d.x; sc[4 * k + 1] = d.y; sc[4 * k + 2] = d.z; sc[4 * k + 3] = d.w;
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
        if (a.scores != nullptr && ok)
          a.scores[((size_t)b * a.n_q_heads + kvh * g + j) * a.ctx_len + t0 + lane] = s;
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
            float al = alpha[jj];
            if (NH > 4 && quarter == 1) al = alpha[(4 + jj) % NH];
            if (NH > 8 && quarter == 2) al = alpha[(8 + jj) % NH];
            if (NH > 8 && quarter == 3) al = alpha[(12 + jj) % NH];
#pragma unroll
            for (int n = 0; n < 8; ++n) oacc[n][jj] *= al;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NH; ++j) l_part[j] += p[j];

      if (!SPARSE) {
        // ---- P' to LDS as [head][token] fp16, read back as the PV operand
        _Float16 *pst = reinterpret_cast<_Float16 *>(wbuf);
#pragma unroll
        for (int j = 0; j < NH; ++j) pst[j * 64 + lane] = (_Float16)(p[j] * nv);
        __builtin_amdgcn_wave_barrier();
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          half8 aop;
          if (m_row < NH) {
            const uint4 pa = *reinterpret_cast<const uint4 *>(wbuf + m_row * 128 + 64 * c + 16 * quarter);
            __builtin_memcpy(&aop, &pa, 16);
          } else {
            aop = half8{0, 0, 0, 0, 0, 0, 0, 0};
          }
          const uint32_t vwd[4] = {vw[c].x, vw[c].y, vw[c].z, vw[c].w};
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const uint32_t w = vwd[n >> 1];
            const uint32_t sel_lo = 0x0C020000u | ((4u + 2u * (n & 1)) << 8);
            const uint32_t sel_hi = 0x0C020000u | ((5u + 2u * (n & 1)) << 8);
            const uint2 lo = lds_u64(lds, __builtin_amdgcn_perm(w, vc8, sel_lo));
            const uint2 hi = lds_u64(lds, __builtin_amdgcn_perm(w, vc8, sel_hi));
            const uint32_t hv[4] = {lo.x, lo.y, hi.x, hi.y};
            half8 bop;
            __builtin_memcpy(&bop, hv, 16);
            oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, oacc[n], 0, 0, 0);
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
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) kw[s][r] = kw_n[s][r];
      vw[0] = vw_n[0];
      vw[1] = vw_n[1];
      nk_h = nk_n;
      nv_h = nv_n;
    }

    // ---- partials of this item
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const float lt = wave_sum(l_part[j]);
      if (lane == 0 && j < g)
        a.part_ml[((size_t)b * a.n_q_heads + kvh * g + j) * S + split] = make_float2(m_ref[j], lt);
    }
    if (!SPARSE) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int head = 4 * quarter + jj;
        if (head < g) {
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
  else if (a.group <= 8) decode_mfma_kernel<BK, 8, SPARSE><<<grid, kThreads, 0, stream>>>(a);
  else decode_mfma_kernel<BK, 16, SPARSE><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs &a) {
  return (a.k.bits == 3 || a.k.bits == 4) && a.v.bits == 2 && a.group <= 16 &&
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
