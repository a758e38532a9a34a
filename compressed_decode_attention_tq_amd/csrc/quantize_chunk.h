// Quantization of one 64-token chunk of a cache plane: the work of a 256-thread block,
// shared by the single-cache and the key-and-value kernels.
//
// [tq-80] "TurboQuant：让大模型本地推理内存占用降低80%的KV缓存压缩技术", §核心创新: random
// orthogonal rotation, per-coordinate Lloyd-Max scalar quantization with a precomputed
// codebook, vector norm stored separately as fp16.  [inferrs] "inferrs & TurboQuant：本地
// LLM 推理的内存革命", §核心技术: the rotation is a Walsh-Hadamard transform.
//
// Quantize mapping: a block of 256 threads covers one 64-token chunk of one (batch, kv head)
// plane and each of its waves owns 16 consecutive tokens (two 8-token value groups), so the
// waves never wait for each other.  4 lanes hold one vector, 32 coordinates each: the
// Walsh-Hadamard transform runs 5 butterfly stages inside a lane and 2 across the lane quad
// (DPP moves).  Codes of codebooks with up to 16 levels come from a per-wave uniform grid in
// LDS (one lookup, one compare); when a codebook does not fit the grid, the code is counted
// with compares against the L/2 - 1 positive boundaries (the codebook is symmetric:
// t_{L-2-j} = -t_j, t_{L/2-1} = 0).  256-level codebooks use a binary search over the
// boundaries in LDS.  Row-layout codes are packed inside the lane; value-group codes go
// through a per-wave LDS transpose.
#pragma once
#include "tq_common.h"
#include "tq_launch.h"

namespace tq {
namespace {

constexpr float kInvSqrtD = 0.08838834764831845f;  // 1 / sqrt(128)

template <int DTYPE>
__device__ __forceinline__ void load32(const void *x, size_t base, float v[32]) {
  if (DTYPE == TQ_F32) {
    const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + base);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float4 f = p[r];
      v[4 * r] = f.x; v[4 * r + 1] = f.y; v[4 * r + 2] = f.z; v[4 * r + 3] = f.w;
    }
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + base);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint4 w = p[r];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (DTYPE == TQ_BF16) {
          v[8 * r + 2 * e] = __uint_as_float(ws[e] << 16);
          v[8 * r + 2 * e + 1] = __uint_as_float(ws[e] & 0xffff0000u);
        } else {
          v[8 * r + 2 * e] = half_bits_to_float((uint16_t)(ws[e] & 0xffffu));
          v[8 * r + 2 * e + 1] = half_bits_to_float((uint16_t)(ws[e] >> 16));
        }
      }
    }
  }
}

// Value of the same register in lane (lane ^ m) of the quad, m = 1 (quad_perm 1,0,3,2:
// control 0xB1) or m = 2 (quad_perm 2,3,0,1: control 0x4E), through a DPP move.
template <int CTRL>
__device__ __forceinline__ float quad_swap(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Unnormalised Walsh-Hadamard transform of 128 values held 32 per lane by a lane quad
// (lane q of the quad holds coordinates 32q .. 32q+31): five butterfly stages inside the
// lane, then two across the quad, where the upper lane of a pair keeps partner - own and
// the lower one partner + own (one multiply-add by a per-lane sign of +-1, exact).
__device__ __forceinline__ void quad_fwht(float v[32], int q) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      if ((e & h) == 0) {
        float a = v[e], c = v[e + h];
        v[e] = a + c;
        v[e + h] = a - c;
      }
    }
  }
  const float s1 = (q & 1) ? -1.f : 1.f, s2 = (q & 2) ? -1.f : 1.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = fmaf(s1, v[e], quad_swap<0xB1>(v[e]));
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = fmaf(s2, v[e], quad_swap<0x4E>(v[e]));
}

// code = #{j : t_j < u} for a symmetric codebook of 2^BITS levels (BITS <= 4); `pos` holds
// the positive boundaries t_{L/2} .. t_{L-2}.
template <int BITS>
__device__ __forceinline__ uint32_t code_of(float u, const float *pos) {
  constexpr int L = 1 << BITS;
  // for u < 0 count the boundaries <= |u|: compare against the next float above |u|
  float a = fabsf(u);
  if (u < 0.f) a = __uint_as_float(__float_as_uint(a) + 1u);
  uint32_t cnt = 0;
#pragma unroll
  for (int k = 0; k < L / 2 - 1; ++k) cnt += pos[k] < a ? 1u : 0u;
  return u > 0.f ? (uint32_t)(L / 2) + cnt : (uint32_t)(L / 2 - 1) - cnt;
}

// code = #{j : t_j < u} by binary search over 255 boundaries in LDS.
__device__ __forceinline__ uint32_t code_of_8(float u, const float *bnd) {
  uint32_t idx = 0;
#pragma unroll
  for (int step = 128; step >= 1; step >>= 1)
    if (bnd[idx + step - 1] < u) idx += step;
  return idx;
}

constexpr int kGridCells = 64;

struct QuantLds {
  __attribute__((aligned(16))) uint8_t stage[4][16][kD];  // value-group transpose
  float bnd8[4][256];                                      // 8-bit boundaries
  uint2 grid[4][kGridCells];                               // per-wave code grid
};

// Code search by a uniform grid over the boundaries (codebooks of up to 16 levels).  Cell
// c = trunc(clamp(u * scale + offset, 0, cells - 1)) holds at most one boundary; its entry is
// {#{t_j < lower edge of c}, that boundary or +inf}, so code = entry.x + (u > entry.y).
// Cell 0 reaches down to -inf and the last cell up to +inf.  A u that rounds into a
// neighbouring cell can only change its code when a boundary lies between u and the cell
// edge, i.e. within the rounding of u (far below 1e-6).
struct CodeGrid {
  float scale, offset, last_cell;
  int cells;
  bool ok;
};

// Builds the wave's grid from the L/2 - 1 positive boundaries (the codebook is symmetric:
// t = -pos reversed, 0, pos).  ok is false when the grid would need more than kGridCells
// cells or a cell would hold two boundaries; the caller then counts compares instead.
template <int BITS>
__device__ CodeGrid build_code_grid(const float *pos, uint2 *grid, int lane) {
  constexpr int L = 1 << BITS, NP = L / 2 - 1;
  float gap = pos[0];
#pragma unroll
  for (int k = 0; k + 1 < NP; ++k) gap = fminf(gap, pos[k + 1] - pos[k]);
  const float w = 0.75f * gap;
  const float lo = -pos[NP - 1] - 0.5f * w;
  CodeGrid gd;
  gd.cells = (int)ceilf((2.f * pos[NP - 1] + w) / w) + 1;
  gd.last_cell = (float)(gd.cells - 1);
  gd.scale = 1.f / w;
  gd.offset = -lo / w;
  gd.ok = gap > 0.f && gd.cells <= kGridCells;
  if (!gd.ok) return gd;
  const int cidx = lane;
  const float e0 = lo + (float)cidx * w;        // lower edge (cell 0: -inf)
  const float e1 = lo + (float)(cidx + 1) * w;  // upper edge (last cell: +inf)
  const bool first = cidx == 0, last = cidx == gd.cells - 1;
  uint32_t base = 0, inside = 0;
  float bnd = INFINITY;
  auto visit = [&](float t) {
    const bool below = !first && t < e0;
    const bool in = !below && (last || t < e1);
    base += below ? 1u : 0u;
    inside += in ? 1u : 0u;
    if (in) bnd = fminf(bnd, t);
  };
#pragma unroll
  for (int k = NP - 1; k >= 0; --k) visit(-pos[k]);
  visit(0.f);
#pragma unroll
  for (int k = 0; k < NP; ++k) visit(pos[k]);
  const bool bad = cidx < gd.cells && inside > 1u;
  gd.ok = __ballot(bad) == 0ull;
  if (cidx < gd.cells) grid[cidx] = make_uint2(base, __float_as_uint(bnd));
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
  return gd;
}

__device__ __forceinline__ uint32_t code_by_grid(float u, const CodeGrid &gd, const uint2 *grid) {
  const int cidx = (int)__builtin_amdgcn_fmed3f(fmaf(u, gd.scale, gd.offset), 0.f, gd.last_cell);
  const uint2 e = grid[cidx];
  return e.x + (u > __uint_as_float(e.y) ? 1u : 0u);
}

// One 64-token chunk (chunk index bx counted from the chunk of start_pos) of the plane of
// (batch b, kv head h).
template <int DTYPE, int BITS, int LAYOUT>
__device__ __forceinline__ void quantize_chunk(const CacheView &c, const void *__restrict__ x,
                                               int start_pos, int n_tokens, int h, int b, int bx,
                                               QuantLds &sh) {
  constexpr int L = 1 << BITS;
  const int chunk0 = (start_pos / kChunk + bx) * kChunk;
  const int lo = max(chunk0, start_pos), hi = min(chunk0 + kChunk, start_pos + n_tokens);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wt0 = chunk0 + 16 * wave;
  if (wt0 + 16 <= lo || wt0 >= hi) return;  // no token of this wave is in the range

  const int j = lane >> 2, q = lane & 3;
  const int t = wt0 + j;
  const bool valid = t >= lo && t < hi;

  float pos[L / 2 > 1 ? L / 2 - 1 : 1];
  CodeGrid gd{0.f, 0.f, 0.f, 0, false};
  if (BITS <= 4) {
#pragma unroll
    for (int k = 0; k < L / 2 - 1; ++k) pos[k] = c.boundaries[L / 2 + k];
    gd = build_code_grid<BITS <= 4 ? BITS : 4>(pos, sh.grid[wave], lane);
  } else {
    for (int k = lane; k < L - 1; k += 64) sh.bnd8[wave][k] = c.boundaries[k];
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
  }

  float v[32];
  if (valid) {
    const size_t row = ((size_t)b * n_tokens + (t - start_pos)) * c.n_kv_heads + h;
    load32<DTYPE>(x, row * kD + 32 * q, v);
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) ss = fmaf(v[e], v[e], ss);
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  {
    const int4 sw0 = *reinterpret_cast<const int4 *>(c.signs + 32 * q);
    const int4 sw1 = *reinterpret_cast<const int4 *>(c.signs + 32 * q + 16);
    const int sw[8] = {sw0.x, sw0.y, sw0.z, sw0.w, sw1.x, sw1.y, sw1.z, sw1.w};
#pragma unroll
    for (int e = 0; e < 32; ++e) {  // flip the sign bit where s_i = -1 (byte 0xff)
      const uint32_t neg = ((uint32_t)sw[e >> 2] >> (8 * (e & 3) + 7)) & 1u;
      v[e] = __uint_as_float(__float_as_uint(v[e]) ^ (neg << 31));
    }
  }
  quad_fwht(v, q);
  const float n = sqrtf(ss);
  const float inv = n > 0.f ? 1.0f / (n * 11.313708498984761f) : 0.f;
  uint32_t code[32];
  if (BITS <= 4 && gd.ok) {
#pragma unroll
    for (int e = 0; e < 32; ++e) code[e] = code_by_grid(v[e] * inv, gd, sh.grid[wave]);
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float u = v[e] * inv;
      code[e] = BITS <= 4 ? code_of<BITS <= 4 ? BITS : 4>(u, pos) : code_of_8(u, sh.bnd8[wave]);
    }
  }
  if (valid && q == 0) c.norm_plane(b, h)[t] = float_to_half_bits(n);

  uint8_t *plane = c.plane(b, h);
  if (LAYOUT == TQ_LAYOUT_ROWS) {
    // the lane's 32 codes are bits [32*BITS*q, 32*BITS*(q+1)) of the token's row
    uint32_t w[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k] = 0u;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int bit = e * BITS;
      w[bit >> 5] |= code[e] << (bit & 31);
      if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= code[e] >> (32 - (bit & 31));
    }
    if (valid) {
      uint32_t *dst = reinterpret_cast<uint32_t *>(plane + (size_t)t * 16 * BITS + 4 * BITS * q);
#pragma unroll
      for (int k = 0; k < BITS; ++k) dst[k] = w[k];
    }
  } else {
    // stage codes [token][coord] as bytes, then lane r of a group builds coordinates
    // 4r .. 4r+3 of its group: 8 tokens x BITS bits per coordinate, BITS bytes each
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint32_t pk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        pk[k] = code[16 * r + 4 * k] | (code[16 * r + 4 * k + 1] << 8) | (code[16 * r + 4 * k + 2] << 16) |
                (code[16 * r + 4 * k + 3] << 24);
      *reinterpret_cast<uint4 *>(&sh.stage[wave][j][32 * q + 16 * r]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
    const int gi = lane >> 5, r = lane & 31;
    const int tg = wt0 + 8 * gi;  // first token of the group
    uint64_t chunk[4] = {0, 0, 0, 0}, mask = 0;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const uint32_t cw = *reinterpret_cast<const uint32_t *>(&sh.stage[wave][8 * gi + tt][4 * r]);
      const bool in = tg + tt >= lo && tg + tt < hi;
      if (in) mask |= (uint64_t)(L - 1) << (tt * BITS);
#pragma unroll
      for (int k = 0; k < 4; ++k) chunk[k] |= (uint64_t)((cw >> (8 * k)) & 0xffu) << (tt * BITS);
    }
    if (mask != 0) {
      // the 4 coordinate chunks are 4*BITS consecutive bytes: pack them into BITS dwords
      uint32_t out[BITS], msk[BITS];
#pragma unroll
      for (int k = 0; k < BITS; ++k) { out[k] = 0u; msk[k] = 0u; }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int bit = k * 8 * BITS;  // bit offset of chunk k
        const uint64_t cv = chunk[k] & mask;
#pragma unroll
        for (int part = 0; part < (8 * BITS + 31) / 32 + 1; ++part) {
          const int wb = (bit >> 5) + part;  // destination dword
          if (wb >= BITS) break;
          const int sh = 32 * wb - bit;     // chunk bit that lands at bit 0 of dword wb
          if (sh >= 8 * BITS) break;
          if (sh >= 0) {
            out[wb] |= (uint32_t)(cv >> sh);
            msk[wb] |= (uint32_t)(mask >> sh);
          } else {
            out[wb] |= (uint32_t)(cv << (-sh));
            msk[wb] |= (uint32_t)(mask << (-sh));
          }
        }
      }
      uint32_t *dst = reinterpret_cast<uint32_t *>(plane + (size_t)(tg >> 3) * kD * BITS + 4 * BITS * r);
#pragma unroll
      for (int k = 0; k < BITS; ++k) {
        if (msk[k] == 0xffffffffu) dst[k] = out[k];
        else if (msk[k] != 0u) dst[k] = (dst[k] & ~msk[k]) | out[k];
      }
    }
  }
}

}  // namespace
}  // namespace tq
