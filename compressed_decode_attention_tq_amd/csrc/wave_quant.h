// Per-wave quantization of one token (two coordinates per lane, the transform and the
// reductions in registers): the input pair of a lane, the norm and rotation, the Lloyd-Max
// code search and the assembly of a key row.  Shared by the small-append kernels and the QJL
// quantize kernel ([tq-80] §核心创新: norm split off, random rotation, data-independent
// Lloyd-Max code; [inferrs] §核心技术: Walsh-Hadamard rotation).
#pragma once

#include "tq_common.h"
#include "lanes.h"

namespace tq {

// input element pair (2 lane, 2 lane + 1) of one token row
template <int DTYPE>
__device__ __forceinline__ void load_pair(const void *x, size_t i, float &x0, float &x1) {
  if constexpr (DTYPE == TQ_F32) {
    const float2 f = *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(x) + i);
    x0 = f.x;
    x1 = f.y;
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(x) + i);
    if constexpr (DTYPE == TQ_BF16) {
      x0 = __uint_as_float(w << 16);
      x1 = __uint_as_float(w & 0xffff0000u);
    } else {
      x0 = __half2float(__ushort_as_half((uint16_t)(w & 0xffffu)));
      x1 = __half2float(__ushort_as_half((uint16_t)(w >> 16)));
    }
  }
}

// The norm of one token and coordinates 2 lane, 2 lane + 1 of H (s . x) (the rotation before
// its 1 / sqrt(d)).
__device__ __forceinline__ void token_transform(const CacheView &c, float x0, float x1, int lane, float &h0,
                                                float &h1, float &n) {
  n = sqrtf(wave_reduce<false>(x0 * x0 + x1 * x1));
  const float y0 = c.signs[2 * lane] < 0 ? -x0 : x0, y1 = c.signs[2 * lane + 1] < 0 ? -x1 : x1;
  h0 = y0 + y1;  // stage 0 of the transform, inside the lane
  h1 = y0 - y1;
  wave_fwht_upper(h0, h1, lane);
}

// codes of coordinates 2 lane, 2 lane + 1 and the norm of one token; h0, h1 as token_transform
template <int BITS>
__device__ __forceinline__ void token_codes(const CacheView &c, float x0, float x1, int lane, uint32_t &c0,
                                            uint32_t &c1, float &n, float &h0, float &h1) {
  token_transform(c, x0, x1, lane, h0, h1, n);
  const float inv = n > 0.f ? 1.0f / (n * 11.313708498984761f) : 0.f;
  const float u0 = h0 * inv, u1 = h1 * inv;
  c0 = 0u;
  c1 = 0u;
  for (int j = 0; j < (1 << BITS) - 1; ++j) {
    const float t = c.boundaries[j];
    c0 += u0 > t ? 1u : 0u;
    c1 += u1 > t ? 1u : 0u;
  }
}

// Key rows: lane l's two codes are bits [2 BITS l, 2 BITS (l + 1)) of the token's row of
// 16 BITS bytes; the row is assembled in LDS (4 BITS words) and stored by the first lanes.
template <int BITS>
__device__ __forceinline__ void store_row(uint8_t *row, uint32_t c0, uint32_t c1, int lane, uint32_t *words) {
  constexpr int kWords = 4 * BITS;
  if (lane < kWords) words[lane] = 0u;
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
  const uint32_t f = c0 | (c1 << BITS);
  const int bit = 2 * BITS * lane, wi = bit >> 5, sh = bit & 31;
  atomicOr(&words[wi], f << sh);
  if (sh + 2 * BITS > 32) atomicOr(&words[wi + 1], f >> (32 - sh));
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
  if (lane < kWords) reinterpret_cast<uint32_t *>(row)[lane] = words[lane];
}

}  // namespace tq
