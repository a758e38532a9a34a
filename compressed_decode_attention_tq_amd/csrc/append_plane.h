// One wave per new token of one (batch, kv head) plane, shared by the small-append kernels
// (append_small.hip) and the QJL key-and-value append (qjl.hip): keys write their rows,
// value codes meet in LDS and wave 0 then updates each 8-token value group once.
#pragma once

#include "tq_common.h"
#include "tq_launch.h"
#include "lanes.h"
#include "wave_quant.h"

namespace tq {
namespace {

// Value groups: coordinate i of token p of a group sits at bit (8 i + p) BITS, so lane l's
// coordinates 2l and 2l + 1 of all 8 tokens are the 2 BITS bytes at 2 BITS l of the group,
// which the lane reads, updates for every new token of the group, and writes back.
template <int BITS>
struct GroupSlice {
  uint64_t lo = 0, hi = 0;
  __device__ void load(const uint8_t *g, int lane) {
    const uint8_t *p = g + 2 * BITS * lane;
    if constexpr (BITS == 2) {
      lo = *reinterpret_cast<const uint32_t *>(p);
    } else if constexpr (BITS == 3) {
      const uint16_t *h = reinterpret_cast<const uint16_t *>(p);
      lo = (uint64_t)h[0] | ((uint64_t)h[1] << 16) | ((uint64_t)h[2] << 32);
    } else if constexpr (BITS == 4) {
      lo = *reinterpret_cast<const uint64_t *>(p);
    } else {
      const uint2 a = *reinterpret_cast<const uint2 *>(p), b = *reinterpret_cast<const uint2 *>(p + 8);
      lo = (uint64_t)a.x | ((uint64_t)a.y << 32);
      hi = (uint64_t)b.x | ((uint64_t)b.y << 32);
    }
  }
  __device__ void store(uint8_t *g, int lane) const {
    uint8_t *p = g + 2 * BITS * lane;
    if constexpr (BITS == 2) {
      *reinterpret_cast<uint32_t *>(p) = (uint32_t)lo;
    } else if constexpr (BITS == 3) {
      uint16_t *h = reinterpret_cast<uint16_t *>(p);
      h[0] = (uint16_t)lo;
      h[1] = (uint16_t)(lo >> 16);
      h[2] = (uint16_t)(lo >> 32);
    } else if constexpr (BITS == 4) {
      *reinterpret_cast<uint64_t *>(p) = lo;
    } else {
      *reinterpret_cast<uint2 *>(p) = make_uint2((uint32_t)lo, (uint32_t)(lo >> 32));
      *reinterpret_cast<uint2 *>(p + 8) = make_uint2((uint32_t)hi, (uint32_t)(hi >> 32));
    }
  }
  __device__ void set(int pos, uint32_t code) {  // no field straddles bit 64
    constexpr uint64_t kMask = (1ull << BITS) - 1ull;
    if (pos < 64) lo = (lo & ~(kMask << pos)) | ((uint64_t)code << pos);
    else hi = (hi & ~(kMask << (pos - 64))) | ((uint64_t)code << (pos - 64));
  }
};

// Wave j of the block takes token j of the plane: keys write their rows directly; value
// codes meet in LDS and wave 0 then updates each value group the tokens touch, once.
struct SmallLds {
  uint32_t words[kSmallAppendMax][32];  // key row assembly, per wave
  uint2 codes[kSmallAppendMax][64];     // value codes (coordinates 2 lane, 2 lane + 1)
};

template <int DTYPE, int BITS, bool KEY>
__device__ void append_plane(const CacheView &c, const void *x, int b, int h, int start_pos, int n_tokens, int wave,
                             int lane, SmallLds &sh) {
  uint8_t *plane = c.plane(b, h);
  if (wave < n_tokens) {
    const int t = start_pos + wave;
    float x0, x1;
    load_pair<DTYPE>(x, (((size_t)b * n_tokens + wave) * c.n_kv_heads + h) * kD + 2 * lane, x0, x1);
    uint32_t c0, c1;
    float n;
    float h0, h1;
    token_codes<BITS>(c, x0, x1, lane, c0, c1, n, h0, h1);
    if (lane == 0) c.norm_plane(b, h)[t] = float_to_half_bits(n);
    if constexpr (KEY) store_row<BITS>(plane + (size_t)t * (16 * BITS), c0, c1, lane, sh.words[wave]);
    else sh.codes[wave][lane] = make_uint2(c0, c1);
  }
  if constexpr (!KEY) {
    __syncthreads();
    if (wave == 0) {
      GroupSlice<BITS> slice;
      int group = -1;
      for (int j = 0; j < n_tokens; ++j) {
        const int t = start_pos + j;
        if ((t >> 3) != group) {
          if (group >= 0) slice.store(plane + (size_t)group * (kD * BITS), lane);
          group = t >> 3;
          slice.load(plane + (size_t)group * (kD * BITS), lane);
        }
        const uint2 cc = sh.codes[j][lane];
        slice.set((t & 7) * BITS, cc.x);
        slice.set((8 + (t & 7)) * BITS, cc.y);
      }
      slice.store(plane + (size_t)group * (kD * BITS), lane);
    }
  }
}

}  // namespace
}  // namespace tq
