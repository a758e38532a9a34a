// Shared device helpers and launch-parameter structs for the TurboQuant HIP kernels.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace tq {

constexpr int kD = 128;            // head dim supported by the kernels
constexpr int kChunk = 64;         // tokens per quantize / dequantize block (capacity multiple)

// One (batch, kv head) plane of a cache as the kernels see it.
struct CacheView {
  uint8_t *codes;
  uint16_t *norms;
  const float *centroids;
  const float *boundaries;
  const int8_t *signs;
  int bits;
  int layout;
  int n_kv_heads;
  int capacity;
  float table_scale;  // value centroids in the fp16 operand table are scaled by this (1: none)
  __host__ __device__ size_t code_plane_bytes() const { return (size_t)capacity * kD * bits / 8; }
  __device__ uint8_t *plane(int b, int h) const {
    return codes + ((size_t)b * n_kv_heads + h) * code_plane_bytes();
  }
  __device__ uint16_t *norm_plane(int b, int h) const {
    return norms + ((size_t)b * n_kv_heads + h) * capacity;
  }
};

__device__ __forceinline__ float load_elem(const void *p, size_t i, int dtype) {
  if (dtype == TQ_F32) return reinterpret_cast<const float *>(p)[i];
  uint16_t bits = reinterpret_cast<const uint16_t *>(p)[i];
  if (dtype == TQ_BF16) return __uint_as_float((uint32_t)bits << 16);
  return __half2float(__ushort_as_half(bits));
}

__device__ __forceinline__ void store_elem(void *p, size_t i, float v, int dtype) {
  if (dtype == TQ_F32) {
    reinterpret_cast<float *>(p)[i] = v;
  } else if (dtype == TQ_BF16) {
    reinterpret_cast<__hip_bfloat16 *>(p)[i] = __float2bfloat16(v);
  } else {
    reinterpret_cast<__half *>(p)[i] = __float2half(v);
  }
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

// fp32 -> IEEE fp16 bits, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __half_as_ushort(__float2half_rn(f));
}

// Read the `bits`-bit field starting at bit offset `pos` of a byte array (LSB first).
// Only the bytes that hold the field are read.
__device__ __forceinline__ uint32_t read_field(const uint8_t *base, uint64_t pos, int bits) {
  const uint8_t *p = base + (pos >> 3);
  uint32_t sh = pos & 7;
  uint32_t w = p[0];
  if (bits + sh > 8) w |= (uint32_t)p[1] << 8;
  if (bits + sh > 16) w |= (uint32_t)p[2] << 16;
  return (w >> sh) & ((1u << bits) - 1u);
}

// Bit offset of code (t, i) inside a plane, for the two layouts of tq.h.
__device__ __forceinline__ uint64_t code_bit_offset(int layout, int bits, int t, int i) {
  if (layout == TQ_LAYOUT_ROWS) return ((uint64_t)t * kD + i) * bits;
  return (uint64_t)(t >> 3) * (kD * 8 * bits) + ((uint32_t)i * 8 + (t & 7)) * bits;
}

// In-place Walsh-Hadamard transform (Sylvester order, unnormalised) of `n_vec` vectors of
// length 128 stored contiguously in shared memory, by all threads of the block.
__device__ __forceinline__ void block_fwht128(float *buf, int n_vec) {
  for (int h = 1; h < kD; h <<= 1) {
    __syncthreads();
    for (int e = threadIdx.x; e < n_vec * (kD / 2); e += blockDim.x) {
      int v = e / (kD / 2), r = e % (kD / 2);
      int i = (r / h) * 2 * h + (r % h);
      float a = buf[v * kD + i], c = buf[v * kD + i + h];
      buf[v * kD + i] = a + c;
      buf[v * kD + i + h] = a - c;
    }
  }
  __syncthreads();
}

}  // namespace tq
