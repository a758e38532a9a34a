// Quantize (rotate, split off the fp16 norm, Lloyd-Max code, bit-pack) and dequantize
// kernels.
//
// [tq-80] "TurboQuant：让大模型本地推理内存占用降低80%的KV缓存压缩技术", §核心创新: random
// orthogonal rotation, per-coordinate Lloyd-Max scalar quantization with a precomputed
// codebook, vector norm stored separately as fp16.  [inferrs] "inferrs & TurboQuant：本地
// LLM 推理的内存革命", §核心技术: the rotation is a Walsh-Hadamard transform.
//
// Thread mapping: a block of 256 threads owns one 64-token chunk of one (batch, kv head)
// plane; 4 consecutive lanes own one vector, 32 coordinates each.  The Walsh-Hadamard
// transform runs 5 butterfly stages inside a lane and 2 across the lane quad.  Codes are
// staged in LDS and written out in the cache layout, so a GROUP8 group (8 tokens) is always
// produced by one block.
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
        uint16_t lo = ws[e] & 0xffff, hi = ws[e] >> 16;
        if (DTYPE == TQ_BF16) {
          v[8 * r + 2 * e] = __uint_as_float((uint32_t)lo << 16);
          v[8 * r + 2 * e + 1] = __uint_as_float((uint32_t)hi << 16);
        } else {
          v[8 * r + 2 * e] = half_bits_to_float(lo);
          v[8 * r + 2 * e + 1] = half_bits_to_float(hi);
        }
      }
    }
  }
}

// Unnormalised Walsh-Hadamard transform of 128 values held 32 per lane by a lane quad
// (lane q of the quad holds coordinates 32q .. 32q+31).
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
#pragma unroll
  for (int m = 1; m <= 2; m <<= 1) {
    const bool upper = (q & m) != 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      float o = __shfl_xor(v[e], m);
      v[e] = upper ? (o - v[e]) : (v[e] + o);
    }
  }
}

template <int DTYPE>
__global__ __launch_bounds__(256) void quantize_kernel(CacheView c, const void *__restrict__ x,
                                                       int start_pos, int n_tokens) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int chunk0 = (start_pos / kChunk + (int)blockIdx.x) * kChunk;
  const int lo = max(chunk0, start_pos), hi = min(chunk0 + kChunk, start_pos + n_tokens);
  const int bits = c.bits, levels = 1 << bits;

  __shared__ uint8_t codes[kChunk][kD];
  __shared__ float bnd[256];
  for (int i = threadIdx.x; i < levels - 1; i += blockDim.x) bnd[i] = c.boundaries[i];
  __syncthreads();

  const int j = threadIdx.x >> 2, q = threadIdx.x & 3;
  const int t = chunk0 + j;
  const bool valid = t >= lo && t < hi;
  float v[32];
  if (valid) {
    size_t row = ((size_t)b * n_tokens + (t - start_pos)) * c.n_kv_heads + h;
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
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = c.signs[32 * q + e] < 0 ? -v[e] : v[e];
  quad_fwht(v, q);
  const float n = sqrtf(ss);
  const float inv = n > 0.f ? 1.0f / (n * 11.313708498984761f) : 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const float u = v[e] * inv;
    int idx = 0;
    for (int step = levels >> 1; step >= 1; step >>= 1)
      if (u > bnd[idx + step - 1]) idx += step;
    codes[j][32 * q + e] = (uint8_t)idx;
  }
  if (valid && q == 0) c.norm_plane(b, h)[t] = float_to_half_bits(n);
  __syncthreads();

  uint8_t *plane = c.plane(b, h);
  if (c.layout == TQ_LAYOUT_ROWS) {
    const int words = 4 * bits;  // 16*bits bytes per row
    for (int idx = threadIdx.x; idx < kChunk * words; idx += blockDim.x) {
      const int jj = idx / words, w = idx % words, tt = chunk0 + jj;
      if (tt < lo || tt >= hi) continue;
      uint64_t acc = 0;
      for (int i = (32 * w) / bits; i < kD; ++i) {
        const int sh = bits * i - 32 * w;
        if (sh >= 32) break;
        const uint64_t cv = codes[jj][i];
        acc |= sh >= 0 ? (cv << sh) : (cv >> (-sh));
      }
      reinterpret_cast<uint32_t *>(plane + (size_t)tt * 16 * bits)[w] = (uint32_t)acc;
    }
  } else {
    for (int idx = threadIdx.x; idx < (kChunk / 8) * kD; idx += blockDim.x) {
      const int grp = idx / kD, i = idx % kD, tg = chunk0 + 8 * grp;
      uint64_t val = 0, mask = 0;
      const uint64_t field = (1ull << bits) - 1ull;
      for (int r = 0; r < 8; ++r) {
        const int tt = tg + r;
        if (tt < lo || tt >= hi) continue;
        val |= (uint64_t)codes[8 * grp + r][i] << (r * bits);
        mask |= field << (r * bits);
      }
      if (mask == 0) continue;
      uint8_t *dst = plane + (size_t)(tg >> 3) * kD * bits + (size_t)i * bits;
      for (int by = 0; by < bits; ++by) {
        const uint8_t m = (uint8_t)(mask >> (8 * by)), nv = (uint8_t)(val >> (8 * by));
        if (m == 0xff) dst[by] = nv;
        else if (m != 0) dst[by] = (uint8_t)((dst[by] & ~m) | (nv & m));
      }
    }
  }
}

template <int DTYPE>
__global__ __launch_bounds__(256) void dequantize_kernel(CacheView c, void *__restrict__ out,
                                                         int start_pos, int n_tokens) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int chunk0 = (start_pos / kChunk + (int)blockIdx.x) * kChunk;
  const int lo = max(chunk0, start_pos), hi = min(chunk0 + kChunk, start_pos + n_tokens);
  const int bits = c.bits, levels = 1 << bits;
  __shared__ float cen[256];
  for (int i = threadIdx.x; i < levels; i += blockDim.x) cen[i] = c.centroids[i];
  __syncthreads();
  const int j = threadIdx.x >> 2, q = threadIdx.x & 3;
  const int t = chunk0 + j;
  const bool valid = t >= lo && t < hi;
  const uint8_t *plane = c.plane(b, h);
  float v[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    v[e] = valid ? cen[read_field(plane, code_bit_offset(c.layout, bits, t, 32 * q + e), bits)] : 0.f;
  }
  quad_fwht(v, q);
  if (!valid) return;
  const float scale = half_bits_to_float(c.norm_plane(b, h)[t]) * kInvSqrtD;
  const size_t row = ((size_t)b * n_tokens + (t - start_pos)) * c.n_kv_heads + h;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const float s = c.signs[32 * q + e] < 0 ? -scale : scale;
    store_elem(out, row * kD + 32 * q + e, v[e] * s, DTYPE);
  }
}

}  // namespace

hipError_t launch_quantize(const CacheView &c, int batch, const void *x, int x_dtype,
                           int start_pos, int n_tokens, hipStream_t stream) {
  const int first = start_pos / kChunk, last = (start_pos + n_tokens - 1) / kChunk;
  dim3 grid(last - first + 1, c.n_kv_heads, batch);
  if (x_dtype == TQ_F32)
    quantize_kernel<TQ_F32><<<grid, 256, 0, stream>>>(c, x, start_pos, n_tokens);
  else if (x_dtype == TQ_BF16)
    quantize_kernel<TQ_BF16><<<grid, 256, 0, stream>>>(c, x, start_pos, n_tokens);
  else
    quantize_kernel<TQ_F16><<<grid, 256, 0, stream>>>(c, x, start_pos, n_tokens);
  return hipGetLastError();
}

hipError_t launch_dequantize(const CacheView &c, int batch, void *out, int out_dtype,
                             int start_pos, int n_tokens, hipStream_t stream) {
  const int first = start_pos / kChunk, last = (start_pos + n_tokens - 1) / kChunk;
  dim3 grid(last - first + 1, c.n_kv_heads, batch);
  if (out_dtype == TQ_F32)
    dequantize_kernel<TQ_F32><<<grid, 256, 0, stream>>>(c, out, start_pos, n_tokens);
  else if (out_dtype == TQ_BF16)
    dequantize_kernel<TQ_BF16><<<grid, 256, 0, stream>>>(c, out, start_pos, n_tokens);
  else
    dequantize_kernel<TQ_F16><<<grid, 256, 0, stream>>>(c, out, start_pos, n_tokens);
  return hipGetLastError();
}

}  // namespace tq
