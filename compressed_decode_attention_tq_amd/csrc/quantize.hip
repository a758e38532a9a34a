// Quantize (rotate, split off the fp16 norm, Lloyd-Max code, bit-pack) and dequantize
// kernels; the per-chunk quantization is in quantize_chunk.h.
#include "quantize_chunk.h"

namespace tq {
namespace {

template <int DTYPE, int BITS, int LAYOUT>
__global__ __launch_bounds__(256) void quantize_kernel(CacheView c, const void *__restrict__ x,
                                                       int start_pos, int n_tokens) {
  __shared__ QuantLds sh;
  quantize_chunk<DTYPE, BITS, LAYOUT>(c, x, start_pos, n_tokens, blockIdx.y, blockIdx.z, blockIdx.x, sh);
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
  const float scale = half_bits_to_float(c.norm_plane(b, h)[t]) * kInvSqrtD * quad_fwht_sign(q);
  const size_t row = ((size_t)b * n_tokens + (t - start_pos)) * c.n_kv_heads + h;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const float s = c.signs[32 * q + e] < 0 ? -scale : scale;
    store_elem(out, row * kD + 32 * q + e, v[e] * s, DTYPE);
  }
}


template <int DTYPE, int BITS>
void launch_q(const CacheView &c, dim3 grid, const void *x, int start_pos, int n_tokens, hipStream_t stream) {
  if (c.layout == TQ_LAYOUT_ROWS)
    quantize_kernel<DTYPE, BITS, TQ_LAYOUT_ROWS><<<grid, 256, 0, stream>>>(c, x, start_pos, n_tokens);
  else
    quantize_kernel<DTYPE, BITS, TQ_LAYOUT_GROUP8><<<grid, 256, 0, stream>>>(c, x, start_pos, n_tokens);
}

template <int DTYPE>
void launch_qd(const CacheView &c, dim3 grid, const void *x, int start_pos, int n_tokens, hipStream_t stream) {
  switch (c.bits) {
    case 2: launch_q<DTYPE, 2>(c, grid, x, start_pos, n_tokens, stream); break;
    case 3: launch_q<DTYPE, 3>(c, grid, x, start_pos, n_tokens, stream); break;
    case 4: launch_q<DTYPE, 4>(c, grid, x, start_pos, n_tokens, stream); break;
    default: launch_q<DTYPE, 8>(c, grid, x, start_pos, n_tokens, stream); break;
  }
}

}  // namespace

hipError_t launch_quantize(const CacheView &c, int batch, const void *x, int x_dtype,
                           int start_pos, int n_tokens, hipStream_t stream) {
  const int first = start_pos / kChunk, last = (start_pos + n_tokens - 1) / kChunk;
  dim3 grid((last - first + kChunksPerBlock) / kChunksPerBlock, c.n_kv_heads, batch);
  if (x_dtype == TQ_F32) launch_qd<TQ_F32>(c, grid, x, start_pos, n_tokens, stream);
  else if (x_dtype == TQ_BF16) launch_qd<TQ_BF16>(c, grid, x, start_pos, n_tokens, stream);
  else launch_qd<TQ_F16>(c, grid, x, start_pos, n_tokens, stream);
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
