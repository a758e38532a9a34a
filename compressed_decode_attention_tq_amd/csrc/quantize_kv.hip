// Quantize one token range into a key cache (row layout) and a value cache (8-token value
// groups) with a single launch: blocks with blockIdx.z < batch take the key planes, the
// others the value planes.  Decoding appends the new token's key and value at every step,
// and one launch instead of two halves the fixed launch latency of that step.
#include "quantize_chunk.h"

namespace tq {
namespace {

template <int DTYPE, int BK, int BV>
__global__ __launch_bounds__(256) void quantize_kv_kernel(CacheView kc, CacheView vc,
                                                          const void *__restrict__ xk,
                                                          const void *__restrict__ xv,
                                                          int start_pos, int n_tokens, int batch) {
  __shared__ QuantLds sh;
  const int z = blockIdx.z;
  if (z < batch)
    quantize_chunk<DTYPE, BK, TQ_LAYOUT_ROWS>(kc, xk, start_pos, n_tokens, blockIdx.y, z, blockIdx.x, sh);
  else
    quantize_chunk<DTYPE, BV, TQ_LAYOUT_GROUP8>(vc, xv, start_pos, n_tokens, blockIdx.y, z - batch,
                                                blockIdx.x, sh);
}

template <int DTYPE, int BK>
void launch_kv_bv(const CacheView &kc, const CacheView &vc, dim3 grid, const void *xk, const void *xv,
                  int start_pos, int n_tokens, int batch, hipStream_t stream) {
  switch (vc.bits) {
    case 2: quantize_kv_kernel<DTYPE, BK, 2><<<grid, 256, 0, stream>>>(kc, vc, xk, xv, start_pos, n_tokens, batch); break;
    case 3: quantize_kv_kernel<DTYPE, BK, 3><<<grid, 256, 0, stream>>>(kc, vc, xk, xv, start_pos, n_tokens, batch); break;
    case 4: quantize_kv_kernel<DTYPE, BK, 4><<<grid, 256, 0, stream>>>(kc, vc, xk, xv, start_pos, n_tokens, batch); break;
    default: quantize_kv_kernel<DTYPE, BK, 8><<<grid, 256, 0, stream>>>(kc, vc, xk, xv, start_pos, n_tokens, batch); break;
  }
}

template <int DTYPE>
void launch_kv(const CacheView &kc, const CacheView &vc, dim3 grid, const void *xk, const void *xv,
               int start_pos, int n_tokens, int batch, hipStream_t stream) {
  switch (kc.bits) {
    case 2: launch_kv_bv<DTYPE, 2>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, stream); break;
    case 3: launch_kv_bv<DTYPE, 3>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, stream); break;
    case 4: launch_kv_bv<DTYPE, 4>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, stream); break;
    default: launch_kv_bv<DTYPE, 8>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, stream); break;
  }
}

}  // namespace

hipError_t launch_quantize_kv(const CacheView &kc, const CacheView &vc, int batch, const void *xk,
                              const void *xv, int x_dtype, int start_pos, int n_tokens,
                              hipStream_t stream) {
  const int first = start_pos / kChunk, last = (start_pos + n_tokens - 1) / kChunk;
  dim3 grid((last - first + kChunksPerBlock) / kChunksPerBlock, kc.n_kv_heads, 2 * batch);
  if (x_dtype == TQ_F32) launch_kv<TQ_F32>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, stream);
  else if (x_dtype == TQ_BF16) launch_kv<TQ_BF16>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, stream);
  else launch_kv<TQ_F16>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, stream);
  return hipGetLastError();
}

}  // namespace tq
