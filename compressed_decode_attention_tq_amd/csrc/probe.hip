// Streaming-read probe: the HBM read bandwidth a plain kernel reaches on this device, the
// ceiling the decode kernels' achieved bandwidth is compared with (measurement only; not a
// step of the method).  256 workgroups of 512 threads sweep the buffer grid-stride, four
// 16-byte loads in flight per thread; the data are folded into one word that is stored
// only if it equals a constant, so the loads cannot be dropped.
#include "tq_common.h"

#include "tq_probe.h"

namespace {

__global__ __launch_bounds__(512) void stream_read_kernel(const uint4 *__restrict__ p, size_t n16,
                                                          unsigned *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" int tq_probe_stream_read(const void *buf, size_t bytes, unsigned *sink, void *hip_stream) {
  if (buf == nullptr || sink == nullptr || bytes < 16 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
    return TQ_ERR_INVALID_ARG;
  stream_read_kernel<<<256, 512, 0, static_cast<hipStream_t>(hip_stream)>>>(
      static_cast<const uint4 *>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
