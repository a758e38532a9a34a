// QJL residual variant of the key quantizer ([google] "Google 最新極限壓縮算法…", §第二步：QJL
// —— 1 bit 清理殘差, and its mlx-vlm kernel list: _qjl_score_kernel, _prod_score_kernel;
// [tq-80] "TurboQuant：让大模型本地推理内存占用降低80%的KV缓存压缩技术" §技术背景与学术渊源).
//
// After the rotate-and-code stage, one bit per row of a Gaussian matrix S records the sign of
// the projection of the stage's error, so that inner products with the key (attention scores)
// are unbiased.  Per token, one wave of 64 lanes, two coordinates per lane:
//   n = ||x||, h = H (s . x) (lanes.h butterflies), code_i = #{j : t_j < h_i / (sqrt(d) n)}
//   (the same steps as the small-append kernels, wave_quant.h);
//   r_i = h_i / sqrt(d) - n16 c[code_i]       the error of the reconstruction the decoder
//                                             makes (n16 = the stored fp16 norm), rotated domain
//   ||r|| -> fp16;  z = S r;  bit j = (z_j >= 0), LSB first in a 16-byte row per token.
// Longer appends: S^T sits in LDS with a row pitch of 129 floats (66 KB), so both the
// transposing copy and the reads are free of bank conflicts: lane l reads row i at column l
// (and l + 64) while the residual coordinate r_i is a broadcast; lane l forms z_l and z_{l+64}
// and two ballots give the 128 bits.  Up to 8 tokens: the kernel below.
#include "tq_common.h"
#include "tq_launch.h"
#include "lanes.h"
#include "wave_quant.h"
#include "append_plane.h"

namespace tq {
namespace {

constexpr int kQjlTokens = 64;  // tokens per block (16 per wave)
constexpr int kPitch = kD + 1;   // LDS row pitch of S^T
constexpr float kInvSqrtD = 0.08838834764831845f;

template <int DTYPE, int BITS>
__global__ __launch_bounds__(256) void qjl_quantize_kernel(QjlQuantArgs a) {
  __shared__ float st[kD * kPitch];  // S^T: st[i * kPitch + j] = S[j][i]
  __shared__ __align__(16) float res[4][kD];
  __shared__ uint32_t words[4][4 * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  {  // S^T into LDS: the thread's 16 float4 loads all go out before the first store
    float4 f[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) f[k] = reinterpret_cast<const float4 *>(a.proj)[threadIdx.x + 256 * k];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int e = 4 * (threadIdx.x + 256 * k), j = e >> 7, i = e & (kD - 1);
      st[i * kPitch + j] = f[k].x;
      st[(i + 1) * kPitch + j] = f[k].y;
      st[(i + 2) * kPitch + j] = f[k].z;
      st[(i + 3) * kPitch + j] = f[k].w;
    }
  }
  __syncthreads();
  const CacheView &c = a.k;
  uint8_t *plane = c.plane(b, h);
  uint16_t *norms = c.norm_plane(b, h);
  const size_t unit = (size_t)b * c.n_kv_heads + h;
  uint8_t *bits = a.bits + unit * (size_t)c.capacity * (kD / 8);
  uint16_t *rnorms = a.res_norms + unit * (size_t)c.capacity;
  const int j_end = min(a.n_tokens, (int)(blockIdx.x + 1) * kQjlTokens);
  for (int j = blockIdx.x * kQjlTokens + wave; j < j_end; j += 4) {
    const int t = a.start_pos + j;
    float x0, x1, n, h0, h1;
    load_pair<DTYPE>(a.x, (((size_t)b * a.n_tokens + j) * c.n_kv_heads + h) * kD + 2 * lane, x0, x1);
    uint32_t c0, c1;
    token_codes<BITS>(c, x0, x1, lane, c0, c1, n, h0, h1);
    const uint16_t n16 = float_to_half_bits(n);
    const float nf = half_bits_to_float(n16);
    const float r0 = h0 * kInvSqrtD - nf * c.centroids[c0];
    const float r1 = h1 * kInvSqrtD - nf * c.centroids[c1];
    const float rn = sqrtf(wave_reduce<false>(r0 * r0 + r1 * r1));
    *reinterpret_cast<float2 *>(&res[wave][2 * lane]) = make_float2(r0, r1);
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
    float z_lo = 0.f, z_hi = 0.f;
#pragma unroll 8
    for (int i = 0; i < kD; ++i) {
      const float ri = res[wave][i];
      z_lo = fmaf(st[i * kPitch + lane], ri, z_lo);
      z_hi = fmaf(st[i * kPitch + lane + 64], ri, z_hi);
    }
    const uint64_t b_lo = __ballot(z_lo >= 0.f), b_hi = __ballot(z_hi >= 0.f);
    if (lane < 4) {
      const uint64_t w = lane < 2 ? b_lo : b_hi;
      reinterpret_cast<uint32_t *>(bits + (size_t)t * (kD / 8))[lane] = (uint32_t)(w >> (32 * (lane & 1)));
    }
    if (lane == 0) {
      norms[t] = n16;
      rnorms[t] = float_to_half_bits(rn);
    }
    store_row<BITS>(plane + (size_t)t * (16 * BITS), c0, c1, lane, words[wave]);
    // the residual buffer is read by every lane above before the next token overwrites it
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
  }
}

// A few tokens (a decode step): the sketch rows are shared out instead of S being staged.  Block
// (chunk, h, b) is one wave that handles rows j = 16 chunk .. 16 chunk + 15 of every token of the
// call; lane l holds S[16 chunk + l / 4][32 (l % 4) .. + 31] in registers, forms that quarter of
// (S r)_j against the residual (a broadcast from LDS) and the quad adds the quarters.  Every
// block quantizes the token itself (the same steps as above); chunk 0 stores the codes and both
// norms, each chunk its 16 sign bits.
constexpr int kQjlSmallMax = 8;   // tokens per call for this kernel
constexpr int kQjlChunks = kD / 16;

template <int DTYPE, int BITS>
__device__ void qjl_append_small_body(const QjlQuantArgs &a, int chunk, int h, int b, int lane, float *res,
                                      uint32_t *words) {
  const int q = lane & 3;
  float4 srow[8];
  const float4 *src = reinterpret_cast<const float4 *>(a.proj + (size_t)(16 * chunk + (lane >> 2)) * kD + 32 * q);
#pragma unroll
  for (int m = 0; m < 8; ++m) srow[m] = src[m];
  const CacheView &c = a.k;
  uint8_t *plane = c.plane(b, h);
  uint16_t *norms = c.norm_plane(b, h);
  const size_t unit = (size_t)b * c.n_kv_heads + h;
  uint8_t *bits = a.bits + unit * (size_t)c.capacity * (kD / 8);
  uint16_t *rnorms = a.res_norms + unit * (size_t)c.capacity;
  for (int j = 0; j < a.n_tokens; ++j) {
    const int t = a.start_pos + j;
    float x0, x1, n, h0, h1;
    load_pair<DTYPE>(a.x, (((size_t)b * a.n_tokens + j) * c.n_kv_heads + h) * kD + 2 * lane, x0, x1);
    uint32_t c0, c1;
    token_codes<BITS>(c, x0, x1, lane, c0, c1, n, h0, h1);
    const uint16_t n16 = float_to_half_bits(n);
    const float nf = half_bits_to_float(n16);
    const float r0 = h0 * kInvSqrtD - nf * c.centroids[c0];
    const float r1 = h1 * kInvSqrtD - nf * c.centroids[c1];
    *reinterpret_cast<float2 *>(&res[2 * lane]) = make_float2(r0, r1);
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
    float z = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float4 r4 = *reinterpret_cast<const float4 *>(&res[32 * q + 4 * m]);
      z = fmaf(srow[m].x, r4.x, z);
      z = fmaf(srow[m].y, r4.y, z);
      z = fmaf(srow[m].z, r4.z, z);
      z = fmaf(srow[m].w, r4.w, z);
    }
    z += dpp_mov<kDppQuadXor1>(z);
    z += dpp_mov<kDppQuadXor2>(z);
    const uint64_t ball = __ballot(z >= 0.f);
    uint32_t sb = 0u;  // bit i: row 16 chunk + i, read from lane 4 i
#pragma unroll
    for (int i = 0; i < 16; ++i) sb |= (uint32_t)((ball >> (4 * i)) & 1u) << i;
    if (lane == 0) reinterpret_cast<uint16_t *>(bits + (size_t)t * (kD / 8))[chunk] = (uint16_t)sb;
    if (chunk == 0) {
      const float rn = sqrtf(wave_reduce<false>(r0 * r0 + r1 * r1));
      if (lane == 0) {
        norms[t] = n16;
        rnorms[t] = float_to_half_bits(rn);
      }
      store_row<BITS>(plane + (size_t)t * (16 * BITS), c0, c1, lane, words);
    }
    // every lane has read the residual before the next token overwrites it
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
  }
}

template <int DTYPE, int BITS>
__global__ __launch_bounds__(64) void qjl_append_small_kernel(QjlQuantArgs a) {
  __shared__ __align__(16) float res[kD];
  __shared__ uint32_t words[4 * 8];
  qjl_append_small_body<DTYPE, BITS>(a, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x, res, words);
}

// Keys (with their sketch) and values of up to 8 tokens in one launch: blocks x < kQjlChunks of
// (x, h, b) are the key blocks above (their first wave; the block has one wave per token for the
// value blocks' sake), block x = kQjlChunks appends the tokens' values to plane (b, h) as the
// small-append kernel does (one wave per token, then one update per 8-token value group).
template <int DTYPE, int BK, int BV>
__global__ __launch_bounds__(64 * kSmallAppendMax) void qjl_append_kv_small_kernel(QjlQuantArgs a, CacheView vc,
                                                                                  const void *__restrict__ xv) {
  __shared__ __align__(16) float res[kD];
  __shared__ uint32_t words[4 * 8];
  __shared__ SmallLds sh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if ((int)blockIdx.x < kQjlChunks) {
    if (wave == 0) qjl_append_small_body<DTYPE, BK>(a, blockIdx.x, blockIdx.y, blockIdx.z, lane, res, words);
    return;  // (no block-wide barrier on this path)
  }
  append_plane<DTYPE, BV, false>(vc, xv, blockIdx.z, blockIdx.y, a.start_pos, a.n_tokens, wave, lane, sh);
}

template <int DTYPE, int BK>
void launch_kv_small_bv(const QjlQuantArgs &a, const CacheView &vc, const void *xv, dim3 grid, hipStream_t stream) {
  const int threads = 64 * a.n_tokens;
  switch (vc.bits) {
    case 2: qjl_append_kv_small_kernel<DTYPE, BK, 2><<<grid, threads, 0, stream>>>(a, vc, xv); break;
    case 3: qjl_append_kv_small_kernel<DTYPE, BK, 3><<<grid, threads, 0, stream>>>(a, vc, xv); break;
    case 4: qjl_append_kv_small_kernel<DTYPE, BK, 4><<<grid, threads, 0, stream>>>(a, vc, xv); break;
    default: qjl_append_kv_small_kernel<DTYPE, BK, 8><<<grid, threads, 0, stream>>>(a, vc, xv); break;
  }
}

template <int DTYPE>
void launch_kv_small(const QjlQuantArgs &a, const CacheView &vc, const void *xv, dim3 grid, hipStream_t stream) {
  switch (a.k.bits) {
    case 2: launch_kv_small_bv<DTYPE, 2>(a, vc, xv, grid, stream); break;
    case 3: launch_kv_small_bv<DTYPE, 3>(a, vc, xv, grid, stream); break;
    case 4: launch_kv_small_bv<DTYPE, 4>(a, vc, xv, grid, stream); break;
    default: launch_kv_small_bv<DTYPE, 8>(a, vc, xv, grid, stream); break;
  }
}

template <int DTYPE>
hipError_t launch_dtype(const QjlQuantArgs &a, dim3 grid, hipStream_t stream) {
  if (a.n_tokens <= kQjlSmallMax) {
    const dim3 g2(kQjlChunks, grid.y, grid.z);
    switch (a.k.bits) {
      case 2: qjl_append_small_kernel<DTYPE, 2><<<g2, 64, 0, stream>>>(a); break;
      case 3: qjl_append_small_kernel<DTYPE, 3><<<g2, 64, 0, stream>>>(a); break;
      case 4: qjl_append_small_kernel<DTYPE, 4><<<g2, 64, 0, stream>>>(a); break;
      default: qjl_append_small_kernel<DTYPE, 8><<<g2, 64, 0, stream>>>(a); break;
    }
    return hipGetLastError();
  }
  switch (a.k.bits) {
    case 2: qjl_quantize_kernel<DTYPE, 2><<<grid, 256, 0, stream>>>(a); break;
    case 3: qjl_quantize_kernel<DTYPE, 3><<<grid, 256, 0, stream>>>(a); break;
    case 4: qjl_quantize_kernel<DTYPE, 4><<<grid, 256, 0, stream>>>(a); break;
    default: qjl_quantize_kernel<DTYPE, 8><<<grid, 256, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qjl_quantize_kv_small(const QjlQuantArgs &a, const CacheView &vc, const void *xv, int batch,
                                       hipStream_t stream) {
  if (a.n_tokens < 1 || a.n_tokens > kQjlSmallMax || a.n_tokens > kSmallAppendMax || a.k.layout != TQ_LAYOUT_ROWS ||
      vc.layout != TQ_LAYOUT_GROUP8 || batch < 1 || batch > 65535 || a.k.n_kv_heads > 65535)
    return hipErrorInvalidValue;
  const dim3 grid(kQjlChunks + 1, a.k.n_kv_heads, batch);
  if (a.x_dtype == TQ_F32) launch_kv_small<TQ_F32>(a, vc, xv, grid, stream);
  else if (a.x_dtype == TQ_BF16) launch_kv_small<TQ_BF16>(a, vc, xv, grid, stream);
  else launch_kv_small<TQ_F16>(a, vc, xv, grid, stream);
  return hipGetLastError();
}

hipError_t launch_qjl_quantize(const QjlQuantArgs &a, int batch, hipStream_t stream) {
  if (a.n_tokens < 1 || a.k.layout != TQ_LAYOUT_ROWS) return hipErrorInvalidValue;
  const dim3 grid((a.n_tokens + kQjlTokens - 1) / kQjlTokens, a.k.n_kv_heads, batch);
  if (a.x_dtype == TQ_F32) return launch_dtype<TQ_F32>(a, grid, stream);
  if (a.x_dtype == TQ_BF16) return launch_dtype<TQ_BF16>(a, grid, stream);
  return launch_dtype<TQ_F16>(a, grid, stream);
}

}  // namespace tq
