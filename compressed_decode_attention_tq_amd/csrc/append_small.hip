// Appending a few tokens to a key cache (row layout) and a value cache (8-token value
// groups): decode steps and short drafts.  The chunked quantize kernel builds code-search
// tables in LDS before its first token, a fixed chain of loads and barriers that dominates
// when only one token per (batch, kv head) arrives.  Here one block owns one (batch, kv head,
// key or value) plane and one wave of 64 lanes one token, two coordinates per lane, with the
// transform and the reductions in registers (lanes.h).
//
// Steps per token, as in the chunked kernel ([tq-80] §核心创新: norm split off, random
// rotation, data-independent Lloyd-Max code; [inferrs] §核心技术: Walsh-Hadamard rotation):
//   n = ||x||_2 in fp32, stored as fp16 (round to nearest even);
//   u = H (s . x) / (sqrt(d) n);  code_i = #{j : t_j < u_i};
//   the codes go to their bit positions in the cache's layout (tq.h).
#include "tq_common.h"
#include "tq_launch.h"
#include "lanes.h"
#include "wave_quant.h"
#include "append_plane.h"

namespace tq {
namespace {

// block z = z0 + blockIdx.x < batch * Hkv: key plane (b, h) = (z / Hkv, z % Hkv); the rest:
// value planes (z0 = batch * Hkv and kc = vc appends to one value cache alone).  One wave per
// token: blockDim = 64 n_tokens.
template <int DTYPE, int BK, int BV>
__global__ __launch_bounds__(64 * kSmallAppendMax) void append_small_kernel(CacheView kc, CacheView vc,
                                                                           const void *__restrict__ xk,
                                                                           const void *__restrict__ xv,
                                                                           int start_pos, int n_tokens, int batch,
                                                                           int z0) {
  __shared__ SmallLds sh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int planes = batch * kc.n_kv_heads;
  const int z = z0 + (int)blockIdx.x;
  if (z < planes)
    append_plane<DTYPE, BK, true>(kc, xk, z / kc.n_kv_heads, z % kc.n_kv_heads, start_pos, n_tokens, wave, lane, sh);
  else
    append_plane<DTYPE, BV, false>(vc, xv, (z - planes) / vc.n_kv_heads, (z - planes) % vc.n_kv_heads, start_pos,
                                   n_tokens, wave, lane, sh);
}

// Paged caches (kc, vc view the pools: plane(page, h) is one page of one kv head, capacity =
// page_tokens): block (x, y) takes the aligned 8-token window x of plane y's sequence,
// starting at the window that holds start_pos[b]; wave j takes the window's token j.  A
// window lies inside one page (pages are multiples of 64 tokens), so a value group is
// updated by exactly one block.
template <int DTYPE, int BITS, bool KEY>
__device__ void append_window(const CacheView &c, const void *x, const int32_t *table, int max_pages, int n_pages,
                              int b, int h, int s0, int n_tokens, int wave, int lane, SmallLds &sh) {
  const int P = c.capacity;
  const int w0 = ((s0 >> 3) + (int)blockIdx.x) * 8;  // s0 >> 3 rounds down, also below zero
  if (w0 + 8 <= s0 || w0 >= s0 + n_tokens || w0 < 0 || w0 >= max_pages * P) return;  // uniform
  const int slot = w0 / P;
  const int page = table[(size_t)b * max_pages + slot];
  if (page < 0 || page >= n_pages) return;  // no page: nothing is written
  uint8_t *plane = c.plane(page, h);
  const int t = w0 + wave, j = t - s0;
  const int pos = t - slot * P;  // slot of the token inside its page
  if (j >= 0 && j < n_tokens) {
    float x0, x1;
    load_pair<DTYPE>(x, (((size_t)b * n_tokens + j) * c.n_kv_heads + h) * kD + 2 * lane, x0, x1);
    uint32_t c0, c1;
    float n;
    float h0, h1;
    token_codes<BITS>(c, x0, x1, lane, c0, c1, n, h0, h1);
    if (lane == 0) c.norm_plane(page, h)[pos] = float_to_half_bits(n);
    if constexpr (KEY) store_row<BITS>(plane + (size_t)pos * (16 * BITS), c0, c1, lane, sh.words[wave]);
    else sh.codes[wave][lane] = make_uint2(c0, c1);
  }
  if constexpr (!KEY) {
    __syncthreads();
    if (wave == 0) {
      uint8_t *group = plane + (size_t)((w0 - slot * P) >> 3) * (kD * BITS);
      GroupSlice<BITS> slice;
      slice.load(group, lane);
      for (int p = 0; p < 8; ++p) {
        const int jj = w0 + p - s0;
        if (jj < 0 || jj >= n_tokens) continue;
        const uint2 cc = sh.codes[p][lane];
        slice.set(p * BITS, cc.x);
        slice.set((8 + p) * BITS, cc.y);
      }
      slice.store(group, lane);
    }
  }
}

template <int DTYPE, int BK, int BV>
__global__ __launch_bounds__(64 * kSmallAppendMax) void append_paged_kernel(
    CacheView kc, CacheView vc, const int32_t *__restrict__ table, int max_pages, int n_pages,
    const void *__restrict__ xk, const void *__restrict__ xv, const int32_t *__restrict__ start_pos, int n_tokens,
    int batch) {
  __shared__ SmallLds sh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int planes = batch * kc.n_kv_heads;
  const int z = blockIdx.y;
  const bool key = z < planes;
  const int zz = key ? z : z - planes, b = zz / kc.n_kv_heads, h = zz % kc.n_kv_heads;
  const int s0 = __builtin_amdgcn_readfirstlane(start_pos[b]);
  if (key) append_window<DTYPE, BK, true>(kc, xk, table, max_pages, n_pages, b, h, s0, n_tokens, wave, lane, sh);
  else append_window<DTYPE, BV, false>(vc, xv, table, max_pages, n_pages, b, h, s0, n_tokens, wave, lane, sh);
}

struct PagedLaunch {
  const int32_t *table;
  int max_pages, n_pages;
  const int32_t *start_pos;
};

template <int DTYPE, int BK, int BV>
void launch_paged3(const CacheView &kc, const CacheView &vc, const PagedLaunch &pl, dim3 grid, const void *xk,
                   const void *xv, int n_tokens, int batch, hipStream_t stream) {
  append_paged_kernel<DTYPE, BK, BV><<<grid, 64 * kSmallAppendMax, 0, stream>>>(
      kc, vc, pl.table, pl.max_pages, pl.n_pages, xk, xv, pl.start_pos, n_tokens, batch);
}

template <int DTYPE, int BK>
void launch_paged2(const CacheView &kc, const CacheView &vc, const PagedLaunch &pl, dim3 grid, const void *xk,
                   const void *xv, int n_tokens, int batch, hipStream_t stream) {
  switch (vc.bits) {
    case 2: launch_paged3<DTYPE, BK, 2>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream); break;
    case 3: launch_paged3<DTYPE, BK, 3>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream); break;
    case 4: launch_paged3<DTYPE, BK, 4>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream); break;
    default: launch_paged3<DTYPE, BK, 8>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream); break;
  }
}

template <int DTYPE>
void launch_paged1(const CacheView &kc, const CacheView &vc, const PagedLaunch &pl, dim3 grid, const void *xk,
                   const void *xv, int n_tokens, int batch, hipStream_t stream) {
  switch (kc.bits) {
    case 2: launch_paged2<DTYPE, 2>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream); break;
    case 3: launch_paged2<DTYPE, 3>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream); break;
    case 4: launch_paged2<DTYPE, 4>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream); break;
    default: launch_paged2<DTYPE, 8>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream); break;
  }
}

template <int DTYPE, int BK>
hipError_t launch_bv(const CacheView &kc, const CacheView &vc, int grid, const void *xk, const void *xv,
                     int start_pos, int n_tokens, int batch, int z0, hipStream_t stream) {
  switch (vc.bits) {
    case 2: append_small_kernel<DTYPE, BK, 2><<<grid, 64 * n_tokens, 0, stream>>>(kc, vc, xk, xv, start_pos, n_tokens, batch, z0); break;
    case 3: append_small_kernel<DTYPE, BK, 3><<<grid, 64 * n_tokens, 0, stream>>>(kc, vc, xk, xv, start_pos, n_tokens, batch, z0); break;
    case 4: append_small_kernel<DTYPE, BK, 4><<<grid, 64 * n_tokens, 0, stream>>>(kc, vc, xk, xv, start_pos, n_tokens, batch, z0); break;
    default: append_small_kernel<DTYPE, BK, 8><<<grid, 64 * n_tokens, 0, stream>>>(kc, vc, xk, xv, start_pos, n_tokens, batch, z0); break;
  }
  return hipGetLastError();
}

template <int DTYPE>
hipError_t launch_bk(const CacheView &kc, const CacheView &vc, int grid, const void *xk, const void *xv,
                     int start_pos, int n_tokens, int batch, int z0, hipStream_t stream) {
  switch (kc.bits) {
    case 2: return launch_bv<DTYPE, 2>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, z0, stream);
    case 3: return launch_bv<DTYPE, 3>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, z0, stream);
    case 4: return launch_bv<DTYPE, 4>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, z0, stream);
    default: return launch_bv<DTYPE, 8>(kc, vc, grid, xk, xv, start_pos, n_tokens, batch, z0, stream);
  }
}

}  // namespace

hipError_t launch_append_paged(const CacheView &kc, const CacheView &vc, const int32_t *block_table,
                               int max_pages, int n_pages, int batch, const void *xk, const void *xv,
                               int x_dtype, const int32_t *start_pos, int n_tokens, hipStream_t stream) {
  if (n_tokens < 1 || kc.capacity % 8 != 0 || kc.layout != TQ_LAYOUT_ROWS || vc.layout != TQ_LAYOUT_GROUP8)
    return hipErrorInvalidValue;
  const long windows = (long)(n_tokens + 7) / 8 + 1, planes = 2L * batch * kc.n_kv_heads;
  if (windows > 0x7fffffffL || planes < 1 || planes > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)windows, (unsigned)planes);
  const PagedLaunch pl{block_table, max_pages, n_pages, start_pos};
  if (x_dtype == TQ_F32) launch_paged1<TQ_F32>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream);
  else if (x_dtype == TQ_BF16) launch_paged1<TQ_BF16>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream);
  else launch_paged1<TQ_F16>(kc, vc, pl, grid, xk, xv, n_tokens, batch, stream);
  return hipGetLastError();
}

hipError_t launch_append_small(const CacheView &kc, const CacheView &vc, int batch, const void *xk,
                               const void *xv, int x_dtype, int start_pos, int n_tokens, hipStream_t stream) {
  if (n_tokens < 1 || n_tokens > kSmallAppendMax || kc.layout != TQ_LAYOUT_ROWS || vc.layout != TQ_LAYOUT_GROUP8)
    return hipErrorInvalidValue;
  const long grid = 2L * batch * kc.n_kv_heads;
  if (grid < 1 || grid > 0x7fffffffL) return hipErrorInvalidValue;
  if (x_dtype == TQ_F32) return launch_bk<TQ_F32>(kc, vc, (int)grid, xk, xv, start_pos, n_tokens, batch, 0, stream);
  if (x_dtype == TQ_BF16) return launch_bk<TQ_BF16>(kc, vc, (int)grid, xk, xv, start_pos, n_tokens, batch, 0, stream);
  return launch_bk<TQ_F16>(kc, vc, (int)grid, xk, xv, start_pos, n_tokens, batch, 0, stream);
}

hipError_t launch_append_small_one(const CacheView &c, int batch, const void *x, int x_dtype, int start_pos,
                                   int n_tokens, hipStream_t stream) {
  if (n_tokens < 1 || n_tokens > kSmallAppendMax) return hipErrorInvalidValue;
  const long planes = (long)batch * c.n_kv_heads;
  if (planes < 1 || planes > 0x3fffffffL) return hipErrorInvalidValue;
  // the key path for a row cache (blocks 0 .. planes - 1), the value path for a group cache
  const int z0 = c.layout == TQ_LAYOUT_ROWS ? 0 : (int)planes;
  if (x_dtype == TQ_F32) return launch_bk<TQ_F32>(c, c, (int)planes, x, x, start_pos, n_tokens, batch, z0, stream);
  if (x_dtype == TQ_BF16) return launch_bk<TQ_BF16>(c, c, (int)planes, x, x, start_pos, n_tokens, batch, z0, stream);
  return launch_bk<TQ_F16>(c, c, (int)planes, x, x, start_pos, n_tokens, batch, z0, stream);
}

}  // namespace tq
