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

// Value of the same register in lane (lane ^ m) of the quad, m = 1 (quad_perm 1,0,3,2:
// control 0xB1) or m = 2 (quad_perm 2,3,0,1: control 0x4E), through a DPP move.
template <int CTRL>
__device__ __forceinline__ float quad_swap(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Walsh-Hadamard transform (unnormalised) of 128 values held 32 per lane by a lane quad (lane
// q of the quad holds coordinates 32q .. 32q+31): five butterfly stages inside the lane,
// then two across the quad as v += s * partner (s = +1 for the lower lane of a pair, -1 for
// the upper), one DPP multiply-add each.  The upper lane thereby holds own - partner, the
// negative of its butterfly output, so the lane ends with (-1)^popcount(q) times the
// transform: quad_fwht_sign(q) gives that factor, which the caller folds into its scale.
// FIRST = 2 skips the in-lane stage of distance 1, for a caller that has done it already
// (the stages commute).
template <int FIRST = 1>
__device__ __forceinline__ void quad_fwht(float v[32], int q) {
#pragma unroll
  for (int h = FIRST; h < 32; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      if ((e & h) == 0) {
        float a = v[e], c = v[e + h];
        v[e] = a + c;
        v[e + h] = a - c;
      }
    }
  }
  // v += s * partner as v_fmac_f32_dpp (the compiler does not fold the DPP move into a
  // multiply-accumulate).  A DPP read needs two wait states after a vector write of its
  // source: the s_nop covers the instructions before each block, and inside a block no
  // instruction reads a register the two before it wrote.
  {
    const float s = (q & 1) ? -1.f : 1.f;
    asm volatile(
      "s_nop 1\n"
      "v_fmac_f32_dpp %0, %0, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %1, %1, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %2, %2, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %3, %3, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %4, %4, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %5, %5, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %6, %6, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %7, %7, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %8, %8, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %9, %9, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %10, %10, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %11, %11, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %12, %12, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %13, %13, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %14, %14, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %15, %15, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      : "+v"(v[0+0]), "+v"(v[0+1]), "+v"(v[0+2]), "+v"(v[0+3]), "+v"(v[0+4]), "+v"(v[0+5]), "+v"(v[0+6]), "+v"(v[0+7]), "+v"(v[0+8]), "+v"(v[0+9]), "+v"(v[0+10]), "+v"(v[0+11]), "+v"(v[0+12]), "+v"(v[0+13]), "+v"(v[0+14]), "+v"(v[0+15])
      : "v"(s));
    asm volatile(
      "s_nop 1\n"
      "v_fmac_f32_dpp %0, %0, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %1, %1, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %2, %2, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %3, %3, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %4, %4, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %5, %5, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %6, %6, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %7, %7, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %8, %8, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %9, %9, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %10, %10, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %11, %11, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %12, %12, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %13, %13, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %14, %14, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %15, %15, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      : "+v"(v[16+0]), "+v"(v[16+1]), "+v"(v[16+2]), "+v"(v[16+3]), "+v"(v[16+4]), "+v"(v[16+5]), "+v"(v[16+6]), "+v"(v[16+7]), "+v"(v[16+8]), "+v"(v[16+9]), "+v"(v[16+10]), "+v"(v[16+11]), "+v"(v[16+12]), "+v"(v[16+13]), "+v"(v[16+14]), "+v"(v[16+15])
      : "v"(s));
  }
  {
    const float s = (q & 2) ? -1.f : 1.f;
    asm volatile(
      "s_nop 1\n"
      "v_fmac_f32_dpp %0, %0, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %1, %1, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %2, %2, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %3, %3, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %4, %4, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %5, %5, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %6, %6, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %7, %7, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %8, %8, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %9, %9, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %10, %10, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %11, %11, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %12, %12, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %13, %13, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %14, %14, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %15, %15, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      : "+v"(v[0+0]), "+v"(v[0+1]), "+v"(v[0+2]), "+v"(v[0+3]), "+v"(v[0+4]), "+v"(v[0+5]), "+v"(v[0+6]), "+v"(v[0+7]), "+v"(v[0+8]), "+v"(v[0+9]), "+v"(v[0+10]), "+v"(v[0+11]), "+v"(v[0+12]), "+v"(v[0+13]), "+v"(v[0+14]), "+v"(v[0+15])
      : "v"(s));
    asm volatile(
      "s_nop 1\n"
      "v_fmac_f32_dpp %0, %0, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %1, %1, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %2, %2, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %3, %3, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %4, %4, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %5, %5, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %6, %6, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %7, %7, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %8, %8, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %9, %9, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %10, %10, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %11, %11, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %12, %12, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %13, %13, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %14, %14, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_fmac_f32_dpp %15, %15, %16 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      : "+v"(v[16+0]), "+v"(v[16+1]), "+v"(v[16+2]), "+v"(v[16+3]), "+v"(v[16+4]), "+v"(v[16+5]), "+v"(v[16+6]), "+v"(v[16+7]), "+v"(v[16+8]), "+v"(v[16+9]), "+v"(v[16+10]), "+v"(v[16+11]), "+v"(v[16+12]), "+v"(v[16+13]), "+v"(v[16+14]), "+v"(v[16+15])
      : "v"(s));
  }
}

__device__ __forceinline__ float quad_fwht_sign(int q) { return ((q ^ (q >> 1)) & 1) ? -1.f : 1.f; }

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

constexpr int kGridCells = 128;

struct QuantLds {
  __attribute__((aligned(16))) uint8_t stage[4][16][kD];  // value-group transpose
  float bnd8[256];                                         // 256-level boundaries
  uint2 grid[4][kGridCells];                               // per-wave code grid (<= 16 levels)
  uint2 grid8[1024];                                       // block code grid (256 levels)
  float red[4];
  int flag;
};

// Code search by a uniform grid over u in [-1.01, 1.01) (codebooks of up to 16 levels).  In
// cell coordinates f = (u + 1.01) / w, cell c = trunc(f) holds at most one boundary; its
// entry is {#{t_j < lower edge of c}, f of that boundary (+inf if none)}, so
// code = entry.x + (f > entry.y): one multiply-add, one conversion, one lookup, one compare.
// A unit vector's coordinates satisfy |u| <= 1 (the fp32 norm makes it 1 + 1e-5 at most), so
// f stays inside the table without a clamp; a NaN converts to cell 0.  A u that rounds into
// a neighbouring cell, or a comparison rounded in cell coordinates, can only change a code
// within the rounding of u (far below 1e-6) of a boundary.
struct CodeGrid {
  float scale, offset;  // f = u * scale + offset
  bool ok;
};

// Builds the wave's grid from the L/2 - 1 positive boundaries (the codebook is symmetric:
// t = -pos reversed, 0, pos).  ok is false when the grid would need more than kGridCells
// cells or a cell would hold two boundaries; the caller then counts compares instead.
template <int BITS>
__device__ CodeGrid build_code_grid(const float *pos, uint2 *grid, int lane) {
  constexpr int L = 1 << BITS, NP = L / 2 - 1;
  constexpr float kLo = -1.01f, kHi = 1.01f;
  float gap = pos[0];
#pragma unroll
  for (int k = 0; k + 1 < NP; ++k) gap = fminf(gap, pos[k + 1] - pos[k]);
  const float w = 0.75f * gap;
  CodeGrid gd;
  gd.scale = 1.f / w;
  gd.offset = -kLo / w;
  gd.ok = gap > 0.f && pos[NP - 1] < kHi && (kHi - kLo) / w <= (float)kGridCells;
  if (!gd.ok) return gd;
  bool bad = false;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int cidx = lane + 64 * half;
    const float e0 = kLo + (float)cidx * w;  // lower edge
    const float e1 = e0 + w;                 // upper edge
    uint32_t base = 0, inside = 0;
    float bnd = INFINITY;
    auto visit = [&](float t) {
      base += t < e0 ? 1u : 0u;
      const bool in = t >= e0 && t < e1;
      inside += in ? 1u : 0u;
      if (in) bnd = fminf(bnd, (t - kLo) * gd.scale);
    };
#pragma unroll
    for (int k = NP - 1; k >= 0; --k) visit(-pos[k]);
    visit(0.f);
#pragma unroll
    for (int k = 0; k < NP; ++k) visit(pos[k]);
    bad |= inside > 1u;
    grid[cidx] = make_uint2(base, __float_as_uint(bnd));
  }
  gd.ok = __ballot(bad) == 0ull;
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
  return gd;
}

// code of coordinate v of a vector whose u = v * inv; sinv = inv * gd.scale
__device__ __forceinline__ uint32_t code_by_grid(float v, float sinv, const CodeGrid &gd, const uint2 *grid) {
  const float f = fmaf(v, sinv, gd.offset);
  const uint2 e = grid[(int)f];
  return e.x + (f > __uint_as_float(e.y) ? 1u : 0u);
}

// The grid for 256-level codebooks, shared by the block and built by all its threads (the
// caller synchronises before and after): cells of 0.75 x the smallest boundary gap over
// [t_0 - w/2, t_254 + w/2), at most 1024 of them; cell 0 reaches down to -inf and the last
// cell up to +inf, so lookups clamp the cell index.  Entry and check as for the wave grid;
// the boundaries are copied to sh.bnd8 for the entries' binary searches and the fallback.
struct CodeGrid8 {
  float scale, offset, last_cell;
  bool ok;
};

__device__ CodeGrid8 build_code_grid8(const float *boundaries, QuantLds &sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float gmin = INFINITY;
  if (tid < 255) sh.bnd8[tid] = boundaries[tid];
  __syncthreads();
  if (tid < 254) gmin = sh.bnd8[tid + 1] - sh.bnd8[tid];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) gmin = fminf(gmin, __shfl_xor(gmin, m));
  if (lane == 0) sh.red[wave] = gmin;
  if (tid == 0) sh.flag = 0;
  __syncthreads();
  gmin = fminf(fminf(sh.red[0], sh.red[1]), fminf(sh.red[2], sh.red[3]));
  const float w = 0.75f * gmin;
  const float lo = sh.bnd8[0] - 0.5f * w;
  CodeGrid8 gd;
  const float span = (sh.bnd8[254] + 0.5f * w - lo) / w;
  gd.ok = gmin > 0.f && span < 1023.f;
  if (!gd.ok) return gd;  // uniform: every thread sees the same values
  const int cells = (int)ceilf(span) + 1;
  gd.scale = 1.f / w;
  gd.offset = -lo / w;
  gd.last_cell = (float)(cells - 1);
  bool bad = false;
  for (int cidx = tid; cidx < cells; cidx += blockDim.x) {
    const float e0 = lo + (float)cidx * w, e1 = e0 + w;
    // base = #{t < e0} (0 for the first cell, which reaches down to -inf)
    uint32_t base = 0;
    if (cidx > 0) {
#pragma unroll
      for (int step = 128; step >= 1; step >>= 1)
        if (base + step - 1 < 255 && sh.bnd8[base + step - 1] < e0) base += step;
    }
    const bool last = cidx == cells - 1;
    float bnd = INFINITY;
    if (base < 255 && (last || sh.bnd8[base] < e1)) {
      bnd = (sh.bnd8[base] - lo) * gd.scale;
      if (base + 1 < 255 && (last || sh.bnd8[base + 1] < e1)) bad = true;
    }
    sh.grid8[cidx] = make_uint2(base, __float_as_uint(bnd));
  }
  if (bad) sh.flag = 1;
  __syncthreads();
  gd.ok = sh.flag == 0;
  return gd;
}

__device__ __forceinline__ uint32_t code_by_grid8(float v, float sinv, const CodeGrid8 &gd, const uint2 *grid) {
  const float f = fmaf(v, sinv, gd.offset);
  const uint2 e = grid[(int)__builtin_amdgcn_fmed3f(f, 0.f, gd.last_cell)];
  return e.x + (f > __uint_as_float(e.y) ? 1u : 0u);
}

// Packs the 32 codes of coordinates 32q .. 32q+31 of token t into bits
// [32*BITS*q, 32*BITS*(q+1)) of the token's row.
template <int BITS>
__device__ __forceinline__ void store_row_quarter(uint8_t *plane, int t, int q, const uint32_t (&code)[32]) {
  uint32_t w[BITS];
#pragma unroll
  for (int k = 0; k < BITS; ++k) w[k] = 0u;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int bit = e * BITS;
    w[bit >> 5] |= code[e] << (bit & 31);
    if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= code[e] >> (32 - (bit & 31));
  }
  uint32_t *dst = reinterpret_cast<uint32_t *>(plane + (size_t)t * 16 * BITS + 4 * BITS * q);
#pragma unroll
  for (int k = 0; k < BITS; ++k) dst[k] = w[k];
}

// Value groups from the wave's staged codes stage[16 tokens][128] (bytes): lane r of a
// group builds coordinates 4r .. 4r+3 of its group, 8 tokens x BITS bits per coordinate,
// BITS bytes each; bytes of tokens outside [lo, hi) are read-modified-written.
template <int BITS>
__device__ __forceinline__ void store_groups_from_stage(const uint8_t (*stage)[kD], uint8_t *plane, int lane,
                                                        int wt0, int lo, int hi) {
  constexpr int L = 1 << BITS;
  const int gi = lane >> 5, r = lane & 31;
  const int tg = wt0 + 8 * gi;  // first token of the group
  uint64_t chunk[4] = {0, 0, 0, 0}, mask = 0;
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const uint32_t cw = *reinterpret_cast<const uint32_t *>(&stage[8 * gi + tt][4 * r]);
    const bool in = tg + tt >= lo && tg + tt < hi;
    if (in) mask |= (uint64_t)(L - 1) << (tt * BITS);
#pragma unroll
    for (int k = 0; k < 4; ++k) chunk[k] |= (uint64_t)((cw >> (8 * k)) & 0xffu) << (tt * BITS);
  }
  if (mask == 0) return;
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

// Code search set-up shared by both paths: the positive boundaries and the code grid
// (codebooks of up to 16 levels), or the 255 boundaries in LDS (256 levels).
template <int BITS>
__device__ __forceinline__ CodeGrid setup_code_search(const CacheView &c, QuantLds &sh, int wave, int lane,
                                                      float (&pos)[(1 << BITS) / 2 > 1 ? (1 << BITS) / 2 - 1 : 1]) {
  constexpr int L = 1 << BITS;
  CodeGrid gd{0.f, 0.f, false};
  if (BITS <= 4) {
#pragma unroll
    for (int k = 0; k < L / 2 - 1; ++k) pos[k] = c.boundaries[L / 2 + k];
    gd = build_code_grid<BITS <= 4 ? BITS : 4>(pos, sh.grid[wave], lane);
  }
  return gd;
}

// Code without the grid: compare count (up to 16 levels) or binary search (256 levels).
template <int BITS>
__device__ __forceinline__ uint32_t code_by_search(float u, const QuantLds &sh, int wave, const float *pos) {
  return BITS <= 4 ? code_of<BITS <= 4 ? BITS : 4>(u, pos) : code_of_8(u, sh.bnd8);
}

constexpr int kChunksPerBlock = 4;  // chunks one block quantizes, reusing the set-up

// Loads the lane's 32 coordinates with the rotation signs applied: the sign masks m (0 or the
// sign bit) are folded into the conversion, (w << 16) + m and (w & 0xffff0000) ^ m for bf16.
// 32 fp32 coordinates with the sign bits of s applied (XOR masks m).
__device__ __forceinline__ void load32_f32_signed(const float *x, const uint32_t (&m)[32], float v[32]) {
  const uint4 *p = reinterpret_cast<const uint4 *>(x);
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint4 f = p[r];
    v[4 * r] = __uint_as_float(f.x ^ m[4 * r]);
    v[4 * r + 1] = __uint_as_float(f.y ^ m[4 * r + 1]);
    v[4 * r + 2] = __uint_as_float(f.z ^ m[4 * r + 2]);
    v[4 * r + 3] = __uint_as_float(f.w ^ m[4 * r + 3]);
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + c for two 16-bit values per word (bf16 or fp16), fp32 result:
// the products are exact, so with b = {+-1, +-1} this is a signed sum of two inputs rounded
// once, and with b = a a sum of squares.
template <int DTYPE>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (DTYPE == TQ_BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}
// The same with c = 0, as the three-operand instruction with an inline zero: the builtin
// above becomes the accumulating two-operand form plus a move of 0 for every call.
template <int DTYPE>
__device__ __forceinline__ float dot2_0(uint32_t a, uint32_t b) {
  float r;
  if constexpr (DTYPE == TQ_BF16) asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  else asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Up to kChunksPerBlock 64-token chunks (block bx takes chunks kChunksPerBlock * bx .. counted
// from the chunk of start_pos) of the plane of (batch b, kv head h).  Each wave owns 16
// tokens of every chunk; the code search set-up and the sign masks are made once.
template <int DTYPE, int BITS, int LAYOUT>
__device__ __forceinline__ void quantize_chunk(const CacheView &c, const void *__restrict__ x,
                                               int start_pos, int n_tokens, int h, int b, int bx,
                                               QuantLds &sh) {
  constexpr int L = 1 << BITS;
  const int first = start_pos / kChunk + bx * kChunksPerBlock;
  const int last = min(first + kChunksPerBlock - 1, (start_pos + n_tokens - 1) / kChunk);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  CodeGrid8 gd8{0.f, 0.f, 0.f, false};
  if (BITS == 8) gd8 = build_code_grid8(c.boundaries, sh);  // whole block, before any wave leaves
  // tokens of this wave: [first*64 + 16 wave, +16), ... ; none in range -> done
  {
    bool any = false;
    for (int ch = first; ch <= last; ++ch) {
      const int wt0 = ch * kChunk + 16 * wave;
      any |= wt0 + 16 > start_pos && wt0 < start_pos + n_tokens;
    }
    if (!any) return;
  }
  const int j = lane >> 2, q = lane & 3;

  float pos[L / 2 > 1 ? L / 2 - 1 : 1];
  const CodeGrid gd = setup_code_search<BITS>(c, sh, wave, lane, pos);
  // Signs s_(32q + e) of this lane's coordinates.  fp32 input: sign-bit XOR masks.  16-bit
  // input: the load does the first butterfly stage as two dot products of each input word
  // (coordinates 2e, 2e+1) with the +-1 pairs {s_2e, s_2e+1} and {s_2e, -s_2e+1} written in
  // the input's format.
  uint32_t smask[32], spair[16], sdiff[16];
  {
    const int4 sw0 = *reinterpret_cast<const int4 *>(c.signs + 32 * q);
    const int4 sw1 = *reinterpret_cast<const int4 *>(c.signs + 32 * q + 16);
    const uint32_t sw[8] = {(uint32_t)sw0.x, (uint32_t)sw0.y, (uint32_t)sw0.z, (uint32_t)sw0.w,
                            (uint32_t)sw1.x, (uint32_t)sw1.y, (uint32_t)sw1.z, (uint32_t)sw1.w};
#pragma unroll
    for (int e = 0; e < 32; ++e) smask[e] = (sw[e >> 2] << (24 - 8 * (e & 3))) & 0x80000000u;
    const uint32_t one = DTYPE == TQ_BF16 ? 0x3F80u : 0x3C00u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      spair[e] = (one | (smask[2 * e] >> 16)) | ((one << 16) | smask[2 * e + 1]);
      sdiff[e] = spair[e] ^ 0x80000000u;
    }
  }
  uint8_t *plane = c.plane(b, h);

  for (int ch = first; ch <= last; ++ch) {
    const int chunk0 = ch * kChunk;
    const int lo = max(chunk0, start_pos), hi = min(chunk0 + kChunk, start_pos + n_tokens);
    const int wt0 = chunk0 + 16 * wave;
    if (wt0 + 16 <= lo || wt0 >= hi) continue;  // no token of this wave in this chunk
    const int t = wt0 + j;
    const bool valid = t >= lo && t < hi;

    float v[32];
    float ss = 0.f;
    if constexpr (DTYPE == TQ_F32) {
      if (valid) {
        const size_t row = ((size_t)b * n_tokens + (t - start_pos)) * c.n_kv_heads + h;
        load32_f32_signed(reinterpret_cast<const float *>(x) + row * kD + 32 * q, smask, v);
      } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) v[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) ss = fmaf(v[e], v[e], ss);
      quad_fwht(v, q);
    } else {
      // Buffer loads over the rows of tokens lo .. hi-1: a lane of a token outside that range
      // reads past the end and gets zeros, so no branch and no clearing.  The range is at
      // most 64 rows of n_kv_heads * 256 bytes (n_kv_heads < 65536, the grid's y limit).
      // (Prefetching the next chunk's words into registers cost a wave per SIMD and was
      // slower.)
      const uint32_t row_bytes = (uint32_t)c.n_kv_heads * (kD * 2);
      const uint32_t range = (uint32_t)(hi - lo) * row_bytes;
      const size_t row_lo = ((size_t)b * n_tokens + (lo - start_pos)) * c.n_kv_heads + h;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t *>(reinterpret_cast<const uint16_t *>(x) + row_lo * kD), (short)0, (int)range, 0x00020000);
      const uint32_t off = valid ? (uint32_t)(t - lo) * row_bytes + 64u * q : range;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u * r, 0, 0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e = 4 * r + k;
          v[2 * e] = dot2_0<DTYPE>(w[k], spair[e]);
          v[2 * e + 1] = dot2_0<DTYPE>(w[k], sdiff[e]);
          ss = dot2<DTYPE>(w[k], w[k], ss);
        }
      }
      quad_fwht<2>(v, q);
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    const float n = sqrtf(ss);
    const float inv = (n > 0.f ? 1.0f / (n * 11.313708498984761f) : 0.f) * quad_fwht_sign(q);
    uint32_t code[32];
    if (BITS <= 4 && gd.ok) {
      const float sinv = inv * gd.scale;
#pragma unroll
      for (int e = 0; e < 32; ++e) code[e] = code_by_grid(v[e], sinv, gd, sh.grid[wave]);
    } else if (BITS == 8 && gd8.ok) {
      const float sinv = inv * gd8.scale;
#pragma unroll
      for (int e = 0; e < 32; ++e) code[e] = code_by_grid8(v[e], sinv, gd8, sh.grid8);
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) code[e] = code_by_search<BITS>(v[e] * inv, sh, wave, pos);
    }
    if (valid && q == 0) c.norm_plane(b, h)[t] = float_to_half_bits(n);

    if (LAYOUT == TQ_LAYOUT_ROWS) {
      if (valid) store_row_quarter<BITS>(plane, t, q, code);
    } else {
      // stage codes [token][coord] as bytes for the value-group packing
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
      store_groups_from_stage<BITS>(sh.stage[wave], plane, lane, wt0, lo, hi);
      __builtin_amdgcn_wave_barrier();  // the stage is rewritten by the next chunk
      __asm__ volatile("" ::: "memory");
    }
  }
}

}  // namespace
}  // namespace tq
