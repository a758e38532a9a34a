// Lane exchanges, reductions and the 128-point Walsh-Hadamard butterflies across one wave
// of 64 lanes (two coordinates per lane), for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// Lane exchanges and reductions inside a wave of 64 that stay in the vector ALU, with no LDS
// round trip: DPP quad permutes and row shifts / rotations within rows of 16 lanes, and the
// gfx950 lane swaps between rows 16 apart (permlane16) and halves 32 apart (permlane32).
// A swap of x with itself gives {x of the lane's own row (half), x of the partner's} in an
// order that depends on the lane, so a lane picks the partner's copy by its row (half) bit.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int kDppRowShl4 = 0x104;  // lane i takes lane i + 4 of its row
constexpr int kDppRowShr4 = 0x114;  // lane i takes lane i - 4 of its row
constexpr int kDppRowRor4 = 0x124;  // rotate the row by 4
constexpr int kDppRowRor8 = 0x128;  // rotate the row by 8 (= lane xor 8)

// the value of lane (lane xor M)
template <int M>
__device__ __forceinline__ float lane_xor(float v, int lane) {
  if constexpr (M == 1) {
    return dpp_mov<kDppQuadXor1>(v);
  } else if constexpr (M == 2) {
    return dpp_mov<kDppQuadXor2>(v);
  } else if constexpr (M == 4) {
    const float up = dpp_mov<kDppRowShr4>(v), down = dpp_mov<kDppRowShl4>(v);
    return (lane & 4) ? up : down;
  } else if constexpr (M == 8) {
    return dpp_mov<kDppRowRor8>(v);
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    static_assert(M == 32, "lane_xor: M is a power of two below 64");
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
}

// all-reduce over each row of 16 lanes: quads first, then the row's quads by rotation
template <bool MAX>
__device__ __forceinline__ float row16_reduce(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  v = op(v, dpp_mov<kDppQuadXor1>(v));
  v = op(v, dpp_mov<kDppQuadXor2>(v));
  v = op(v, dpp_mov<kDppRowRor4>(v));
  return op(v, dpp_mov<kDppRowRor8>(v));
}
// all-reduce over each half wave (32 lanes): the two copies of a self-swap are the row pair
template <bool MAX>
__device__ __forceinline__ float half_reduce(float v) {
  v = row16_reduce<MAX>(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return MAX ? fmaxf(a, b) : a + b;
}
template <bool MAX>
__device__ __forceinline__ float wave_reduce(float v) {
  v = half_reduce<MAX>(v);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return MAX ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float half_max(float v) { return half_reduce<true>(v); }
__device__ __forceinline__ float half_sum(float v) { return half_reduce<false>(v); }

template <int M>
__device__ __forceinline__ void fwht_stage(float &x0, float &x1, int lane) {
  const bool upper = (lane & M) != 0;
  const float o0 = lane_xor<M>(x0, lane), o1 = lane_xor<M>(x1, lane);
  x0 = upper ? o0 - x0 : x0 + o0;
  x1 = upper ? o1 - x1 : x1 + o1;
}
// Butterfly stages 1..6 of a 128-point Walsh-Hadamard transform whose coordinates 2l, 2l+1
// sit in lane l (stage 0, inside the lane, is done by the caller).
__device__ __forceinline__ void wave_fwht_upper(float &x0, float &x1, int lane) {
  fwht_stage<1>(x0, x1, lane);
  fwht_stage<2>(x0, x1, lane);
  fwht_stage<4>(x0, x1, lane);
  fwht_stage<8>(x0, x1, lane);
  fwht_stage<16>(x0, x1, lane);
  fwht_stage<32>(x0, x1, lane);
}

}  // namespace tq
