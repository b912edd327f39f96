// Cross-lane reductions without an LDS round trip (gfx950).
#pragma once

#include <hip/hip_runtime.h>

namespace tq {

// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 with the gfx950 row
// swaps (v_permlane16_swap / v_permlane32_swap: plain VALU moves, no LDS round
// trip).  With both operands equal, a swap leaves lane l's partner value in one
// of the two results and its own in the other.
__device__ __forceinline__ float max_over_row_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_row_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over each aligned group of 8 lanes, left in every lane of the group:
// DPP reads of lane ^ 1 and lane ^ 2 (quad permutes), then of lane 7 - l
// within the half row (row_half_mirror), which after the first two steps
// holds the other quad's sum.
__device__ __forceinline__ float sum_over_8_lanes(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  return v;
}

}  // namespace tq
