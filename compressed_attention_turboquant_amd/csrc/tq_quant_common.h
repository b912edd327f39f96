// Device helpers shared by the quantize kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

// Magnitude index m = #{i : t_i < a} over the K = 2^(BITS-1) - 1 positive
// boundaries t (sorted), by a branchless binary search (value selects only).
template <int BITS>
__device__ __forceinline__ uint32_t magnitude(float a, const float (&t)[BITS > 1 ? (1 << (BITS - 1)) - 1 : 1]) {
  if constexpr (BITS == 1) {
    return 0u;
  } else if constexpr (BITS == 2) {
    return a > t[0] ? 1u : 0u;
  } else if constexpr (BITS == 3) {
    const float t0 = t[0], t1 = t[1], t2 = t[2];
    const bool c1 = a > t1;
    const float h = c1 ? t2 : t0;
    const bool c0 = a > h;
    return (c1 ? 2u : 0u) + (c0 ? 1u : 0u);
  } else {
    const float t0 = t[0], t1 = t[1], t2 = t[2], t3 = t[3], t4 = t[4], t5 = t[5], t6 = t[6];
    const bool c2 = a > t3;
    const float h1 = c2 ? t5 : t1;
    const float h04 = c2 ? t4 : t0;
    const float h26 = c2 ? t6 : t2;
    const bool c1 = a > h1;
    const float h0 = c1 ? h26 : h04;
    const bool c0 = a > h0;
    return (c2 ? 4u : 0u) + (c1 ? 2u : 0u) + (c0 ? 1u : 0u);
  }
}

// Code #{i : beta_i < y} of a value y for the symmetric boundaries whose
// positive half (scaled like y) is t: the magnitude index m, mirrored for y <= 0
// (y = 0 takes the lower middle code).
template <int BITS>
__device__ __forceinline__ uint32_t symmetric_code(float y, const float (&t)[BITS > 1 ? (1 << (BITS - 1)) - 1 : 1]) {
  constexpr uint32_t K = (1u << (BITS - 1)) - 1u;
  return magnitude<BITS>(fabsf(y), t) ^ (y > 0.f ? K + 1u : K);
}

// Workgroup barrier that orders LDS only: global loads and stores stay in
// flight across it (a plain __syncthreads also waits for every outstanding
// global access, which drains prefetched loads and pending stores).  For
// barriers whose only purpose is to hand LDS data between waves.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace tq
